// tile_gemv.hip -- instances of the matrix-vector kernel (1, 2 and 4 rows).
#include "configs.h"
#include "kernel_gemv.h"

namespace gb {

hipError_t launch_gemv(const GemmArgs &args, hipStream_t stream) {
    if (args.M <= 1) return launch_gemv_rows<1>(args, stream);
    if (args.M <= 2) return launch_gemv_rows<2>(args, stream);
    return launch_gemv_rows<4>(args, stream);
}

}  // namespace gb
