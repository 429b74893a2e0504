// tile_gemv.hip -- instances of the matrix-vector kernel (1, 2 and 4 rows;
// bf16 or FP8 E4M3 operands).
#include "configs.h"
#include "kernel_gemv.h"

namespace gb {

hipError_t launch_gemv(const GemmArgs &args, hipStream_t stream, bool fp8) {
    if (fp8) {
        if (args.M <= 1) return launch_gemv_rows<1, true>(args, stream);
        if (args.M <= 2) return launch_gemv_rows<2, true>(args, stream);
        return launch_gemv_rows<4, true>(args, stream);
    }
    if (args.M <= 1) return launch_gemv_rows<1, false>(args, stream);
    if (args.M <= 2) return launch_gemv_rows<2, false>(args, stream);
    return launch_gemv_rows<4, false>(args, stream);
}

}  // namespace gb
