// tile_skinny_t.hip -- instances of the streaming kernel on transposed
// products (at most 64 columns of C: A is the streamed operand), writing C
// transposed; the configurations of tile_skinny.hip.
#include "configs.h"
#include "kernel_skinny.h"

namespace gb {

hipError_t launch_skinny_t(int rows, int cols, const GemmArgs &args, const SkinnyWork &work, int cus,
                           hipStream_t stream) {
    if (rows == 64) {
        if (cols == 32) return launch_skinny<SkinnyM64N32, false, false, true>(args, work, cus, stream);
        if (cols == 64) return launch_skinny<SkinnyM64N64, false, false, true>(args, work, cus, stream);
        return launch_skinny<SkinnyM64N128, false, false, true>(args, work, cus, stream);
    }
    if (cols == 32) return launch_skinny<SkinnyM32N32, false, false, true>(args, work, cus, stream);
    if (cols == 64) return launch_skinny<SkinnyM32N64, false, false, true>(args, work, cus, stream);
    return launch_skinny<SkinnyM32N128, false, false, true>(args, work, cus, stream);
}

}  // namespace gb
