// tile_fp8_ring16.hip -- instances of the FP8 tile kernel on 16x16x128
// MFMAs (kernel_fp8_ring16.h), the default for FP8 inputs on grids that
// need no split: exact multiples and the masked instance for shapes with
// tails.
#include "configs.h"
#include "kernel_fp8_ring16.h"

namespace gb {

hipError_t launch_tile_fp8(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_fp8_ring16<false>(args, cus, stream);
}

hipError_t launch_tile_fp8_masked(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_fp8_ring16<true>(args, cus, stream);
}

}  // namespace gb
