// tile_fp8_ring16.hip -- instances of the FP8 tile kernel on 16x16x128
// MFMAs (kernel_fp8_ring16.h): exact multiples (the default for FP8 tiles
// on grids that need no split), and the masked instance for shapes with
// tails (chosen only when forced: on tails the 32x32x64 kernel is faster).
#include "configs.h"
#include "kernel_fp8_ring16.h"

namespace gb {

hipError_t launch_tile_fp8(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_fp8_ring16<false>(args, cus, stream);
}

hipError_t launch_tile_fp8_mfma16_masked(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_fp8_ring16<true>(args, cus, stream);
}

}  // namespace gb
