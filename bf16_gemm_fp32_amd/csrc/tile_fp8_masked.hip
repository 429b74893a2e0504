// tile_fp8_masked.hip -- instances of the 256x256 FP8 (E4M3) tile kernel on
// 32x32x64 MFMAs for shapes with tails (zero-filled out-of-range loads,
// masked epilogue): whole-K (the default for FP8 tails) and split-K.
#include "configs.h"
#include "kernel_fp8.h"

namespace gb {

hipError_t launch_tile_fp8_mfma32_masked(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_fp8_ring<true>(args, cus, stream);
}

hipError_t launch_tile_fp8_splitk_masked(const GemmArgs &args, const TileSplit &split, int cus,
                                         hipStream_t stream) {
    return launch_fp8_splitk<true>(args, split, cus, stream);
}

}  // namespace gb
