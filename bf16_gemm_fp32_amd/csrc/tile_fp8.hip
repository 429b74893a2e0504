// tile_fp8.hip -- instances of the 256x256 FP8 (E4M3) tile kernel on
// 32x32x64 MFMAs: whole-K (chosen only when forced) and split-K (with its
// reduction).
#include "configs.h"
#include "kernel_fp8.h"

namespace gb {

static_assert(Fp8Config::BM == ShapeFp8::BM && Fp8Config::BN == ShapeFp8::BN && Fp8Config::BK == ShapeFp8::BK);

hipError_t launch_tile_fp8_mfma32(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_fp8_ring<false>(args, cus, stream);
}

hipError_t launch_tile_fp8_splitk(const GemmArgs &args, const TileSplit &split, int cus, hipStream_t stream) {
    return launch_fp8_splitk<false>(args, split, cus, stream);
}

}  // namespace gb
