// tile_fp8_medium.hip -- instances of the 128x128 tile kernel on FP8 E4M3
// operands (K-slices of 128, 32x32x64 MFMAs, 4 stages): whole K and split-K
// with its reduction, for exact tile multiples and for shapes with tails.
#include "configs.h"
#include "kernel_tile.h"

namespace gb {

using CfgFp8Medium = TileConfig<128, 128, 128, 2, 2, 4, 1>;
static_assert(CfgFp8Medium::BM == ShapeFp8M::BM && CfgFp8Medium::BN == ShapeFp8M::BN &&
              CfgFp8Medium::BK == ShapeFp8M::BK && CfgFp8Medium::kRowBytes == 128);

hipError_t launch_tile_fp8_medium(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_tile<CfgFp8Medium>(args, cus, stream);
}

hipError_t launch_tile_fp8_medium_masked(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_tile<CfgFp8Medium, true>(args, cus, stream);
}

hipError_t launch_tile_fp8_medium_splitk(const GemmArgs &args, const TileSplit &split, int cus, hipStream_t stream) {
    return launch_tile_splitk<CfgFp8Medium>(args, split, cus, stream);
}

hipError_t launch_tile_fp8_medium_splitk_masked(const GemmArgs &args, const TileSplit &split, int cus,
                                                hipStream_t stream) {
    return launch_tile_splitk<CfgFp8Medium, false, true>(args, split, cus, stream);
}

}  // namespace gb
