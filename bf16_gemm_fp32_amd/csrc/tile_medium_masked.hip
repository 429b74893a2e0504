// tile_medium_masked.hip -- instances of the masked 128x128x64, 4-stage
// tile kernel for shapes with tails on small and mid-sized grids (whole K,
// and split-K with its reduction over a workspace padded to tile multiples,
// bf16 or int8 output).
#include "configs.h"
#include "kernel_tile.h"

namespace gb {

using CfgMediumMasked = TileConfig<128, 128, 64, 2, 2, 4>;
static_assert(CfgMediumMasked::BM == ShapeM::BM && CfgMediumMasked::BN == ShapeM::BN &&
              CfgMediumMasked::BK == ShapeM::BK);

hipError_t launch_tile_medium_masked(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_tile<CfgMediumMasked, true>(args, cus, stream);
}

hipError_t launch_tile_medium_splitk_masked(const GemmArgs &args, const TileSplit &split, int cus,
                                            hipStream_t stream) {
    return launch_tile_splitk<CfgMediumMasked, false, true>(args, split, cus, stream);
}

hipError_t launch_tile_medium_splitk_q8_masked(const GemmArgs &args, const TileSplit &split, int cus,
                                               hipStream_t stream) {
    return launch_tile_splitk<CfgMediumMasked, true, true>(args, split, cus, stream);
}

}  // namespace gb
