// tile_medium.hip -- instances of the 128x128x64, 4-stage tile kernel (whole
// K, and split-K with its reduction).
#include "configs.h"
#include "kernel_tile.h"

namespace gb {

using CfgMedium = TileConfig<128, 128, 64, 2, 2, 4>;
static_assert(CfgMedium::BM == ShapeM::BM && CfgMedium::BN == ShapeM::BN && CfgMedium::BK == ShapeM::BK);

hipError_t launch_tile_medium(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_tile<CfgMedium>(args, cus, stream);
}

hipError_t launch_tile_medium_splitk(const GemmArgs &args, const TileSplit &split, int cus, hipStream_t stream) {
    return launch_tile_splitk<CfgMedium>(args, split, cus, stream);
}

hipError_t launch_tile_medium_splitk_q8(const GemmArgs &args, const TileSplit &split, int cus,
                                        hipStream_t stream) {
    return launch_tile_splitk<CfgMedium, true>(args, split, cus, stream);
}

}  // namespace gb
