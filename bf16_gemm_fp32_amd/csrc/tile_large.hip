// tile_large.hip -- instances of the 256x256x32, 5-stage tile kernel.
#include "configs.h"
#include "kernel_tile.h"

namespace gb {

using CfgLarge = TileConfig<256, 256, 32, 2, 2, 5>;
static_assert(CfgLarge::BM == ShapeL::BM && CfgLarge::BN == ShapeL::BN && CfgLarge::BK == ShapeL::BK);

hipError_t launch_tile_large(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_tile<CfgLarge>(args, cus, stream);
}

}  // namespace gb
