// tile_ring16.hip -- instances of the 256x256x64 unit-ring tile kernel on
// 16x16x32 MFMAs.
#include "configs.h"
#include "kernel_ring.h"

namespace gb {

static_assert(RingConfig::BM == ShapeRing::BM && RingConfig::BN == ShapeRing::BN &&
              RingConfig::BK == ShapeRing::BK);

hipError_t launch_tile_ring(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_ring(args, cus, stream);
}

}  // namespace gb
