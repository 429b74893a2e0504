// tile_ring.hip -- instances of the 256x256x64 unit-ring tile kernel for
// shapes without tails (M, N multiples of 256, K a multiple of 64).
#include "configs.h"
#include "kernel_ring.h"

namespace gb {

static_assert(RingConfig::BM == ShapeRing::BM && RingConfig::BN == ShapeRing::BN &&
              RingConfig::BK == ShapeRing::BK);

hipError_t launch_tile_ring(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_ring_t<false>(args, ring_schedule(args, cus), stream);
}

}  // namespace gb
