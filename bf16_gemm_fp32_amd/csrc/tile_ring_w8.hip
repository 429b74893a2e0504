// tile_ring_w8.hip -- the 256x256x64 unit-ring kernel on eight waves of
// 128x64 (two per SIMD), for shapes without tails.
#include "configs.h"
#include "kernel_ring.h"

namespace gb {

static_assert(RingConfigW8::BM == ShapeRing::BM && RingConfigW8::BN == ShapeRing::BN &&
              RingConfigW8::BK == ShapeRing::BK);

hipError_t launch_tile_ring_w8(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_ring_t<false, false, RingConfigW8>(args, ring_schedule(args, cus), stream);
}

}  // namespace gb
