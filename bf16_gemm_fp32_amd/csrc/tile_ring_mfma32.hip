// tile_ring.hip -- instances of the 256x256x64 unit-ring tile kernel.
#include "configs.h"
#include "kernel_ring_mfma32.h"

namespace gb {

static_assert(Ring32Config::BM == ShapeRing::BM && Ring32Config::BN == ShapeRing::BN && Ring32Config::BK == ShapeRing::BK);

hipError_t launch_tile_ring_mfma32(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_ring32(args, cus, stream);
}

}  // namespace gb
