// tile_ring_masked.hip -- instances of the 256x256x64 unit-ring tile kernel
// with masked loads and stores, for shapes with tails (any M and N; K and
// the leading dimensions multiples of 8).
#include "configs.h"
#include "kernel_ring.h"

namespace gb {

hipError_t launch_tile_ring_masked(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_ring_t<true>(args, ring_schedule(args, cus), stream);
}

}  // namespace gb
