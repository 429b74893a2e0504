// tile_ring_q8.hip -- instances of the masked 256x256x64 unit-ring tile
// kernel whose epilogue writes int8 (per-row scale and a zero point) instead
// of bf16: the quantizing entry point for shapes with tails.
#include "configs.h"
#include "kernel_ring.h"

namespace gb {

hipError_t launch_tile_ring_q8_masked(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_ring_t<true, true>(args, ring_schedule(args, cus), stream);
}

}  // namespace gb
