// tile_ring_q8_exact.hip -- instances of the unmasked 256x256x64 unit-ring
// tile kernel with the int8 epilogue, for exact tile multiples (no masking
// code in the loads or the epilogue).
#include "configs.h"
#include "kernel_ring.h"

namespace gb {

hipError_t launch_tile_ring_q8(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_ring_t<false, true>(args, ring_schedule(args, cus), stream);
}

}  // namespace gb
