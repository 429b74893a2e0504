// tile_skinny_q8.hip -- instances of the streaming kernel for at most 64
// rows (or, on the transposed product, 64 columns) with the int8 output
// (per-row scale and zero point): 32-column strips with K-slices of 256.
#include "configs.h"
#include "kernel_skinny.h"

namespace gb {

static_assert(SkinnyM64N32::KS == ShapeSkinny::KS_N32 && SkinnyM32N32::KS == ShapeSkinny::KS_N32,
              "the host plans splits with these slice lengths");

hipError_t launch_skinny_q8(int rows, const GemmArgs &args, const SkinnyWork &work, int cus, hipStream_t stream) {
    if (rows == 64) return launch_skinny<SkinnyM64N32, false, true>(args, work, cus, stream);
    return launch_skinny<SkinnyM32N32, false, true>(args, work, cus, stream);
}

hipError_t launch_skinny_q8_t(int rows, const GemmArgs &args, const SkinnyWork &work, int cus, hipStream_t stream) {
    if (rows == 64) return launch_skinny<SkinnyM64N32, false, true, true>(args, work, cus, stream);
    return launch_skinny<SkinnyM32N32, false, true, true>(args, work, cus, stream);
}

}  // namespace gb
