// tile_skinny_fp8.hip -- instances of the streaming kernel on FP8 (E4M3)
// operands, direct and on the transposed product: 32-column strips, slices
// of 512 values (512-byte rows).
#include "configs.h"
#include "kernel_skinny.h"

namespace gb {

using SkinnyFp8M64 = SkinnyConfig<2, 1, 256, 3, 4>;
using SkinnyFp8M32 = SkinnyConfig<1, 1, 256, 3, 6>;
static_assert(SkinnyFp8M64::kRowBytes == ShapeSkinny::KS_FP8 && SkinnyFp8M32::kRowBytes == ShapeSkinny::KS_FP8,
              "the host plans splits with this slice length (values = bytes)");

hipError_t launch_skinny_fp8(int rows, const GemmArgs &args, const SkinnyWork &work, int cus, hipStream_t stream) {
    if (rows == 64) return launch_skinny<SkinnyFp8M64, true>(args, work, cus, stream);
    return launch_skinny<SkinnyFp8M32, true>(args, work, cus, stream);
}

hipError_t launch_skinny_fp8_t(int rows, const GemmArgs &args, const SkinnyWork &work, int cus,
                               hipStream_t stream) {
    if (rows == 64) return launch_skinny<SkinnyFp8M64, true, false, true>(args, work, cus, stream);
    return launch_skinny<SkinnyFp8M32, true, false, true>(args, work, cus, stream);
}

}  // namespace gb
