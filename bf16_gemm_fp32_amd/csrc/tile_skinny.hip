// tile_skinny.hip -- instances of the streaming kernel for at most 64 rows:
// 32-column strips with K-slices of 256 in A/B rings of 3/4 slices, 64-column
// strips (split K within an XCD) with K-slices of 256 in rings of 2/3 (2/4
// for 32 rows), and 128-column strips with K-slices of 128.
#include "configs.h"
#include "kernel_skinny.h"

namespace gb {

static_assert(SkinnyM64N32::KS == ShapeSkinny::KS_N32 && SkinnyM64N64::KS == ShapeSkinny::KS_N64 &&
                  SkinnyM64N128::KS == ShapeSkinny::KS_N128 && SkinnyM32N32::KS == ShapeSkinny::KS_N32 &&
                  SkinnyM32N64::KS == ShapeSkinny::KS_N64 && SkinnyM32N128::KS == ShapeSkinny::KS_N128,
              "the host plans splits with these slice lengths");

hipError_t launch_skinny(int rows, int cols, const GemmArgs &args, const SkinnyWork &work, int cus,
                         hipStream_t stream) {
    if (rows == 64) {
        if (cols == 32) return launch_skinny<SkinnyM64N32>(args, work, cus, stream);
        if (cols == 64) return launch_skinny<SkinnyM64N64>(args, work, cus, stream);
        return launch_skinny<SkinnyM64N128>(args, work, cus, stream);
    }
    if (cols == 32) return launch_skinny<SkinnyM32N32>(args, work, cus, stream);
    if (cols == 64) return launch_skinny<SkinnyM32N64>(args, work, cus, stream);
    return launch_skinny<SkinnyM32N128>(args, work, cus, stream);
}

}  // namespace gb
