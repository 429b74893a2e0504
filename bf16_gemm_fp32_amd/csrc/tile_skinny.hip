// tile_skinny.hip -- instances of the streaming kernel for M = 64 and M = 32
// (32-column strips, K-slices of 256, A/B rings of 3/4 slices; wider strips
// and shorter slices measured slower on the 64 x 8192 x 8192 product).
#include "configs.h"
#include "kernel_skinny.h"

namespace gb {

hipError_t launch_skinny_m64(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_skinny<SkinnyConfig<2>>(args, cus, stream);
}

hipError_t launch_skinny_m32(const GemmArgs &args, int cus, hipStream_t stream) {
    return launch_skinny<SkinnyConfig<1>>(args, cus, stream);
}

}  // namespace gb
