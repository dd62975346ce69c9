// mk_interp_b4.hip - resident interpreter variants for batches padded to 4.
#include "mk_interp.h"

namespace mk {

const void *interp_kernel_b4(int G) {
    switch (G) {
        case 1: return (const void *)mk_megakernel<4, 1>;
        case 2: return (const void *)mk_megakernel<4, 2>;
        case 4: return (const void *)mk_megakernel<4, 4>;
        case 8: return (const void *)mk_megakernel<4, 8>;
        default: return nullptr;
    }
}

}  // namespace mk
