// mk_interp_b2.hip - resident interpreter variants for batches padded to 2.
#include "mk_interp.h"

namespace mk {

const void *interp_kernel_b2(int G) {
    switch (G) {
        case 1: return (const void *)mk_megakernel<2, 1>;
        case 2: return (const void *)mk_megakernel<2, 2>;
        case 4: return (const void *)mk_megakernel<2, 4>;
        case 8: return (const void *)mk_megakernel<2, 8>;
        default: return nullptr;
    }
}

}  // namespace mk
