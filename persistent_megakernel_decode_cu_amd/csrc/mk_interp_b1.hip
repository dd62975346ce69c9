// mk_interp_b1.hip - resident interpreter variants for batches padded to 1.
#include "mk_interp.h"

namespace mk {

const void *interp_kernel_b1(int G) {
    switch (G) {
        case 1: return (const void *)mk_megakernel<1, 1>;
        case 2: return (const void *)mk_megakernel<1, 2>;
        case 4: return (const void *)mk_megakernel<1, 4>;
        case 8: return (const void *)mk_megakernel<1, 8>;
        default: return nullptr;
    }
}

}  // namespace mk
