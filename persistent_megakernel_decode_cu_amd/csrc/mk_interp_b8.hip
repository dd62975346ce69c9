// mk_interp_b8.hip - resident interpreter variants for batches padded to 8.
#include "mk_interp.h"

namespace mk {

const void *interp_kernel_b8(int G) {
    switch (G) {
        case 1: return (const void *)mk_megakernel<8, 1>;
        case 2: return (const void *)mk_megakernel<8, 2>;
        case 4: return (const void *)mk_megakernel<8, 4>;
        case 8: return (const void *)mk_megakernel<8, 8>;
        default: return nullptr;
    }
}

}  // namespace mk
