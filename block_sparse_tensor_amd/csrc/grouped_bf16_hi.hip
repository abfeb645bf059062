// Grouped-contraction kernel variants for bf16 operands (fp32 accumulation and
// output) holding the direct-to-LDS tile with K-contiguous B.
#include "grouped_kernel.h"

namespace bsc {

KernelRef grouped_kernel_bf16_hi(int32_t feat) {
    switch (feat) {
        case 4: return kernel_ref<uint16_t, float, float, 4>();
        case 5: return kernel_ref<uint16_t, float, float, 5>();
        case 6: return kernel_ref<uint16_t, float, float, 6>();
        default: return kernel_ref<uint16_t, float, float, 7>();
    }
}

}  // namespace bsc
