// Grouped-contraction kernel variants for bf16 operands (fp32 accumulation and
// output) without the direct-to-LDS tiles: generic, skinny and general
// matrix-core tile bodies.
#include "grouped_kernel.h"

namespace bsc {

KernelRef grouped_kernel_bf16_lo(int32_t feat) {
    switch (feat) {
        case 0: return kernel_ref<uint16_t, float, float, 0>();
        case 1: return kernel_ref<uint16_t, float, float, 1>();
        case 2: return kernel_ref<uint16_t, float, float, 2>();
        default: return kernel_ref<uint16_t, float, float, 3>();
    }
}

}  // namespace bsc
