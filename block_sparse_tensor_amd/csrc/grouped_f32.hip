// Grouped-contraction kernel variants for f32 operands.
#include "grouped_kernel.h"

namespace bsc {

KernelRef grouped_kernel_f32(int32_t feat) {
    return (feat & FEAT_MFMA) ? kernel_ref<float, float, float, FEAT_MFMA>() : kernel_ref<float, float, float, 0>();
}

}  // namespace bsc
