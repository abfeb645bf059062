// Grouped-contraction kernel variants for f64 operands.
#include "grouped_kernel.h"

namespace bsc {

KernelRef grouped_kernel_f64(int32_t feat) {
    return (feat & FEAT_MFMA) ? kernel_ref<double, double, double, FEAT_MFMA>() : kernel_ref<double, double, double, 0>();
}

}  // namespace bsc
