// Grouped-contraction kernel variants for bf16 operands (fp32 accumulation and
// output) holding the wide direct-to-LDS tile (one workgroup per CU).
#include "grouped_kernel.h"

namespace bsc {

KernelRef grouped_kernel_bf16_wide(int32_t feat) {
    return (feat & FEAT_MFMA) ? kernel_ref<uint16_t, float, float, FEAT_WIDE | FEAT_MFMA>()
                              : kernel_ref<uint16_t, float, float, FEAT_WIDE>();
}

}  // namespace bsc
