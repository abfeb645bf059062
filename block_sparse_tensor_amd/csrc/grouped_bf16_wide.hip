// Grouped-contraction kernel variants for bf16 operands (fp32 accumulation and
// output) holding the wide direct-to-LDS tile (one workgroup per CU), and the
// eight-wave launch of wide tiles only.
#include "grouped_kernel.h"

namespace bsc {

// A launch of wide tiles and tail bundles only, on eight waves per
// workgroup.  The planner puts no other task class into such a launch; a
// task's class is the same for every wave of the workgroup, so a class this
// body does not hold is skipped by all waves together.  A tail bundle (no
// barrier inside) runs on waves 0-3, one group per wave; the others go on to
// the next task and meet the bundle's waves at its first barrier.
union Wide8Smem {
    WideSmemBf16 x;
    TailSmem<float> t;
};

__device__ __forceinline__ void wide8_body(const KArgs &ka) {
    Wide8Smem &sm = *reinterpret_cast<Wide8Smem *>(bsc_dyn_smem);
    for (int32_t t = blockIdx.x; t < ka.ntasks; t += gridDim.x) {
        const int32_t ti = ka.task0 + t;
        const DTask task = ka.tasks[ti];
        if (task.cls == T_MFMA_WIDE_N) wide8_tile_bf16<float, true>(ka, ka.fast[ti], sm.x);
        else if (task.cls == T_MFMA_WIDE_K) wide8_tile_bf16<float, false>(ka, ka.fast[ti], sm.x);
        else if (task.cls == T_TAIL) tail_bundle<uint16_t, float, float>(ka, task, sm.t);
    }
}

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void grouped_contract_wide8(KArgs ka) {
    wide8_body(ka);
}

KernelRef grouped_kernel_bf16_wide(int32_t feat) {
    return (feat & FEAT_MFMA) ? kernel_ref<uint16_t, float, float, FEAT_WIDE | FEAT_MFMA>()
                              : kernel_ref<uint16_t, float, float, FEAT_WIDE>();
}

KernelRef grouped_kernel_bf16_wide8() {
    const size_t lds = sizeof(Wide8Smem);
    static const hipError_t once = hipFuncSetAttribute(reinterpret_cast<const void *>(grouped_contract_wide8),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    (void)once;
    return {grouped_contract_wide8, lds, 512};
}

}  // namespace bsc
