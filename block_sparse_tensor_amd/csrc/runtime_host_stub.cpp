// Device entry points for the host-only planner library used in sanitizer runs
// on machines without a GPU.  They apply the same argument checks as the HIP
// runtime (so those host paths run under the sanitizers too) and then fail
// loudly with BSC_ERR_UNSUPPORTED; the shipped library links runtime.hip instead.
#include "bsc_internal.h"

using namespace bsc;

extern "C" bsc_status bsc_plan_bind(bsc_plan_t plan, void *dev, size_t bytes, void *) {
    set_error("");
    if (!plan || !dev) {
        set_error("bsc_plan_bind: NULL argument");
        return BSC_ERR_ARG;
    }
    if (bytes < reinterpret_cast<Plan *>(plan)->dev_bytes) {
        set_error("bsc_plan_bind: device region smaller than bsc_plan_device_bytes");
        return BSC_ERR_DEVICE_BYTES;
    }
    set_error("bsc_plan_bind: host-only planner build has no device runtime");
    return BSC_ERR_UNSUPPORTED;
}

extern "C" bsc_status bsc_contract(bsc_plan_t plan, const void *, const void *, void *, void *) {
    if (!plan) {
        set_error("bsc_contract: NULL plan");
        return BSC_ERR_ARG;
    }
    if (!reinterpret_cast<Plan *>(plan)->dev) {
        set_error("bsc_contract: plan is not bound to a device region");
        return BSC_ERR_NOT_BOUND;
    }
    set_error("bsc_contract: host-only planner build has no device runtime");
    return BSC_ERR_UNSUPPORTED;
}

extern "C" bsc_status bsc_contract_noalloc(bsc_plan_t plan, const void *, const void *, void *, void *) {
    if (!plan) {
        set_error("bsc_contract_noalloc: NULL plan");
        return BSC_ERR_ARG;
    }
    set_error("bsc_contract_noalloc: host-only planner build has no device runtime");
    return BSC_ERR_UNSUPPORTED;
}

extern "C" bsc_status bsc_chain_create(const bsc_plan_t *, const void *const *, const void *const *, void *const *,
                                       int32_t, bsc_chain_t *out) {
    if (out) *out = nullptr;
    set_error("bsc_chain_create: host-only planner build has no device runtime");
    return BSC_ERR_UNSUPPORTED;
}

extern "C" bsc_status bsc_chain_launch(bsc_chain_t, void *) {
    set_error("bsc_chain_launch: host-only planner build has no device runtime");
    return BSC_ERR_UNSUPPORTED;
}

extern "C" void bsc_chain_destroy(bsc_chain_t) {}

extern "C" bsc_status bsc_fused_bind(bsc_fused_t plan, void *dev, size_t, void *) {
    if (!plan || !dev) {
        set_error("bsc_fused_bind: NULL argument");
        return BSC_ERR_ARG;
    }
    set_error("bsc_fused_bind: host-only planner build has no device runtime");
    return BSC_ERR_UNSUPPORTED;
}

extern "C" bsc_status bsc_fused_contract(bsc_fused_t plan, const void *, const void *, const void *, void *, void *) {
    if (!plan) {
        set_error("bsc_fused_contract: NULL plan");
        return BSC_ERR_ARG;
    }
    set_error("bsc_fused_contract: host-only planner build has no device runtime");
    return BSC_ERR_UNSUPPORTED;
}

extern "C" bsc_status bsc_probe_mfma(bsc_dtype, int32_t iters, float *sink, void *, double *flops) {
    if (!sink || !flops || iters < 1) {
        set_error("bsc_probe_mfma: NULL sink or flops, or iters < 1");
        return BSC_ERR_ARG;
    }
    set_error("bsc_probe_mfma: host-only planner build has no device runtime");
    return BSC_ERR_UNSUPPORTED;
}
