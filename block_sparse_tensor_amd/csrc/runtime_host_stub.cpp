// Device entry points for the host-only planner library used in sanitizer runs
// on machines without a GPU.  They fail loudly; the shipped library links
// runtime.hip instead.
#include "bsc_internal.h"

using namespace bsc;

extern "C" bsc_status bsc_plan_bind(bsc_plan_t, void *, size_t, void *) {
    set_error("bsc_plan_bind: host-only planner build has no device runtime");
    return BSC_ERR_UNSUPPORTED;
}

extern "C" bsc_status bsc_contract(bsc_plan_t, const void *, const void *, void *, void *) {
    set_error("bsc_contract: host-only planner build has no device runtime");
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
