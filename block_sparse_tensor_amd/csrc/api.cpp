// C-ABI entry points that need no device: options, planning, statistics,
// export, destruction and error reporting.  bsc_plan_bind and bsc_contract
// live in runtime.hip.
#include <cstring>
#include <new>
#include <string>

#include "bsc_internal.h"

namespace bsc {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }

}  // namespace bsc

using namespace bsc;

extern "C" {

void bsc_options_default(bsc_options *opt) {
    if (!opt) return;
    std::memset(opt, 0, sizeof(*opt));
    opt->launch_mode = BSC_LAUNCH_GROUPED;
    opt->layout_policy = BSC_LAYOUT_AUTO;
    opt->accumulate = 0;
    opt->grid_limit = 0;
}

static void fill_cost_defaults(bsc_options &o, bsc_dtype dt) {
    // MI355X defaults, measured on one MI355X with this library by the pack
    // calibration of the benchmark driver (calibrated constants may be passed
    // in instead).  Over six gathers of the environment-update chains' stages
    // and the unpadded block-diagonal bf16 workload (4.3 to 33.8 MB), the
    // gather kernel's time fits 6.4 us + 2 x bytes / 4.9 TB/s (a 19.7 KB
    // gather took 5.4 us):
    //   t_launch_us  a plan's extra (gather) launch: the gather's fixed 6.4 us
    //                plus the 0.6 us gap the second launch leaves;
    //   pack_gbps    the gather's bandwidth, read + write bytes;
    //   tile_gflops  sustained whole-GPU rate of the matrix-core tiles on
    //                mid-sized sector GEMMs (bf16 ~ 250 TFLOP/s, fp32 and fp64
    //                ~ 10 TFLOP/s);
    //   t_seg_us     per extra piece walked by one tile: gathering every
    //                operand of the U(1)xU(1) W stage saves 16.8 us of grouped
    //                kernel time (beyond its padding term) for 35,364 units of
    //                the piece term, 0.00047 us each.
    if (o.t_launch_us <= 0) o.t_launch_us = 7.0;
    if (o.t_seg_us <= 0) o.t_seg_us = 0.00047;
    if (o.pack_gbps <= 0) o.pack_gbps = 4900.0;
    if (o.tile_gflops <= 0) o.tile_gflops = dt == BSC_BF16_F32 ? 250000.0 : 10000.0;
}

bsc_status bsc_plan(const bsc_index *m, const bsc_index *k, const bsc_index *n, const bsc_operand *A,
                    const bsc_operand *B, const bsc_operand *C, bsc_dtype dtype, bsc_axis axis,
                    const bsc_options *opt, bsc_plan_t *out) {
    set_error("");
    if (!out) {
        set_error("bsc_plan: out is NULL");
        return BSC_ERR_ARG;
    }
    *out = nullptr;
    if (dtype != BSC_F64 && dtype != BSC_F32 && dtype != BSC_BF16_F32) {
        set_error("bsc_plan: unknown dtype");
        return BSC_ERR_ARG;
    }
    if (axis < BSC_AXIS_NONE || axis > BSC_AXIS_AUTO) {
        set_error("bsc_plan: unknown axis");
        return BSC_ERR_ARG;
    }
    Plan *p = new (std::nothrow) Plan();
    if (!p) {
        set_error("bsc_plan: out of host memory");
        return BSC_ERR_UNSUPPORTED;
    }
    if (opt) p->opt = *opt;
    else bsc_options_default(&p->opt);
    if (p->opt.launch_mode != BSC_LAUNCH_GROUPED && p->opt.launch_mode != BSC_LAUNCH_PER_SECTOR) {
        delete p;
        set_error("bsc_plan: unknown launch mode");
        return BSC_ERR_ARG;
    }
    if (p->opt.layout_policy < BSC_LAYOUT_AUTO || p->opt.layout_policy > BSC_LAYOUT_FORCE_PACK || p->opt.grid_limit < 0 ||
        p->opt.split_k < -1 || (p->opt.tile_rows != 0 && p->opt.tile_rows != 128 && p->opt.tile_rows != 256) ||
        (p->opt.tile_cols != 0 && p->opt.tile_cols != 128 && p->opt.tile_cols != 256)) {
        delete p;
        set_error("bsc_plan: bad layout policy, grid limit, split_k, tile_rows or tile_cols");
        return BSC_ERR_ARG;
    }
    fill_cost_defaults(p->opt, dtype);
    p->dtype = dtype;
    p->axis = axis;
    bsc_status st = build_plan(*p, m, k, n, A, B, C);
    if (st != BSC_OK) {
        delete p;
        return st;
    }
    *out = reinterpret_cast<bsc_plan_t>(p);
    return BSC_OK;
}

bsc_status bsc_plan_device_bytes(bsc_plan_t plan, size_t *bytes) {
    if (!plan || !bytes) {
        set_error("bsc_plan_device_bytes: NULL argument");
        return BSC_ERR_ARG;
    }
    *bytes = reinterpret_cast<Plan *>(plan)->dev_bytes;
    return BSC_OK;
}

bsc_status bsc_plan_stats(bsc_plan_t plan, bsc_stats *out) {
    if (!plan || !out) {
        set_error("bsc_plan_stats: NULL argument");
        return BSC_ERR_ARG;
    }
    Plan *p = reinterpret_cast<Plan *>(plan);
    *out = p->stats;
    out->grid = p->grid;
    return BSC_OK;
}

bsc_status bsc_plan_export(bsc_plan_t plan, int32_t *triples, int32_t *group_of_triple, int32_t *group_mode) {
    if (!plan) {
        set_error("bsc_plan_export: NULL plan");
        return BSC_ERR_ARG;
    }
    Plan *p = reinterpret_cast<Plan *>(plan);
    if (triples)
        for (size_t i = 0; i < p->triples.size(); ++i)
            for (int j = 0; j < 3; ++j) triples[3 * i + j] = p->triples[i][(size_t)j];
    if (group_of_triple)
        for (size_t i = 0; i < p->group_of_triple.size(); ++i) group_of_triple[i] = p->group_of_triple[i];
    if (group_mode)
        for (size_t g = 0; g < p->group_mode.size(); ++g)
            for (int j = 0; j < 3; ++j) group_mode[3 * g + j] = p->group_mode[g][(size_t)j];
    return BSC_OK;
}

bsc_status bsc_plan_worklist(bsc_plan_t plan, bsc_worklist_info *info, void *image, size_t bytes) {
    if (!plan || !info) {
        set_error("bsc_plan_worklist: NULL argument");
        return BSC_ERR_ARG;
    }
    Plan *p = reinterpret_cast<Plan *>(plan);
    info->n_groups = (int64_t)p->groups.size();
    info->n_runs = (int64_t)p->runs.size();
    info->n_apieces = (int64_t)p->apieces.size();
    info->n_bpieces = (int64_t)p->bpieces.size();
    info->n_cpieces = (int64_t)p->cpieces.size();
    info->n_tasks = (int64_t)p->tasks.size();
    info->n_dense = (int64_t)p->fast.size();
    info->off_groups = (int64_t)p->off_groups;
    info->off_runs = (int64_t)p->off_runs;
    info->off_apieces = (int64_t)p->off_ap;
    info->off_bpieces = (int64_t)p->off_bp;
    info->off_cpieces = (int64_t)p->off_cp;
    info->off_tasks = (int64_t)p->off_tasks;
    info->off_dense = (int64_t)p->off_fast;
    info->n_packs = (int64_t)p->packs.size();
    info->n_pack_tasks = (int64_t)p->pack_tasks.size();
    info->off_packs = (int64_t)p->off_packs;
    info->off_pack_tasks = (int64_t)p->off_ptasks;
    info->off_workspace = (int64_t)p->off_ws;
    info->workspace_elems = p->ws_elems;
    info->bytes = (int64_t)p->image.size();
    info->n_launches = (int64_t)p->launches.size() + (p->packs.empty() ? 0 : 1);
    info->n_counters = p->n_counters;
    info->off_counters = (int64_t)p->off_cnt;
    info->off_partials = (int64_t)p->off_part;
    info->partial_elems = p->part_elems;
    info->n_tail = (int64_t)p->tail.size();
    info->off_tail = (int64_t)p->off_tail;
    if (image) {
        if (bytes < p->image.size()) {
            set_error("bsc_plan_worklist: image buffer too small");
            return BSC_ERR_ARG;
        }
        std::memcpy(image, p->image.data(), p->image.size());
    }
    return BSC_OK;
}

void bsc_plan_destroy(bsc_plan_t plan) { delete reinterpret_cast<Plan *>(plan); }

const char *bsc_status_string(bsc_status s) {
    switch (s) {
        case BSC_OK: return "BSC_OK";
        case BSC_ERR_ARG: return "BSC_ERR_ARG";
        case BSC_ERR_CHARGE: return "BSC_ERR_CHARGE";
        case BSC_ERR_SHAPE: return "BSC_ERR_SHAPE";
        case BSC_ERR_BOUNDS: return "BSC_ERR_BOUNDS";
        case BSC_ERR_OVERLAP: return "BSC_ERR_OVERLAP";
        case BSC_ERR_MISSING_OUTPUT: return "BSC_ERR_MISSING_OUTPUT";
        case BSC_ERR_UNSUPPORTED: return "BSC_ERR_UNSUPPORTED";
        case BSC_ERR_NOT_BOUND: return "BSC_ERR_NOT_BOUND";
        case BSC_ERR_DEVICE_BYTES: return "BSC_ERR_DEVICE_BYTES";
        case BSC_ERR_HIP: return "BSC_ERR_HIP";
    }
    return "BSC_ERR_UNKNOWN";
}

const char *bsc_last_error(void) { return bsc::g_last_error.c_str(); }

}  // extern "C"
