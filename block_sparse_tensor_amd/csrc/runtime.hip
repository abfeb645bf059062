// Device side of the engine: work-list upload, the launches of one contraction
// (gathers, then the grouped kernel: grouped_kernel.h) and captured chains.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <string>
#include <type_traits>

#include "bsc_internal.h"
#include "launch.h"

namespace bsc {

static bsc_status hip_fail(hipError_t e, const char *what) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return BSC_ERR_HIP;
}

// bf16 launches pick the variant that holds exactly the tile bodies the plan uses;
// when an operand base is not 16-byte aligned the direct-to-LDS tiles fall back
// to the general matrix-core tile (task class T_MFMA_FAST_* is accepted there).
// A plan of wide tiles only runs them on eight waves per workgroup.
static KernelRef pick_bf16(int32_t feat, bool vec, bool only_wide) {
    constexpr int32_t DIRECT = FEAT_FAST_N | FEAT_FAST_K | FEAT_WIDE;
    if (!vec && (feat & DIRECT)) feat = (feat & ~DIRECT) | FEAT_MFMA;
    if (feat == FEAT_WIDE && only_wide) return grouped_kernel_bf16_wide8();   // (tail bundles hold no FEAT bit)
    if (feat & FEAT_WIDE) return grouped_kernel_bf16_wide(feat);
    return feat < 4 ? grouped_kernel_bf16_lo(feat) : grouped_kernel_bf16_hi(feat);
}

// Grid of a launch: one workgroup per task up to a persistent cap of 16 per CU
// (four to eight times what is resident at once, so a workgroup that finishes
// is replaced by a fresh one more often than it loops to its next task); the
// cap is a multiple of BSC_XCDS so task t keeps running on XCD t % BSC_XCDS.
static int32_t grid_for(const Plan &p, int32_t ntasks, int32_t cu_count) {
    int32_t cap = p.opt.grid_limit > 0 ? p.opt.grid_limit : std::max(1, cu_count) * 16;
    if (cap >= BSC_XCDS) cap -= cap % BSC_XCDS;
    return std::max(1, std::min(ntasks, cap));
}

}  // namespace bsc

using namespace bsc;

extern "C" bsc_status bsc_plan_bind(bsc_plan_t plan, void *dev, size_t bytes, void *stream) {
    set_error("");
    if (!plan || !dev) {
        set_error("bsc_plan_bind: NULL argument");
        return BSC_ERR_ARG;
    }
    Plan *p = reinterpret_cast<Plan *>(plan);
    if (bytes < p->dev_bytes) {
        set_error("bsc_plan_bind: device region smaller than bsc_plan_device_bytes");
        return BSC_ERR_DEVICE_BYTES;
    }
    if (reinterpret_cast<uintptr_t>(dev) % 256 != 0) {
        set_error("bsc_plan_bind: device region must be 256-byte aligned");
        return BSC_ERR_ARG;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int dev_id = 0;
    hipError_t e = hipGetDevice(&dev_id);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev_id);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    e = hipMemcpyAsync(dev, p->image.data(), p->image.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (work list upload)");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize (work list upload)");
    p->dev = dev;
    p->cu_count = cus;
    int32_t g = 0;
    for (auto &l : p->launches) g = std::max(g, grid_for(*p, l[1] - l[0], cus));
    p->grid = g;
    return BSC_OK;
}

namespace bsc {

// Enqueue one contraction of plan p whose device region (work-list image,
// pack workspace, K-split partials) starts at `region`, on a device with
// `cu_count` compute units.
static bsc_status contract_on(Plan *p, const void *region, int32_t cu_count, const void *A, const void *B, void *C,
                              hipStream_t s) {
    const unsigned char *base = static_cast<const unsigned char *>(region);
    KArgs ka;
    ka.groups = reinterpret_cast<const DGroup *>(base + p->off_groups);
    ka.runs = reinterpret_cast<const DRun *>(base + p->off_runs);
    ka.ap = reinterpret_cast<const DView *>(base + p->off_ap);
    ka.bp = reinterpret_cast<const DView *>(base + p->off_bp);
    ka.cp = reinterpret_cast<const DView *>(base + p->off_cp);
    ka.tasks = reinterpret_cast<const DTask *>(base + p->off_tasks);
    ka.fast = reinterpret_cast<const DFast *>(base + p->off_fast);
    ka.tail = reinterpret_cast<const DFast *>(base + p->off_tail);
    ka.A = A;
    ka.B = B;
    ka.C = C;
    ka.W = base + p->off_ws;
    ka.P = reinterpret_cast<float *>(const_cast<unsigned char *>(base) + p->off_part);
    ka.cnt = reinterpret_cast<int32_t *>(const_cast<unsigned char *>(base) + p->off_cnt);
    {
        const int64_t esz = p->dtype == BSC_F64 ? 8 : (p->dtype == BSC_F32 ? 4 : 2);
        ka.a_bytes = p->a_elems * esz;
        ka.b_bytes = p->b_elems * esz;
        ka.w_bytes = p->ws_elems * esz;
    }
    if (!p->pack_tasks.empty()) {
        // gathers first, on the same stream: the grouped launch reads the workspace after them
        PArgs pa;
        pa.packs = reinterpret_cast<const DPack *>(base + p->off_packs);
        pa.tasks = reinterpret_cast<const DTask *>(base + p->off_ptasks);
        pa.ntasks = (int32_t)p->pack_tasks.size();
        pa.pad = 0;
        pa.A = A;
        pa.B = B;
        pa.W = const_cast<unsigned char *>(base) + p->off_ws;
        const int32_t cap = std::max(1, cu_count) * 8;
        dim3 grid((unsigned)std::max(1, std::min(pa.ntasks, cap)));
        launch_pack(p->dtype, grid, s, pa);
        p->stats.launches_issued++;
    }
    ka.vec_a = (reinterpret_cast<uintptr_t>(A) % 16) == 0;
    ka.vec_b = (reinterpret_cast<uintptr_t>(B) % 16) == 0;
    for (auto &l : p->launches) {
        ka.task0 = l[0];
        ka.ntasks = l[1] - l[0];
        const KernelRef k = p->dtype == BSC_F64   ? grouped_kernel_f64(p->features)
                            : p->dtype == BSC_F32 ? grouped_kernel_f32(p->features)
                                                  : pick_bf16(p->features, ka.vec_a && ka.vec_b, p->only_wide);
        dim3 grid((unsigned)grid_for(*p, ka.ntasks, cu_count)), block(k.threads);
        hipLaunchKernelGGL(k.fn, grid, block, k.lds, s, ka);
        p->stats.launches_issued++;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    return BSC_OK;
}

}  // namespace bsc

extern "C" bsc_status bsc_contract(bsc_plan_t plan, const void *A, const void *B, void *C, void *stream) {
    if (!plan) {
        set_error("bsc_contract: NULL plan");
        return BSC_ERR_ARG;
    }
    Plan *p = reinterpret_cast<Plan *>(plan);
    if (!p->dev) {
        set_error("bsc_contract: plan is not bound to a device region");
        return BSC_ERR_NOT_BOUND;
    }
    if ((!A && p->a_elems > 0) || (!B && p->b_elems > 0) || (!C && p->c_elems > 0)) {
        set_error("bsc_contract: NULL operand buffer");
        return BSC_ERR_ARG;
    }
    return contract_on(p, p->dev, p->cu_count, A, B, C, reinterpret_cast<hipStream_t>(stream));
}

// ---- contraction without a caller-provided device region ---------------------------
//
// For callers that cannot allocate device memory when they contract (code under
// graph capture, tight serving loops, harnesses that forbid allocation): the
// plan's device region — work-list image, pack workspace, K-split partial tiles
// and their counters — lives in one file-scope device array of fixed size
// instead of a region passed to bsc_plan_bind.  Each GPU holds its own copy of
// the array (loaded with the code object, held until the process ends); its
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is used from host code.

namespace bsc {

constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
constexpr int NOALLOC_MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

struct NoallocDevice {
    void *ptr = nullptr;   // device address of this GPU's scratch array
    int32_t cus = 0;       // compute units of this GPU
};
static std::mutex noalloc_mu;
static NoallocDevice noalloc_dev[NOALLOC_MAX_DEVICES];

// The current device's scratch address and CU count, looked up on first use.
static bsc_status noalloc_device(NoallocDevice &out) {
    int dev_id = 0;
    hipError_t e = hipGetDevice(&dev_id);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev_id < 0 || dev_id >= NOALLOC_MAX_DEVICES) {
        set_error("bsc_contract_noalloc: device index beyond " + std::to_string(NOALLOC_MAX_DEVICES));
        return BSC_ERR_UNSUPPORTED;
    }
    std::lock_guard<std::mutex> lock(noalloc_mu);
    NoallocDevice &d = noalloc_dev[dev_id];
    if (!d.ptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (scratch)");
        int cus = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev_id);
        if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
        d.cus = cus;
        d.ptr = ptr;
    }
    out = d;
    return BSC_OK;
}

}  // namespace bsc

extern "C" bsc_status bsc_contract_noalloc(bsc_plan_t plan, const void *A, const void *B, void *C, void *stream) {
    if (!plan) {
        set_error("bsc_contract_noalloc: NULL plan");
        return BSC_ERR_ARG;
    }
    Plan *p = reinterpret_cast<Plan *>(plan);
    if ((!A && p->a_elems > 0) || (!B && p->b_elems > 0) || (!C && p->c_elems > 0)) {
        set_error("bsc_contract_noalloc: NULL operand buffer");
        return BSC_ERR_ARG;
    }
    if (p->dev_bytes > NOALLOC_SCRATCH_BYTES) {
        set_error("bsc_contract_noalloc: the plan needs " + std::to_string(p->dev_bytes) +
                  " bytes of device scratch (work list + pack workspace + K-split partials), more than the " +
                  std::to_string(NOALLOC_SCRATCH_BYTES) + " the library holds per GPU; bind a region instead");
        return BSC_ERR_DEVICE_BYTES;
    }
    NoallocDevice d;
    bsc_status st = noalloc_device(d);
    if (st != BSC_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // the work-list image (its K-split counters zero) replaces whatever the last
    // call on this GPU left in the array, in stream order
    if (!p->image.empty()) {
        const hipError_t e = hipMemcpyAsync(d.ptr, p->image.data(), p->image.size(), hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (work list into scratch)");
    }
    return contract_on(p, d.ptr, d.cus, A, B, C, s);
}

// ---- captured chains (one graph launch per sequence of contractions) ----------------

namespace bsc {
struct Chain {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
};
}  // namespace bsc

extern "C" bsc_status bsc_chain_create(const bsc_plan_t *plans, const void *const *A, const void *const *B,
                                       void *const *C, int32_t n, bsc_chain_t *out) {
    set_error("");
    if (!plans || !A || !B || !C || !out || n < 1) {
        set_error("bsc_chain_create: NULL argument or n < 1");
        return BSC_ERR_ARG;
    }
    *out = nullptr;
    for (int32_t i = 0; i < n; ++i) {
        if (!plans[i]) {
            set_error("bsc_chain_create: NULL plan");
            return BSC_ERR_ARG;
        }
        if (!reinterpret_cast<Plan *>(plans[i])->dev) {
            set_error("bsc_chain_create: plan " + std::to_string(i) + " is not bound to a device region");
            return BSC_ERR_NOT_BOUND;
        }
    }
    hipStream_t cs = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);   // default priority
    if (e != hipSuccess) return hip_fail(e, "hipStreamCreateWithFlags (chain capture)");
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeRelaxed);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(cs);
        return hip_fail(e, "hipStreamBeginCapture");
    }
    bsc_status st = BSC_OK;
    for (int32_t i = 0; i < n && st == BSC_OK; ++i) st = bsc_contract(plans[i], A[i], B[i], C[i], cs);
    const std::string err = st == BSC_OK ? std::string() : std::string(bsc_last_error());
    Chain *ch = new Chain;
    e = hipStreamEndCapture(cs, &ch->graph);
    (void)hipStreamDestroy(cs);
    if (st != BSC_OK || e != hipSuccess) {
        if (ch->graph) (void)hipGraphDestroy(ch->graph);
        delete ch;
        if (st != BSC_OK) {
            set_error("bsc_chain_create: " + err);
            return st;
        }
        return hip_fail(e, "hipStreamEndCapture");
    }
    e = hipGraphInstantiate(&ch->exec, ch->graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(ch->graph);
        delete ch;
        return hip_fail(e, "hipGraphInstantiate");
    }
    *out = reinterpret_cast<bsc_chain_t>(ch);
    return BSC_OK;
}

extern "C" bsc_status bsc_chain_launch(bsc_chain_t chain, void *stream) {
    if (!chain) {
        set_error("bsc_chain_launch: NULL chain");
        return BSC_ERR_ARG;
    }
    Chain *ch = reinterpret_cast<Chain *>(chain);
    const hipError_t e = hipGraphLaunch(ch->exec, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
    return BSC_OK;
}

extern "C" void bsc_chain_destroy(bsc_chain_t chain) {
    if (!chain) return;
    Chain *ch = reinterpret_cast<Chain *>(chain);
    if (ch->exec) (void)hipGraphExecDestroy(ch->exec);
    if (ch->graph) (void)hipGraphDestroy(ch->graph);
    delete ch;
}
