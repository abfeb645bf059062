// Device side of the engine: work-list upload and the grouped contraction launch.
//
// One launch walks the whole work list (uni20 "block coalescing", section
// "Summary": issue fewer, larger kernels instead of one per sector GEMM).  A
// workgroup takes tasks blockIdx.x, blockIdx.x + gridDim.x, ... from a
// longest-first list, so the grid can be sized to the machine (persistent
// workgroups) or to the task count.  No task waits on another: every C tile has
// exactly one owner, so sums need no atomics and repeat bit-for-bit.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <string>

#include "bsc_internal.h"
#include "kernels_generic.h"
#include "kernels_mfma_bf16.h"

namespace bsc {

static bsc_status hip_fail(hipError_t e, const char *what) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return BSC_ERR_HIP;
}

template <typename ACC, bool BF16>
union TileSmem;
template <typename ACC>
union TileSmem<ACC, false> {
    GenericSmem<ACC> g;
};
template <typename ACC>
union TileSmem<ACC, true> {
    GenericSmem<ACC> g;
    MfmaSmemBf16 m;
};

template <typename TA, typename TC, typename ACC>
__global__ __launch_bounds__(256) void grouped_contract(KArgs ka) {
    constexpr bool kBf16 = sizeof(TA) == 2;
    __shared__ TileSmem<ACC, kBf16> sm;
    for (int32_t t = blockIdx.x; t < ka.ntasks; t += gridDim.x) {
        const DTask task = ka.tasks[ka.task0 + t];
        if constexpr (kBf16) {
            if (task.cls == T_MFMA) {
                mfma_tile_bf16<TC>(ka, task, sm.m);
                continue;
            }
        }
        generic_tile<TA, TC, ACC>(ka, task, sm.g);
    }
}

static int32_t grid_for(const Plan &p, int32_t ntasks) {
    int32_t cap = p.opt.grid_limit > 0 ? p.opt.grid_limit : std::max(1, p.cu_count) * 8;
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
    e = hipMemcpyAsync(dev, p->image.data(), p->dev_bytes, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync (work list upload)");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize (work list upload)");
    p->dev = dev;
    p->cu_count = cus;
    int32_t g = 0;
    for (auto &l : p->launches) g = std::max(g, grid_for(*p, l[1] - l[0]));
    p->grid = g;
    return BSC_OK;
}

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
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const unsigned char *base = static_cast<const unsigned char *>(p->dev);
    KArgs ka;
    ka.groups = reinterpret_cast<const DGroup *>(base + p->off_groups);
    ka.runs = reinterpret_cast<const DRun *>(base + p->off_runs);
    ka.ap = reinterpret_cast<const DView *>(base + p->off_ap);
    ka.bp = reinterpret_cast<const DView *>(base + p->off_bp);
    ka.cp = reinterpret_cast<const DView *>(base + p->off_cp);
    ka.tasks = reinterpret_cast<const DTask *>(base + p->off_tasks);
    ka.A = A;
    ka.B = B;
    ka.C = C;
    ka.vec_a = (reinterpret_cast<uintptr_t>(A) % 16) == 0;
    ka.vec_b = (reinterpret_cast<uintptr_t>(B) % 16) == 0;
    for (auto &l : p->launches) {
        ka.task0 = l[0];
        ka.ntasks = l[1] - l[0];
        dim3 grid((unsigned)grid_for(*p, ka.ntasks)), block(256);
        switch (p->dtype) {
            case BSC_F64: hipLaunchKernelGGL((grouped_contract<double, double, double>), grid, block, 0, s, ka); break;
            case BSC_F32: hipLaunchKernelGGL((grouped_contract<float, float, float>), grid, block, 0, s, ka); break;
            case BSC_BF16_F32: hipLaunchKernelGGL((grouped_contract<uint16_t, float, float>), grid, block, 0, s, ka); break;
        }
        p->stats.launches_issued++;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    return BSC_OK;
}
