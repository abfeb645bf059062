// Device side of the fused two-stage plan: work-list upload and the launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "kernels_fused.h"

namespace bsc {

static bsc_status fused_hip_fail(hipError_t e, const char *what) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return BSC_ERR_HIP;
}

}  // namespace bsc

using namespace bsc;

extern "C" bsc_status bsc_fused_bind(bsc_fused_t plan, void *dev, size_t bytes, void *stream) {
    set_error("");
    if (!plan || !dev) {
        set_error("bsc_fused_bind: NULL argument");
        return BSC_ERR_ARG;
    }
    FusedPlan *f = reinterpret_cast<FusedPlan *>(plan);
    if (bytes < f->image.size()) {
        set_error("bsc_fused_bind: device region smaller than bsc_fused_device_bytes");
        return BSC_ERR_DEVICE_BYTES;
    }
    if (reinterpret_cast<uintptr_t>(dev) % 256 != 0) {
        set_error("bsc_fused_bind: device region must be 256-byte aligned");
        return BSC_ERR_ARG;
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int dev_id = 0;
    hipError_t e = hipGetDevice(&dev_id);
    if (e != hipSuccess) return fused_hip_fail(e, "hipGetDevice");
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev_id);
    if (e != hipSuccess) return fused_hip_fail(e, "hipDeviceGetAttribute");
    e = hipMemcpyAsync(dev, f->image.data(), f->image.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return fused_hip_fail(e, "hipMemcpyAsync (fused work list upload)");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fused_hip_fail(e, "hipStreamSynchronize (fused work list upload)");
    f->dev = dev;
    f->cu_count = cus;
    return BSC_OK;
}

extern "C" bsc_status bsc_fused_contract(bsc_fused_t plan, const void *A1, const void *B1, const void *B2, void *C2,
                                         void *stream) {
    if (!plan) {
        set_error("bsc_fused_contract: NULL plan");
        return BSC_ERR_ARG;
    }
    FusedPlan *f = reinterpret_cast<FusedPlan *>(plan);
    if (!f->dev) {
        set_error("bsc_fused_contract: plan is not bound to a device region");
        return BSC_ERR_NOT_BOUND;
    }
    if ((!A1 && f->a_elems > 0) || (!B1 && f->b_elems > 0) || (!B2 && !f->stream && f->w_elems > 0) ||
        (!C2 && f->c_elems > 0)) {
        set_error("bsc_fused_contract: NULL operand buffer");
        return BSC_ERR_ARG;
    }
    if (f->parts.empty()) return BSC_OK;
    const unsigned char *base = static_cast<const unsigned char *>(f->dev);
    FArgs fa;
    fa.pchans = reinterpret_cast<const FChan *>(base + f->off_pchans);
    fa.outs = reinterpret_cast<const FOut *>(base + f->off_outs);
    fa.widx = reinterpret_cast<const int32_t *>(base + f->off_widx);
    fa.parts = reinterpret_cast<const FPart *>(base + f->off_parts);
    fa.nwg = (int32_t)(f->parts.size() / 4);
    fa.no = f->outs_per_task;
    fa.A = A1;
    fa.B = B1;
    fa.W = f->stream ? static_cast<const void *>(base + f->off_ones) : B2;   // a stream plan's own weight 1
    fa.C = C2;
    // four part records per workgroup (longest parts first)
    dim3 grid((unsigned)fa.nwg), block(256);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (f->dtype == BSC_F64) {
        if (fa.no == 1) hipLaunchKernelGGL((fused_contract<double, 1, 1>), grid, block, 0, s, fa);
        else if (fa.no == 4) hipLaunchKernelGGL((fused_contract<double, 4, 1>), grid, block, 0, s, fa);
        else if (fa.no == 8) hipLaunchKernelGGL((fused_contract<double, 8, 1>), grid, block, 0, s, fa);
        else hipLaunchKernelGGL((fused_contract<double, FUSED_MAX_OUT, 1>), grid, block, 0, s, fa);
    } else if (f->tile_blocks == 2) {
        if (fa.no == 1) hipLaunchKernelGGL((fused_contract<float, 1, 2>), grid, block, 0, s, fa);
        else hipLaunchKernelGGL((fused_contract<float, 4, 2>), grid, block, 0, s, fa);
    } else {
        if (fa.no == 1) hipLaunchKernelGGL((fused_contract<float, 1, 1>), grid, block, 0, s, fa);
        else if (fa.no == 4) hipLaunchKernelGGL((fused_contract<float, 4, 1>), grid, block, 0, s, fa);
        else if (fa.no == 8) hipLaunchKernelGGL((fused_contract<float, 8, 1>), grid, block, 0, s, fa);
        else hipLaunchKernelGGL((fused_contract<float, FUSED_MAX_OUT, 1>), grid, block, 0, s, fa);
    }
    f->launches_issued++;
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fused_hip_fail(e, "kernel launch (fused)");
    return BSC_OK;
}
