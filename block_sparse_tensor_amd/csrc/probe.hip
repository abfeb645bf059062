// Matrix-core issue-rate probe: the measured peak the roofline fractions can be
// read against, next to the published one.  Every wave keeps several
// independent accumulators busy with back-to-back matrix-core operations of
// one kind (the instruction the tiles of that dtype use), operands in
// registers, no memory traffic: the launch's time is the rate at which the
// chip retires them at its clock under this load.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>

#include "bsc_internal.h"

namespace bsc {

typedef __bf16 pr_bf16x8 __attribute__((ext_vector_type(8)));
typedef float pr_f32x16 __attribute__((ext_vector_type(16)));
typedef float pr_f32x4 __attribute__((ext_vector_type(4)));
typedef double pr_f64x4 __attribute__((ext_vector_type(4)));

constexpr int PROBE_CHAINS = 4;   // independent accumulators per wave
constexpr int PROBE_WGS_PER_CU = 8;  // workgroups per CU: two waves per SIMD

// flops of one operation of each kind
constexpr double PROBE_FLOP_BF16 = 2.0 * 32 * 32 * 16;   // v_mfma_f32_32x32x16_bf16
constexpr double PROBE_FLOP_F32 = 2.0 * 16 * 16 * 4;     // v_mfma_f32_16x16x4_f32
constexpr double PROBE_FLOP_F64 = 2.0 * 16 * 16 * 4;     // v_mfma_f64_16x16x4_f64

// The accumulators feed a store (to sink[0]) that happens only if their sum
// equals sink_key, which no sum reaches (every sum is positive and the key is
// negative), so the work cannot be removed and nothing is ever written.
__global__ __launch_bounds__(256) void probe_bf16(float *sink, int32_t iters, float sink_key) {
    const int32_t t = threadIdx.x;
    pr_bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(1.0f + 0.001f * (t + i));
        b[i] = static_cast<__bf16>(1.0f - 0.001f * (t + i));
    }
    pr_f32x16 c[PROBE_CHAINS];
    for (int q = 0; q < PROBE_CHAINS; ++q)
        for (int i = 0; i < 16; ++i) c[q][i] = 0.0f;
    for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < PROBE_CHAINS; ++q) c[q] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[q], 0, 0, 0);
    }
    float s = 0.0f;
    for (int q = 0; q < PROBE_CHAINS; ++q)
        for (int i = 0; i < 16; ++i) s += c[q][i];
    if (s == sink_key) sink[0] = s;
}

__global__ __launch_bounds__(256) void probe_f32(float *sink, int32_t iters, float sink_key) {
    const int32_t t = threadIdx.x;
    const float a = 1.0f + 0.001f * t, b = 1.0f - 0.001f * t;
    pr_f32x4 c[2 * PROBE_CHAINS];
    for (int q = 0; q < 2 * PROBE_CHAINS; ++q) c[q] = pr_f32x4{0, 0, 0, 0};
    for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < 2 * PROBE_CHAINS; ++q) c[q] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c[q], 0, 0, 0);
    }
    float s = 0.0f;
    for (int q = 0; q < 2 * PROBE_CHAINS; ++q) s += c[q][0] + c[q][1] + c[q][2] + c[q][3];
    if (s == sink_key) sink[0] = s;
}

__global__ __launch_bounds__(256) void probe_f64(float *sink, int32_t iters, float sink_key) {
    const int32_t t = threadIdx.x;
    const double a = 1.0 + 0.001 * t, b = 1.0 - 0.001 * t;
    pr_f64x4 c[2 * PROBE_CHAINS];
    for (int q = 0; q < 2 * PROBE_CHAINS; ++q) c[q] = pr_f64x4{0, 0, 0, 0};
    for (int32_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < 2 * PROBE_CHAINS; ++q) c[q] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c[q], 0, 0, 0);
    }
    double s = 0.0;
    for (int q = 0; q < 2 * PROBE_CHAINS; ++q) s += c[q][0] + c[q][1] + c[q][2] + c[q][3];
    if (static_cast<float>(s) == sink_key) sink[0] = static_cast<float>(s);
}

}  // namespace bsc

using namespace bsc;

extern "C" bsc_status bsc_probe_mfma(bsc_dtype dtype, int32_t iters, float *sink, void *stream, double *flops) {
    set_error("");
    if (!sink || !flops || iters < 1) {
        set_error("bsc_probe_mfma: NULL sink or flops, or iters < 1");
        return BSC_ERR_ARG;
    }
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) {
        set_error(std::string("bsc_probe_mfma: ") + hipGetErrorString(e));
        return BSC_ERR_HIP;
    }
    // eight workgroups of four waves per CU: two waves per SIMD
    const int32_t wgs = std::max(1, cus) * PROBE_WGS_PER_CU;
    const double waves = (double)wgs * 4.0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const float key = -1.0f;   // never reached: every accumulator sum is positive
    switch (dtype) {
    case BSC_BF16_F32:
        hipLaunchKernelGGL(probe_bf16, dim3(wgs), dim3(256), 0, s, sink, iters, key);
        *flops = waves * iters * PROBE_CHAINS * PROBE_FLOP_BF16;
        break;
    case BSC_F32:
        hipLaunchKernelGGL(probe_f32, dim3(wgs), dim3(256), 0, s, sink, iters, key);
        *flops = waves * iters * 2 * PROBE_CHAINS * PROBE_FLOP_F32;
        break;
    case BSC_F64:
        hipLaunchKernelGGL(probe_f64, dim3(wgs), dim3(256), 0, s, sink, iters, key);
        *flops = waves * iters * 2 * PROBE_CHAINS * PROBE_FLOP_F64;
        break;
    default:
        set_error("bsc_probe_mfma: unknown dtype");
        return BSC_ERR_ARG;
    }
    e = hipGetLastError();
    if (e != hipSuccess) {
        set_error(std::string("bsc_probe_mfma: launch: ") + hipGetErrorString(e));
        return BSC_ERR_HIP;
    }
    return BSC_OK;
}
