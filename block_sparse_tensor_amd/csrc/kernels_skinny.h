// Skinny tile: groups whose output has at most SK_SHORT rows or columns.
//
// Such a GEMM moves far more bytes than it computes on (a tall operand times a
// handful of coefficients: the MPO stage of the environment update is the
// typical case), so it is bound by HBM, not by the matrix cores.  The tile
// covers SK_LONG positions of the long output axis and the whole short axis.
// Every thread owns one line along the long axis (neighbouring threads touch
// neighbouring lines), streams its line of the
// long operand straight from global memory, and multiplies them by the short
// operand, which the workgroup stages in LDS once per chunk of the contracted
// axis and every thread reads by broadcast.  No matrix-core step and no
// operand reuse through LDS: the long operand is read exactly once.
#pragma once

#include "kernels_common.h"

namespace bsc {

constexpr int SK_LONG = 256;    // positions along the long axis per tile (one per thread)
constexpr int SK_SHORT = 16;    // largest short extent
constexpr int SK_KC = 64;       // contracted indices per LDS chunk of the short operand
constexpr int SK_PER = SK_LONG / 256;

template <typename ACC>
struct SkinnySmem {
    ACC s[SK_KC][SK_SHORT];     // short operand chunk, [k][y]
    Rec rs[SK_SHORT];           // records of the short operand's lines
    Rec rc[SK_SHORT];           // C records along the short axis (when C is cut along it)
};

// LONG_M: the long axis is M (A is the long operand, B the short one);
// otherwise the long axis is N (B long, A short).
template <typename TA, typename TC, typename ACC, bool LONG_M>
__device__ __forceinline__ void skinny_tile(const KArgs &ka, const DTask &task, SkinnySmem<ACC> &sm) {
    const DGroup g = ka.groups[task.group];
    const int32_t tid = threadIdx.x;
    const int32_t x0 = LONG_M ? task.m0 : task.n0;
    const int32_t X = LONG_M ? g.M : g.N;
    const int32_t Y = LONG_M ? g.N : g.M;
    const int32_t xlen = min(SK_LONG, X - x0);

    ACC acc[SK_PER][SK_SHORT];
#pragma unroll
    for (int q = 0; q < SK_PER; ++q)
#pragma unroll
        for (int y = 0; y < SK_SHORT; ++y) acc[q][y] = ACC(0);

    for (int32_t r = 0; r < g.nrun; ++r) {
        const DRun run = ka.runs[g.run0 + r];
        const DView *lp = LONG_M ? ka.ap + run.ap0 : ka.bp + run.bp0;
        const DView *sp = LONG_M ? ka.bp + run.bp0 : ka.ap + run.ap0;
        const int32_t nl = LONG_M ? run.nap : run.nbp;
        const int32_t ns = LONG_M ? run.nbp : run.nap;
        const TA *Pl = LONG_M ? run_a<TA>(ka, run.flags) : run_b<TA>(ka, run.flags);
        const TA *Ps = LONG_M ? run_b<TA>(ka, run.flags) : run_a<TA>(ka, run.flags);
        Rec rl[SK_PER];
#pragma unroll
        for (int q = 0; q < SK_PER; ++q) {
            const int32_t x = tid + 256 * q;
            if (x < xlen) rl[q] = make_rec(lp, nl, x0 + x);
        }
        __syncthreads();   // the previous run's short chunk may still be read
        if (tid < Y) sm.rs[tid] = make_rec(sp, ns, tid);
        for (int32_t k0 = 0; k0 < run.K; k0 += SK_KC) {
            const int32_t kl = min(SK_KC, run.K - k0);
            __syncthreads();
            // stage the short operand chunk: element (k, y), zero outside the group
#pragma unroll
            for (int i = 0; i < SK_KC * SK_SHORT / 256; ++i) {
                const int32_t e = tid + 256 * i;
                const int32_t k = e / SK_SHORT, y = e % SK_SHORT;
                sm.s[k][y] = (k < kl && y < Y) ? load_acc(Ps, along(sm.rs[y], k0 + k)) : ACC(0);
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < SK_PER; ++q) {
                if (tid + 256 * q >= xlen) continue;
                const Rec rq = rl[q];
#pragma unroll 1
                for (int32_t k = 0; k < kl; ++k) {
                    const ACC a = load_acc(Pl, along(rq, k0 + k));
#pragma unroll
                    for (int y = 0; y < SK_SHORT; ++y) acc[q][y] = fma(a, sm.s[k][y], acc[q][y]);
                }
            }
        }
    }

    // epilogue through the C pieces: C is cut either along the long axis (one
    // record per thread line) or along the short axis (records in LDS)
    const bool cn = (g.flags & G_C_ALONG_N) != 0;
    const bool c_long = LONG_M ? !cn : cn;
    __syncthreads();
    if (!c_long && tid < Y) sm.rc[tid] = make_rec(ka.cp + g.cp0, g.ncp, (LONG_M ? task.n0 : task.m0) + tid);
    __syncthreads();
    TC *Cp = static_cast<TC *>(ka.C);
    const bool accum = (g.flags & G_ACCUMULATE) != 0;
#pragma unroll
    for (int q = 0; q < SK_PER; ++q) {
        const int32_t x = tid + 256 * q;
        if (x >= xlen) continue;
        Rec rcl;
        if (c_long) rcl = make_rec(ka.cp + g.cp0, g.ncp, x0 + x);
#pragma unroll
        for (int y = 0; y < SK_SHORT; ++y) {
            if (y >= Y) break;
            const int64_t ad = c_long ? along(rcl, y) : along(sm.rc[y], x0 + x);
            ACC v = acc[q][y];
            if (accum) v += static_cast<ACC>(Cp[ad]);
            Cp[ad] = static_cast<TC>(v);
        }
    }
    __syncthreads();
}

}  // namespace bsc
