// Generic workgroup tile: any strided views, any dtype, vector-ALU FMAs.
//
// A 256-thread workgroup computes a 64 x 64 tile of one coalesced group GEMM.
// For each run of the group it first resolves, once per tile row and column,
// which piece (member block view) the row or column belongs to and where it
// starts; the K loop then reads elements through those per-row records
// (index decoding paid once per tile, not per element).  Operand chunks of
// 64 x 16 are staged through LDS; each thread owns a 4 x 4 sub-tile with rows
// and columns strided by 16 so LDS reads are conflict-free.
#pragma once

#include "kernels_common.h"

namespace bsc {

template <typename ACC>
struct GenericSmem {
    ACC a[16][65];   // [k][row]
    ACC b[16][65];   // [k][col]
    Rec ra[64];
    Rec rb[64];
};

template <typename TA, typename TC, typename ACC>
__device__ __forceinline__ void generic_tile(const KArgs &ka, const DTask &task, GenericSmem<ACC> &sm) {
    const DGroup g = ka.groups[task.group];
    const int32_t tid = tid_x();
    const int32_t m0 = task.m0, n0 = task.n0;
    const int32_t mlen = min(64, g.M - m0), nlen = min(64, g.N - n0);
    const int32_t tx = tid & 15, ty = tid >> 4;

    ACC acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = ACC(0);

    for (int32_t r = 0; r < g.nrun; ++r) {
        const DRun run = ka.runs[g.run0 + r];
        __syncthreads();
        if (tid < 64) {
            if (tid < mlen) sm.ra[tid] = make_rec(ka.ap + run.ap0, run.nap, m0 + tid);
        } else if (tid < 128) {
            const int32_t j = tid - 64;
            if (j < nlen) sm.rb[j] = make_rec(ka.bp + run.bp0, run.nbp, n0 + j);
        }
        __syncthreads();
        const TA *A = run_a<TA>(ka, run.flags);
        const TA *B = run_b<TA>(ka, run.flags);
        const bool a_k = (run.flags & R_A_KUNIT) != 0;
        const bool b_k = (run.flags & R_B_KUNIT) != 0;
        for (int32_t k0 = 0; k0 < run.K; k0 += 16) {
            const int32_t kl = min(16, run.K - k0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int32_t e = tid + q * 256;
                int32_t i, kk;
                if (a_k) { i = e >> 4; kk = e & 15; }
                else { i = e & 63; kk = e >> 6; }
                ACC v = ACC(0);
                if (i < mlen && kk < kl) v = load_acc(A, along(sm.ra[i], k0 + kk));
                sm.a[kk][i] = v;
                int32_t j, kb;
                if (b_k) { j = e >> 4; kb = e & 15; }
                else { j = e & 63; kb = e >> 6; }
                ACC w = ACC(0);
                if (j < nlen && kb < kl) w = load_acc(B, along(sm.rb[j], k0 + kb));
                sm.b[kb][j] = w;
            }
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) {
                ACC a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = sm.a[kk][ty + 16 * i];
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = sm.b[kk][tx + 16 * j];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
            }
            __syncthreads();
        }
    }

    // epilogue: scatter through the C pieces (the per-block views)
    __syncthreads();
    const bool cn = (g.flags & G_C_ALONG_N) != 0;
    if (tid < 64) {
        if (!cn && tid < mlen) sm.ra[tid] = make_rec(ka.cp + g.cp0, g.ncp, m0 + tid);
        if (cn && tid < nlen) sm.ra[tid] = make_rec(ka.cp + g.cp0, g.ncp, n0 + tid);
    }
    __syncthreads();
    TC *Cp = static_cast<TC *>(ka.C);
    const bool accum = (g.flags & G_ACCUMULATE) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int32_t ii = ty + 16 * i;
        if (ii >= mlen) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int32_t jj = tx + 16 * j;
            if (jj >= nlen) continue;
            const int64_t ad = cn ? along(sm.ra[jj], m0 + ii) : along(sm.ra[ii], n0 + jj);
            ACC v = acc[i][j];
            if (accum) v += static_cast<ACC>(Cp[ad]);
            Cp[ad] = static_cast<TC>(v);
        }
    }
}

}  // namespace bsc
