// Tail bundles: whole tiny groups, one per wave, up to four per workgroup.
//
// About half the sector GEMMs of a block-sparse contraction carry near-zero
// flops (uni20 "block coalescing", Summary), so a 256-thread tile per tiny
// group spends most of its time on set-up and on its chain of dependent
// loads, with most of its threads idle.  A tail task instead hands each of the
// four waves of a workgroup one whole group that the wave computes alone:
//
//  * the wave reads its group's record: bases and strides of A, B and C (a
//    tail group is one run of single views, so every operand address is a
//    multiply-add: the same decode-at-plan-time records the dense tiles use);
//  * the K axis is taken in chunks of KC = TAIL_STAGE / (M + N) contracted
//    indices: the wave gathers the M x KC block of A and the KC x N block of B
//    into its own LDS region (every lane issuing eight loads before it stores
//    any), converted to the accumulation type;
//  * the outputs are spread over the 64 lanes: a group of at most 32 outputs
//    gives each output P lanes (P a power of two, P * M * N <= 64), lane p of
//    an output summing the indices k = p mod P, and the P partial sums are
//    added by a butterfly over the P lanes (a fixed order, so repeats are
//    bit-identical); larger groups give each lane up to TAIL_PER_LANE outputs;
//  * results go through C's record (the block's view).
//
// No workgroup barrier is used: waves of a bundle are independent and a wave
// without a group (bundles of fewer than four) returns at once.  Within a
// wave, LDS accesses execute in order, so the gather of the next chunk cannot
// overtake the reads of the current one.
#pragma once

#include "kernels_common.h"

namespace bsc {

template <typename ACC>
struct TailSmem {
    ACC stage[4][TAIL_STAGE];   // one region per wave: A chunk (M x KC) then B chunk (KC x N)
};

__device__ __forceinline__ int32_t tail_lanes(int32_t mn) { return tail_lanes_host(mn); }

template <typename ACC>
__device__ __forceinline__ ACC tail_xor(ACC v, int32_t m) { return __shfl_xor(v, m, 64); }

// Gather n elements (element e from load(e)) into dst: each lane loads
// TAIL_BATCH elements (e = lane, lane + 64, ...) before storing any, so a
// batch's loads are in flight together instead of one memory round trip each.
constexpr int TAIL_BATCH = 8;
template <typename ACC, typename Load>
__device__ __forceinline__ void tail_gather(ACC *dst, int32_t n, int32_t lane, Load &&load) {
    for (int32_t base = 0; base < n; base += 64 * TAIL_BATCH) {
        ACC v[TAIL_BATCH];
#pragma unroll
        for (int u = 0; u < TAIL_BATCH; ++u) {
            const int32_t e = base + lane + 64 * u;
            v[u] = e < n ? load(e) : ACC(0);
        }
#pragma unroll
        for (int u = 0; u < TAIL_BATCH; ++u) {
            const int32_t e = base + lane + 64 * u;
            if (e < n) dst[e] = v[u];
        }
    }
}

template <typename TA, typename TC, typename ACC>
__device__ __forceinline__ void tail_bundle(const KArgs &ka, const DTask &task, TailSmem<ACC> &sm) {
    const int32_t w = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
    const int32_t lane = tid_x() & 63;
    if (w >= task.m0) return;
    const DFast f = ka.tail[task.group + w];
    const int32_t M = f.mlen, N = f.nlen, MN = M * N;
    const int32_t KC = TAIL_STAGE / (M + N);   // >= 1: the planner keeps M + N <= TAIL_STAGE
    const int32_t P = tail_lanes(MN);
    const int32_t ostep = 64 / P, part = lane % P, o0 = lane / P;
    ACC *const sa = sm.stage[w];
    ACC *const sb = sa + M * KC;

    ACC acc[TAIL_PER_LANE];
#pragma unroll
    for (int q = 0; q < TAIL_PER_LANE; ++q) acc[q] = ACC(0);

    auto compute = [&](int32_t kl) {
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < TAIL_PER_LANE; ++q) {
            const int32_t o = o0 + ostep * q;
            if (o >= MN) break;
            const int32_t i = o / N, j = o - i * N;
            ACC s = acc[q];
            for (int32_t kk = part; kk < kl; kk += P) s = fma(sa[i * kl + kk], sb[kk * N + j], s);
            acc[q] = s;
        }
        __builtin_amdgcn_wave_barrier();
    };

    const TA *A = static_cast<const TA *>((f.flags & F_A_WS) ? ka.W : ka.A);
    const TA *B = static_cast<const TA *>((f.flags & F_B_WS) ? ka.W : ka.B);
    for (int32_t k0 = 0; k0 < f.K; k0 += KC) {
        const int32_t kl = min(KC, f.K - k0);
        tail_gather(sa, M * kl, lane, [&](int32_t e) {
            const int32_t i = e / kl, kk = e - i * kl;
            return load_acc(A, f.a_base + static_cast<int64_t>(i) * f.a_rs + static_cast<int64_t>(k0 + kk) * f.a_ks);
        });
        tail_gather(sb, kl * N, lane, [&](int32_t e) {
            const int32_t kk = e / N, j = e - kk * N;
            return load_acc(B, f.b_base + static_cast<int64_t>(k0 + kk) * f.b_ks + static_cast<int64_t>(j) * f.b_ns);
        });
        compute(kl);
    }
    // the P lanes of an output add their partial sums (butterfly, fixed order)
    for (int32_t m = 1; m < P; m *= 2) {
#pragma unroll
        for (int q = 0; q < TAIL_PER_LANE; ++q) acc[q] += tail_xor(acc[q], m);
    }
    if (part != 0) return;

    TC *Cp = static_cast<TC *>(ka.C);
    const bool accum = (f.flags & G_ACCUMULATE) != 0;
#pragma unroll
    for (int q = 0; q < TAIL_PER_LANE; ++q) {
        const int32_t o = o0 + ostep * q;
        if (o >= MN) break;
        const int32_t i = o / N, j = o - i * N;
        const int64_t ad = f.c_base + static_cast<int64_t>(i) * f.c_rs + static_cast<int64_t>(j) * f.c_cs;
        ACC v = acc[q];
        if (accum) v += static_cast<ACC>(Cp[ad]);
        Cp[ad] = static_cast<TC>(v);
    }
}

}  // namespace bsc
