// Device-side helpers shared by the tile kernels: kernel arguments, per-row
// address records built from the strided pieces, and element loads.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "bsc_internal.h"

namespace bsc {

struct KArgs {
    int32_t vec_a, vec_b;   // operand base pointers are 16-byte aligned
    const DTask *tasks;
    int32_t task0, ntasks;
    const DGroup *groups;
    const DRun *runs;
    const DView *ap, *bp, *cp;
    const DFast *fast;
    const DFast *tail;      // tail entries (record of each wave's group in a T_TAIL bundle)
    const void *A, *B;
    void *C;
    const void *W;          // pack workspace (operands of runs flagged R_A_WS / R_B_WS)
    float *P;               // K-split partial tiles
    int32_t *cnt;           // K-split arrival counters (zero between launches)
    int64_t a_bytes, b_bytes, w_bytes;   // sizes of A, B and the pack workspace
};

// The thread's index within the workgroup, taken through an empty asm so each
// use is a fresh value: lane offsets derived from it are then computed inside
// the persistent task loop, where the tile body that needs them runs, instead
// of being hoisted in front of the loop and held live across every tile body
// (which pushes the register allocation into scratch spills).
__device__ __forceinline__ uint32_t tid_x() {
    uint32_t t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Buffer a run's A (B) pieces address: the caller's operand or the workspace.
template <typename T>
__device__ __forceinline__ const T *run_a(const KArgs &ka, int32_t run_flags) {
    return static_cast<const T *>((run_flags & R_A_WS) ? ka.W : ka.A);
}
template <typename T>
__device__ __forceinline__ const T *run_b(const KArgs &ka, int32_t run_flags) {
    return static_cast<const T *>((run_flags & R_B_WS) ? ka.W : ka.B);
}

// Address function along the non-piece axis of one row/column of a piece.
struct Rec {
    int64_t base;
    int64_t s0, s1;
    int32_t in, pad;
};


__device__ __forceinline__ float load_acc(const uint16_t *p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float load_acc(const float *p, int64_t i) { return p[i]; }
__device__ __forceinline__ double load_acc(const double *p, int64_t i) { return p[i]; }

// last piece whose range starts at or before x (pieces are sorted by begin)
__device__ __forceinline__ int32_t find_piece(const DView *pc, int32_t n, int32_t x) {
    int32_t lo = 0, hi = n - 1;
    while (lo < hi) {
        int32_t mid = (lo + hi + 1) >> 1;
        if (pc[mid].begin <= x) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ Rec make_rec(const DView *pc, int32_t n, int32_t x) {
    const int32_t p = n == 1 ? 0 : find_piece(pc, n, x);
    const DView v = pc[p];
    const int32_t xl = x - v.begin;
    Rec r;
    if (v.ia == 1) r.base = v.off + static_cast<int64_t>(xl) * v.sa0;   // single leg: no division
    else r.base = v.off + static_cast<int64_t>(xl / v.ia) * v.sa0 + static_cast<int64_t>(xl % v.ia) * v.sa1;
    r.s0 = v.sb0;
    r.s1 = v.sb1;
    r.in = v.ib;
    r.pad = 0;
    return r;
}

__device__ __forceinline__ int64_t along(const Rec &r, int32_t y) {
    if (r.in == 1) return r.base + static_cast<int64_t>(y) * r.s0;
    return r.base + static_cast<int64_t>(y / r.in) * r.s0 + static_cast<int64_t>(y % r.in) * r.s1;
}

}  // namespace bsc
