// Skinny tile: groups whose output has at most SK_SHORT rows or columns.
//
// Such a GEMM moves far more bytes than it computes on (a tall operand times a
// handful of coefficients: the MPO stage of the environment update is the
// typical case, often a single output column), so it is bound by HBM, not by
// the matrix cores.  The tile covers 256 * R positions of the long output axis
// and the whole short axis.  Thread t owns lines t, t + 256, ..., t + 256 (R-1)
// of the long axis (so a wave's loads of one contracted index touch 64
// neighbouring lines), streams them straight from global memory and
// multiplies them by the short operand, which the workgroup stages in LDS once
// per chunk of the contracted axis and every thread reads by broadcast.  R is
// chosen so that R times the short extent (rounded up to 4, 8 or 16) fills a
// fixed register budget of accumulators: a single-column group covers 2048
// lines per tile, so every tile streams tens of KB and the per-tile set-up is
// paid rarely.  No matrix-core step and no operand
// reuse through LDS: the long operand is read exactly once.
#pragma once

#include "kernels_common.h"

namespace bsc {

constexpr int SK_SHORT = 16;    // largest short extent
constexpr int SK_KC = 64;       // contracted indices per LDS chunk of the short operand

template <typename ACC>
struct SkinnySmem {
    ACC s[SK_KC][SK_SHORT];     // short operand chunk, [k][y]
    Rec rs[SK_SHORT];           // records of the short operand's lines
    Rec rc[SK_SHORT];           // C records along the short axis (when C is cut along it)
};

// Walks the pieces of one view list forward along the long axis: a thread's
// lines increase, so the piece of the next line is the current one unless the
// line reaches the next piece's start; only then is the list searched.
struct PieceWalk {
    const DView *pc;
    int32_t n, p, next;    // pieces, current piece, first line of the next piece
    DView v;               // current piece
};

__device__ __forceinline__ void walk_start(PieceWalk &w, const DView *pc, int32_t n, int32_t x) {
    w.pc = pc;
    w.n = n;
    w.p = n == 1 ? 0 : find_piece(pc, n, x);
    w.v = pc[w.p];
    w.next = w.p + 1 < n ? pc[w.p + 1].begin : 0x7fffffff;
}

__device__ __forceinline__ void walk_to(PieceWalk &w, int32_t x) {
    if (x < w.next) return;
    int32_t lo = w.p + 1, hi = w.n - 1;   // x lies in a later piece
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (w.pc[mid].begin <= x) lo = mid;
        else hi = mid - 1;
    }
    w.p = lo;
    w.v = w.pc[lo];
    w.next = lo + 1 < w.n ? w.pc[lo + 1].begin : 0x7fffffff;
}

// offset of line x of the walk's current piece along the piece axis
__device__ __forceinline__ int64_t walk_base(const PieceWalk &w, int32_t x) {
    const int32_t xl = x - w.v.begin;
    if (w.v.ia == 1) return w.v.off + static_cast<int64_t>(xl) * w.v.sa0;
    return w.v.off + static_cast<int64_t>(xl / w.v.ia) * w.v.sa0 + static_cast<int64_t>(xl % w.v.ia) * w.v.sa1;
}

// Accumulators per thread.  32 keeps the skinny bodies' register demand below
// the matrix-core tiles' that share the kernel (a larger budget made the whole
// kernel spill).
template <typename ACC>
constexpr int skinny_acc_budget() { return 32; }

// LONG_M: the long axis is M (A is the long operand, B the short one);
// otherwise the long axis is N (B long, A short).  YB: short extent rounded up
// (4, 8 or 16); R = lines per thread.
template <typename TA, typename TC, typename ACC, bool LONG_M, int YB>
__device__ __forceinline__ void skinny_impl(const KArgs &ka, const DTask &task, const DGroup &g, SkinnySmem<ACC> &sm) {
    constexpr int R = skinny_acc_budget<ACC>() / YB;
    const int32_t tid = tid_x();
    const int32_t x0 = LONG_M ? task.m0 : task.n0;
    const int32_t X = LONG_M ? g.M : g.N;
    const int32_t Y = LONG_M ? g.N : g.M;
    const int32_t xlen = min(256 * R, X - x0);

    ACC acc[R][YB];
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
        for (int y = 0; y < YB; ++y) acc[q][y] = ACC(0);

    for (int32_t r = 0; r < g.nrun; ++r) {
        const DRun run = ka.runs[g.run0 + r];
        const DView *lp = LONG_M ? ka.ap + run.ap0 : ka.bp + run.bp0;
        const DView *sp = LONG_M ? ka.bp + run.bp0 : ka.ap + run.ap0;
        const int32_t nl = LONG_M ? run.nap : run.nbp;
        const int32_t ns = LONG_M ? run.nbp : run.nap;
        const TA *Pl = LONG_M ? run_a<TA>(ka, run.flags) : run_b<TA>(ka, run.flags);
        const TA *Ps = LONG_M ? run_b<TA>(ka, run.flags) : run_a<TA>(ka, run.flags);
        // this thread's lines: base offset and contracted-axis stride (the
        // planner sends only groups whose long-operand pieces have a single k leg)
        int64_t base[R], ks[R];
        {
            PieceWalk w;
            walk_start(w, lp, nl, x0 + min(tid, xlen - 1));
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const int32_t x = tid + 256 * q;
                base[q] = 0;
                ks[q] = 0;
                if (x < xlen) {
                    walk_to(w, x0 + x);
                    base[q] = walk_base(w, x0 + x);
                    ks[q] = w.v.sb0;
                }
            }
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
#pragma unroll 2
            for (int32_t k = 0; k < kl; ++k) {
                ACC a[R];
#pragma unroll
                for (int q = 0; q < R; ++q)
                    a[q] = tid + 256 * q < xlen ? load_acc(Pl, base[q] + static_cast<int64_t>(k0 + k) * ks[q]) : ACC(0);
#pragma unroll
                for (int q = 0; q < R; ++q)
#pragma unroll
                    for (int y = 0; y < YB; ++y) acc[q][y] = fma(a[q], sm.s[k][y], acc[q][y]);
            }
        }
    }

    // epilogue through the C pieces: C is cut either along the long axis (a
    // walk over them per thread) or along the short axis (records in LDS)
    const bool cn = (g.flags & G_C_ALONG_N) != 0;
    const bool c_long = LONG_M ? !cn : cn;
    __syncthreads();
    if (!c_long && tid < Y) sm.rc[tid] = make_rec(ka.cp + g.cp0, g.ncp, (LONG_M ? task.n0 : task.m0) + tid);
    __syncthreads();
    TC *Cp = static_cast<TC *>(ka.C);
    const bool accum = (g.flags & G_ACCUMULATE) != 0;
    PieceWalk cw;
    if (c_long) walk_start(cw, ka.cp + g.cp0, g.ncp, x0 + min(tid, xlen - 1));
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int32_t x = tid + 256 * q;
        if (x >= xlen) continue;
        int64_t cb = 0;
        if (c_long) {
            walk_to(cw, x0 + x);
            cb = walk_base(cw, x0 + x);
        }
#pragma unroll
        for (int y = 0; y < YB; ++y) {
            if (y < Y) {
                const int64_t ad = c_long ? cb + (cw.v.ib == 1 ? static_cast<int64_t>(y) * cw.v.sb0
                                                              : static_cast<int64_t>(y / cw.v.ib) * cw.v.sb0 +
                                                                    static_cast<int64_t>(y % cw.v.ib) * cw.v.sb1)
                                          : along(sm.rc[y], x0 + x);
                ACC v = acc[q][y];
                if (accum) v += static_cast<ACC>(Cp[ad]);
                Cp[ad] = static_cast<TC>(v);
            }
        }
    }
    __syncthreads();
}

// The same tile addressed through a record (one view per operand over the
// whole item, as the planner cut it): no group, run or piece lookups.
template <typename TA, typename TC, typename ACC, bool LONG_M, int YB>
__device__ __forceinline__ void skinny_dense_impl(const KArgs &ka, const DFast &fd, SkinnySmem<ACC> &sm) {
    constexpr int R = skinny_acc_budget<ACC>() / YB;
    const int32_t tid = tid_x();
    const int32_t xlen = LONG_M ? fd.mlen : fd.nlen;
    const int32_t Y = LONG_M ? fd.nlen : fd.mlen;
    const TA *A = static_cast<const TA *>((fd.flags & F_A_WS) ? ka.W : ka.A);
    const TA *B = static_cast<const TA *>((fd.flags & F_B_WS) ? ka.W : ka.B);
    const TA *Pl = LONG_M ? A : B;
    const TA *Ps = LONG_M ? B : A;
    const int64_t l_base = LONG_M ? fd.a_base : fd.b_base, l_xs = LONG_M ? fd.a_rs : fd.b_ns;
    const int64_t l_ks = LONG_M ? fd.a_ks : fd.b_ks;
    const int64_t s_base = LONG_M ? fd.b_base : fd.a_base, s_ys = LONG_M ? fd.b_ns : fd.a_rs;
    const int64_t s_ks = LONG_M ? fd.b_ks : fd.a_ks;

    ACC acc[R][YB];
#pragma unroll
    for (int q = 0; q < R; ++q)
#pragma unroll
        for (int y = 0; y < YB; ++y) acc[q][y] = ACC(0);

    for (int32_t k0 = 0; k0 < fd.K; k0 += SK_KC) {
        const int32_t kl = min(SK_KC, fd.K - k0);
        __syncthreads();   // the previous chunk (or task) is done with the LDS chunk
#pragma unroll
        for (int i = 0; i < SK_KC * SK_SHORT / 256; ++i) {
            const int32_t e = tid + 256 * i;
            const int32_t k = e / SK_SHORT, y = e % SK_SHORT;
            sm.s[k][y] = (k < kl && y < Y)
                             ? load_acc(Ps, s_base + static_cast<int64_t>(k0 + k) * s_ks + static_cast<int64_t>(y) * s_ys)
                             : ACC(0);
        }
        __syncthreads();
#pragma unroll 2
        for (int32_t k = 0; k < kl; ++k) {
            ACC a[R];
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const int32_t x = tid + 256 * q;
                a[q] = x < xlen ? load_acc(Pl, l_base + static_cast<int64_t>(x) * l_xs + static_cast<int64_t>(k0 + k) * l_ks)
                                : ACC(0);
            }
#pragma unroll
            for (int q = 0; q < R; ++q)
#pragma unroll
                for (int y = 0; y < YB; ++y) acc[q][y] = fma(a[q], sm.s[k][y], acc[q][y]);
        }
    }

    TC *Cp = static_cast<TC *>(ka.C);
    const bool accum = (fd.flags & G_ACCUMULATE) != 0;
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int32_t x = tid + 256 * q;
        if (x >= xlen) continue;
#pragma unroll
        for (int y = 0; y < YB; ++y) {
            if (y < Y) {
                const int64_t ad = LONG_M ? fd.c_base + static_cast<int64_t>(x) * fd.c_rs + static_cast<int64_t>(y) * fd.c_cs
                                          : fd.c_base + static_cast<int64_t>(y) * fd.c_rs + static_cast<int64_t>(x) * fd.c_cs;
                ACC v = acc[q][y];
                if (accum) v += static_cast<ACC>(Cp[ad]);
                Cp[ad] = static_cast<TC>(v);
            }
        }
    }
}

template <typename TA, typename TC, typename ACC, bool LONG_M>
__device__ __forceinline__ void skinny_dense(const KArgs &ka, const DFast &fd_ref, SkinnySmem<ACC> &sm) {
    const DFast fd = fd_ref;   // one read of the record
    const int32_t Y = LONG_M ? fd.nlen : fd.mlen;
    if (Y <= 4) skinny_dense_impl<TA, TC, ACC, LONG_M, 4>(ka, fd, sm);
    else if (Y <= 8) skinny_dense_impl<TA, TC, ACC, LONG_M, 8>(ka, fd, sm);
    else skinny_dense_impl<TA, TC, ACC, LONG_M, 16>(ka, fd, sm);
}

template <typename TA, typename TC, typename ACC, bool LONG_M>
__device__ __forceinline__ void skinny_tile(const KArgs &ka, const DTask &task, SkinnySmem<ACC> &sm) {
    const DGroup g = ka.groups[task.group];
    const int32_t Y = LONG_M ? g.N : g.M;
    if (Y <= 4) skinny_impl<TA, TC, ACC, LONG_M, 4>(ka, task, g, sm);
    else if (Y <= 8) skinny_impl<TA, TC, ACC, LONG_M, 8>(ka, task, g, sm);
    else skinny_impl<TA, TC, ACC, LONG_M, 16>(ka, task, g, sm);
}

}  // namespace bsc
