// Matrix-core tile for fp32 and fp64 operands (gfx950).
//
// A 256-thread workgroup (4 waves) computes a 64 x 64 output tile of one
// coalesced group GEMM.  Wave w owns the 32 x 32 quadrant (w & 1, w >> 1) as
// 2 x 2 tiles of v_mfma_f32_16x16x4_f32 (fp32) or v_mfma_f64_16x16x4_f64
// (fp64), accumulating in the operand type.
//
// Operands are staged through LDS in chunks of KC contracted indices (32 fp32 /
// 16 fp64 values, 8 KB per operand) with two buffers: the global loads of chunk
// c+1 are in flight while chunk c feeds the matrix cores.  In LDS both operands
// are stored k-major, [k][x] with x the free index of the tile, so one MFMA
// fragment (16 consecutive x for each of 4 k) is a single read per lane.  The
// x position is XOR-swizzled by k, which keeps both the fragment reads and the
// transposing stores of k-contiguous rows on distinct banks.
//
// Global loads follow the operand's memory order:
//   k-contiguous rows        -> 16-byte loads along k, transposed while storing;
//   free-axis-contiguous rows -> 16-byte loads along x, stored as they are;
//   anything else            -> element loads through the per-row records.
#pragma once

#include "kernels_common.h"

namespace bsc {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef double f64x4_t __attribute__((ext_vector_type(4)));
typedef int v4i32_mf __attribute__((ext_vector_type(4)));

constexpr int MF_TILE = 64;

template <typename T>
struct MfTraits;
template <>
struct MfTraits<float> {
    static constexpr int KC = 32;   // contracted indices per LDS chunk
    typedef f32x4_t acc_t;
};
template <>
struct MfTraits<double> {
    static constexpr int KC = 16;
    typedef f64x4_t acc_t;
};

// LDS element index of (k, x) inside one operand chunk: 64 values per k, x
// swizzled by bits of k (the swizzle only flips bits 3..5 of x, so 16-byte
// groups of consecutive x stay contiguous and aligned).
__device__ __forceinline__ int32_t mf_idx(int32_t k, int32_t x) {
    return k * MF_TILE + (x ^ ((16 * (k & 3)) ^ (8 * ((k >> 2) & 7))));
}

template <typename T>
struct MfmaSmemF {
    T a[2][MfTraits<T>::KC * MF_TILE];
    T b[2][MfTraits<T>::KC * MF_TILE];
    Rec ra[MF_TILE];
    Rec rb[MF_TILE];
};

enum : int32_t { MF_KCONTIG = 0, MF_FCONTIG = 1, MF_GENERIC = 2 };

template <typename T>
struct MfCtx {
    int32_t mode;
    int32_t x0, xlen;     // tile origin along the free axis (group coordinates) and valid extent
    int32_t K;            // run length
    int32_t vec;          // base pointer 16-byte aligned
    const T *P;
    int64_t off, sk;      // MF_FCONTIG: element (x, k) at off + x + k * sk, x in group coordinates
    const Rec *rec;       // per-row records (MF_KCONTIG, MF_GENERIC)
};

// registers carrying one chunk of one operand from global memory to LDS
template <typename T>
struct MfStage {
    T v[2][16 / sizeof(T)];
};

template <typename T>
__device__ __forceinline__ MfCtx<T> mf_ctx(const DView *pieces, int32_t np, int32_t flags_k, int32_t flags_f,
                                           int32_t run_flags, int32_t x0, int32_t xlen, int32_t K, const T *P,
                                           int32_t vec, const Rec *rec) {
    MfCtx<T> o;
    o.x0 = x0;
    o.xlen = xlen;
    o.K = K;
    o.vec = vec;
    o.P = P;
    o.rec = rec;
    o.off = 0;
    o.sk = 0;
    if (run_flags & flags_k) {
        o.mode = MF_KCONTIG;
    } else if ((run_flags & flags_f) && np == 1 && pieces[0].ib == 1) {
        o.mode = MF_FCONTIG;
        o.off = pieces[0].off - pieces[0].begin;
        o.sk = pieces[0].sb0;
    } else {
        o.mode = MF_GENERIC;
    }
    return o;
}

// global -> registers for chunk k0 (the element-wise mode loads in mf_store)
template <typename T>
__device__ __forceinline__ void mf_load(const MfCtx<T> &o, int32_t k0, MfStage<T> &st) {
    constexpr int V = 16 / sizeof(T);
    const int32_t tid = tid_x();
    if (o.mode == MF_KCONTIG) {
        // 8 lanes cover one row's KC values; 32 rows per pass, two passes
        const int32_t kx = tid & 7, xr = tid >> 3;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int32_t x = xr + 32 * q, k = k0 + V * kx;
#pragma unroll
            for (int i = 0; i < V; ++i) st.v[q][i] = T(0);
            if (x < o.xlen && k < o.K) {
                const int64_t ad = o.rec[x].base + k;
                if (o.vec && k + V <= o.K && (ad & (V - 1)) == 0) {
                    const uint4 u = *reinterpret_cast<const uint4 *>(o.P + ad);
                    __builtin_memcpy(st.v[q], &u, 16);
                } else {
#pragma unroll
                    for (int i = 0; i < V; ++i)
                        if (k + i < o.K) st.v[q][i] = o.P[ad + i];
                }
            }
        }
    } else if (o.mode == MF_FCONTIG) {
        // 64 / V lanes cover one k row of the tile; two passes cover KC rows
        constexpr int LPR = MF_TILE / V;
        constexpr int RPP = 256 / LPR;
        const int32_t x = V * (tid % LPR), kr = tid / LPR;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int32_t k = k0 + kr + RPP * q;
#pragma unroll
            for (int i = 0; i < V; ++i) st.v[q][i] = T(0);
            if (k < o.K && x < o.xlen) {
                const int64_t ad = o.off + static_cast<int64_t>(o.x0 + x) + static_cast<int64_t>(k) * o.sk;
                if (o.vec && x + V <= o.xlen && (ad & (V - 1)) == 0) {
                    const uint4 u = *reinterpret_cast<const uint4 *>(o.P + ad);
                    __builtin_memcpy(st.v[q], &u, 16);
                } else {
#pragma unroll
                    for (int i = 0; i < V; ++i)
                        if (x + i < o.xlen) st.v[q][i] = o.P[ad + i];
                }
            }
        }
    }
}

// registers (or, element-wise, global memory) -> LDS chunk
template <typename T>
__device__ __forceinline__ void mf_store(const MfCtx<T> &o, const MfStage<T> &st, T *lds, int32_t k0) {
    constexpr int V = 16 / sizeof(T);
    constexpr int KC = MfTraits<T>::KC;
    const int32_t tid = tid_x();
    if (o.mode == MF_KCONTIG) {
        const int32_t kx = tid & 7, xr = tid >> 3;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < V; ++i) lds[mf_idx(V * kx + i, xr + 32 * q)] = st.v[q][i];
    } else if (o.mode == MF_FCONTIG) {
        constexpr int LPR = MF_TILE / V;
        constexpr int RPP = 256 / LPR;
        const int32_t x = V * (tid % LPR), kr = tid / LPR;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uint4 u;
            __builtin_memcpy(&u, st.v[q], 16);
            *reinterpret_cast<uint4 *>(lds + mf_idx(kr + RPP * q, x)) = u;
        }
    } else {
        const int32_t x = tid & 63, kk = tid >> 6;
        const bool row_ok = x < o.xlen;
#pragma unroll 4
        for (int j = 0; j < KC / 4; ++j) {
            const int32_t k = kk + 4 * j;
            lds[mf_idx(k, x)] = (row_ok && k0 + k < o.K) ? o.P[along(o.rec[x], k0 + k)] : T(0);
        }
    }
}

__device__ __forceinline__ f32x4_t mf_mma(float a, float b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f64x4_t mf_mma(double a, double b, f64x4_t c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// One chunk through the matrix cores.  MFMA step s covers chunk indices
// 4s..4s+3; lane l supplies index 4s + (l >> 4) at free position l & 15.
template <typename T>
__device__ __forceinline__ void mf_compute(const T *la, const T *lb, typename MfTraits<T>::acc_t (&acc)[2][2]) {
    constexpr int KC = MfTraits<T>::KC;
    const int32_t lane = tid_x() & 63, w = tid_x() >> 6;
    const int32_t wm = w & 1, wn = w >> 1;
    const int32_t j = lane >> 4, xi = lane & 15;
#pragma unroll
    for (int s = 0; s < KC / 4; ++s) {
        const int32_t k = 4 * s + j;
        T fa[2], fb[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            fa[f] = la[mf_idx(k, wm * 32 + f * 16 + xi)];
            fb[f] = lb[mf_idx(k, wn * 32 + f * 16 + xi)];
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) acc[i][jj] = mf_mma(fa[i], fb[jj], acc[i][jj]);
    }
}

// tile row of accumulator element r of lane `lane` in a 16 x 16 MFMA tile
__device__ __forceinline__ int32_t mf_row(float, int32_t lane, int32_t r) { return (lane >> 4) * 4 + r; }
__device__ __forceinline__ int32_t mf_row(double, int32_t lane, int32_t r) { return (lane >> 4) + 4 * r; }

// The K loop of one operand pair over K contracted indices.  Chunk c + 2 is
// loaded into registers while chunk c runs on the matrix cores and chunk c + 1
// (loaded one iteration earlier) waits in registers to be stored: two chunks of
// global loads are always in flight, against the ~1 us latency of a miss.
template <typename T>
__device__ __forceinline__ void mf_kloop(const MfCtx<T> &oa, const MfCtx<T> &ob, int32_t K, MfmaSmemF<T> &sm,
                                         typename MfTraits<T>::acc_t (&acc)[2][2]) {
    constexpr int KC = MfTraits<T>::KC;
    const int32_t nchunks = (K + KC - 1) / KC;
    MfStage<T> sa, sb, na, nb;
    mf_load(oa, 0, sa);
    mf_load(ob, 0, sb);
    if (nchunks > 1) {
        mf_load(oa, KC, na);
        mf_load(ob, KC, nb);
    }
    mf_store(oa, sa, sm.a[0], 0);
    mf_store(ob, sb, sm.b[0], 0);
    __syncthreads();
    for (int32_t c = 0; c < nchunks; ++c) {
        // registers: na/nb hold chunk c + 1; chunk c + 2 goes into sa/sb
        if (c + 2 < nchunks) {
            mf_load(oa, (c + 2) * KC, sa);
            mf_load(ob, (c + 2) * KC, sb);
        }
        mf_compute<T>(sm.a[c & 1], sm.b[c & 1], acc);
        if (c + 1 < nchunks) {
            mf_store(oa, na, sm.a[(c + 1) & 1], (c + 1) * KC);
            mf_store(ob, nb, sm.b[(c + 1) & 1], (c + 1) * KC);
        }
        __syncthreads();
        na = sa;
        nb = sb;
    }
}

// ---- branch-free K loop for k-contiguous and free-contiguous operands -----------------
//
// The general loop above serves every operand layout with per-lane conditional
// loads; the compiler then cannot count the loads in flight and waits for all
// of them before every LDS store, so each chunk pays a full memory latency.
// When both operands are k-contiguous rows or free-axis-contiguous lines (the
// common case), this loop issues a fixed number of 16-byte buffer loads per
// chunk and lane, unconditionally: addresses of rows or columns past the tile
// edge are clamped to a valid one and indices k >= K are masked to zero after
// the load, and the buffer descriptor (the whole operand buffer) bounds every
// load in hardware (the whole offset travels in the lane offset, which the
// range check covers; a load past the end returns zeros and touches no
// memory).  Two chunks stay in flight with exact wait counts.
constexpr int32_t MF_BUF_DWORD3 = 0x00020000;   // raw 32-bit buffer (gfx9 descriptor word 3)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mf_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t ua = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(a >> 32))) << 32) |
                        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(a)));
    const int32_t n = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(bytes));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ua), 0, n, MF_BUF_DWORD3);
}

// One operand of the branch-free loop: per pass, the lane's byte offset at
// k = 0 and which of its V elements lie inside the tile along the free axis.
template <typename T, int MODE>
struct MfOp2 {
    __amdgpu_buffer_rsrc_t rs;
    int32_t off[2];
    int32_t kstep;       // bytes per chunk
    uint32_t xok[2];     // bit i: element i of pass q is inside the tile (free axis)
    int32_t kbase[2];    // k of element 0 of pass q within a chunk (MF_KCONTIG), or the row (MF_FCONTIG)
};

template <typename T, int MODE>
__device__ __forceinline__ MfOp2<T, MODE> mf_setup2(const MfCtx<T> &o, int64_t bytes) {
    constexpr int V = 16 / sizeof(T);
    constexpr int KC = MfTraits<T>::KC;
    MfOp2<T, MODE> f;
    f.rs = mf_rsrc(o.P, bytes);
    const int32_t tid = tid_x();
    static_assert(MODE == MF_KCONTIG || MODE == MF_FCONTIG, "contiguous modes only");
    if constexpr (MODE == MF_KCONTIG) {
        const int32_t kx = tid & 7, xr = tid >> 3;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int32_t x = xr + 32 * q;
            const int32_t xc = x < o.xlen ? x : 0;           // rows past the edge: a valid row
            f.off[q] = static_cast<int32_t>((o.rec[xc].base + V * kx) * static_cast<int64_t>(sizeof(T)));
            f.xok[q] = x < o.xlen ? 0xffu : 0u;
            f.kbase[q] = V * kx;
        }
        f.kstep = KC * static_cast<int32_t>(sizeof(T));
    } else {
        constexpr int LPR = MF_TILE / V, RPP = 256 / LPR;
        const int32_t x = V * (tid % LPR), kr = tid / LPR;
        const int32_t xc = x < o.xlen ? x : 0;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            f.off[q] = static_cast<int32_t>((o.off + o.x0 + xc + static_cast<int64_t>(kr + RPP * q) * o.sk) *
                                            static_cast<int64_t>(sizeof(T)));
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < V; ++i) m |= (x + i < o.xlen ? 1u : 0u) << i;
            f.xok[q] = m;
            f.kbase[q] = kr + RPP * q;
        }
        f.kstep = static_cast<int32_t>(KC * o.sk * static_cast<int64_t>(sizeof(T)));
    }
    return f;
}

// a lane's range must be addressable with 32-bit offsets from the buffer base
template <typename T>
__device__ __forceinline__ bool mf_fits2(int64_t bytes) { return bytes > 0 && bytes < (int64_t(1) << 31); }

// raw 16-byte loads of one chunk (masked later, when stored: using the loaded
// registers here would wait for the loads)
struct MfRaw {
    v4i32_mf v[2];
};

template <typename T, int MODE>
__device__ __forceinline__ void mf_load2(const MfOp2<T, MODE> &f, int32_t k0, MfRaw &st) {
    // The chunk advance goes into the lane offset, not the scalar offset: the
    // hardware range check of a raw buffer covers the lane offset only, and the
    // last chunk may reach past the end of the operand buffer.
    const uint32_t adv = static_cast<uint32_t>(k0 / MfTraits<T>::KC) * static_cast<uint32_t>(f.kstep);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        __amdgpu_buffer_rsrc_t rs = f.rs;
        st.v[q] = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int32_t>(static_cast<uint32_t>(f.off[q]) + adv),
                                                        0, 0);
    }
}

// registers -> LDS chunk (starting at k0) for a layout known at compile time:
// elements outside the tile or at k >= K become zeros
template <typename T, int MODE>
__device__ __forceinline__ void mf_store2(const MfOp2<T, MODE> &f, const MfRaw &raw, T *lds, int32_t k0, int32_t K) {
    constexpr int V = 16 / sizeof(T);
    const int32_t tid = tid_x();
    T e[2][V];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        __builtin_memcpy(e[q], &raw.v[q], 16);
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int32_t k = MODE == MF_KCONTIG ? k0 + f.kbase[q] + i : k0 + f.kbase[q];
            const bool ok = ((f.xok[q] >> i) & 1u) && k < K;
            e[q][i] = ok ? e[q][i] : T(0);
        }
    }
    if constexpr (MODE == MF_KCONTIG) {
        const int32_t kx = tid & 7, xr = tid >> 3;
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < V; ++i) lds[mf_idx(V * kx + i, xr + 32 * q)] = e[q][i];
    } else {
        constexpr int LPR = MF_TILE / V, RPP = 256 / LPR;
        const int32_t x = V * (tid % LPR), kr = tid / LPR;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            uint4 u;
            __builtin_memcpy(&u, e[q], 16);
            *reinterpret_cast<uint4 *>(lds + mf_idx(kr + RPP * q, x)) = u;
        }
    }
}

template <typename T, int MA, int MB>
__device__ __forceinline__ void mf_kloop2(const MfOp2<T, MA> &fa, const MfOp2<T, MB> &fb, int32_t K, MfmaSmemF<T> &sm,
                                          typename MfTraits<T>::acc_t (&acc)[2][2]) {
    constexpr int KC = MfTraits<T>::KC;
    const int32_t nchunks = (K + KC - 1) / KC;
    const int32_t last = (nchunks - 1) * KC;
    MfRaw a0, b0, a1, b1;
    // loads are unconditional: a chunk index past the end repeats the last chunk
    mf_load2<T, MA>(fa, 0, a0);
    mf_load2<T, MB>(fb, 0, b0);
    mf_load2<T, MA>(fa, min(KC, last), a1);
    mf_load2<T, MB>(fb, min(KC, last), b1);
    mf_store2<T, MA>(fa, a0, sm.a[0], 0, K);
    mf_store2<T, MB>(fb, b0, sm.b[0], 0, K);
    __syncthreads();
    // Unrolled by two so the register sets swap roles without copies (a copy
    // of the set just loaded would wait for its loads): in step (c, X, Y), X
    // holds chunk c + 1 and chunk c + 2 is loaded into Y.
    auto step = [&](int32_t c, MfRaw &xa, MfRaw &xb, MfRaw &ya, MfRaw &yb) {
        const int32_t k2 = min((c + 2) * KC, last);
        mf_load2<T, MA>(fa, k2, ya);
        mf_load2<T, MB>(fb, k2, yb);
        mf_compute<T>(sm.a[c & 1], sm.b[c & 1], acc);
        // (after the last chunk this stores zeros or a repeat into the idle buffer)
        mf_store2<T, MA>(fa, xa, sm.a[(c + 1) & 1], (c + 1) * KC, K);
        mf_store2<T, MB>(fb, xb, sm.b[(c + 1) & 1], (c + 1) * KC, K);
        __syncthreads();
    };
    int32_t c = 0;
    for (; c + 1 < nchunks; c += 2) {
        step(c, a1, b1, a0, b0);
        step(c + 1, a0, b0, a1, b1);
    }
    if (c < nchunks) step(c, a1, b1, a0, b0);
}

// Run the K loop of one operand pair: the branch-free loop when both operands
// are k- or free-contiguous and addressable with 32-bit offsets, else the
// general one.
template <typename T, int MA>
__device__ __forceinline__ void mf_kloop_b(const MfCtx<T> &oa, const MfCtx<T> &ob, int64_t a_bytes, int64_t b_bytes,
                                           int32_t K, MfmaSmemF<T> &sm, typename MfTraits<T>::acc_t (&acc)[2][2]) {
    const MfOp2<T, MA> fa = mf_setup2<T, MA>(oa, a_bytes);
    if (ob.mode == MF_KCONTIG) mf_kloop2<T, MA, MF_KCONTIG>(fa, mf_setup2<T, MF_KCONTIG>(ob, b_bytes), K, sm, acc);
    else mf_kloop2<T, MA, MF_FCONTIG>(fa, mf_setup2<T, MF_FCONTIG>(ob, b_bytes), K, sm, acc);
}

template <typename T>
__device__ __forceinline__ void mf_kloop_any(const MfCtx<T> &oa, const MfCtx<T> &ob, int64_t a_bytes, int64_t b_bytes,
                                             int32_t K, MfmaSmemF<T> &sm, typename MfTraits<T>::acc_t (&acc)[2][2]) {
    // element offsets of the record mode are 32-bit too
    // (the record mode through this loop measured slower than the general loop
    // on the environment-update stages: per-element address arithmetic and
    // register pressure outweigh the better overlap)
    const bool fits = mf_fits2<T>(a_bytes) && mf_fits2<T>(b_bytes);
    if (fits && oa.mode != MF_GENERIC && ob.mode != MF_GENERIC) {
        if (oa.mode == MF_KCONTIG) mf_kloop_b<T, MF_KCONTIG>(oa, ob, a_bytes, b_bytes, K, sm, acc);
        else mf_kloop_b<T, MF_FCONTIG>(oa, ob, a_bytes, b_bytes, K, sm, acc);
        return;
    }
    mf_kloop<T>(oa, ob, K, sm, acc);   // record-mode operands, or operands beyond 2 GiB
}

template <typename T>
__device__ __forceinline__ void mfma_tile_f(const KArgs &ka, const DTask &task, const DFast &fd_ref, MfmaSmemF<T> &sm) {
    typedef typename MfTraits<T>::acc_t acc_t;
    const int32_t tid = tid_x();
    const bool dense = task.cls == T_MFMA_DENSE;
    // dense tiles carry their own record: no group, run or piece lookups
    DGroup g;
    DFast fd;
    int32_t m0, n0, mlen, nlen;
    if (dense) {
        fd = fd_ref;
        m0 = 0;
        n0 = 0;
        mlen = fd.mlen;
        nlen = fd.nlen;
    } else {
        g = ka.groups[task.group];
        m0 = task.m0;
        n0 = task.n0;
        mlen = min(MF_TILE, g.M - m0);
        nlen = min(MF_TILE, g.N - n0);
    }

    acc_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = T(0);

    if (dense) {
        __syncthreads();
        if (tid < MF_TILE) {
            sm.ra[tid] = Rec{fd.a_base + static_cast<int64_t>(tid) * fd.a_rs, fd.a_ks, 0, 1, 0};
        } else if (tid < 2 * MF_TILE) {
            const int32_t j = tid - MF_TILE;
            sm.rb[j] = Rec{fd.b_base + static_cast<int64_t>(j) * fd.b_ns, fd.b_ks, 0, 1, 0};
        }
        __syncthreads();
        // element loads by mode: k-contiguous rows, free-axis-contiguous lines, or per-row records
        const T *A = static_cast<const T *>((fd.flags & F_A_WS) ? ka.W : ka.A);
        const T *B = static_cast<const T *>((fd.flags & F_B_WS) ? ka.W : ka.B);
        MfCtx<T> oa, ob;
        oa.x0 = 0; oa.xlen = mlen; oa.K = fd.K; oa.vec = (fd.flags & F_A_WS) ? 1 : ka.vec_a; oa.P = A; oa.rec = sm.ra;
        ob.x0 = 0; ob.xlen = nlen; ob.K = fd.K; ob.vec = (fd.flags & F_B_WS) ? 1 : ka.vec_b; ob.P = B; ob.rec = sm.rb;
        oa.mode = (fd.a_ks == 1 || fd.K == 1) ? MF_KCONTIG : (fd.a_rs == 1 ? MF_FCONTIG : MF_GENERIC);
        ob.mode = (fd.b_ks == 1 || fd.K == 1) ? MF_KCONTIG : (fd.b_ns == 1 ? MF_FCONTIG : MF_GENERIC);
        oa.off = fd.a_base; oa.sk = fd.a_ks;
        ob.off = fd.b_base; ob.sk = fd.b_ks;
        mf_kloop_any<T>(oa, ob, (fd.flags & F_A_WS) ? ka.w_bytes : ka.a_bytes, (fd.flags & F_B_WS) ? ka.w_bytes : ka.b_bytes,
                        fd.K, sm, acc);
    } else {
        for (int32_t r = 0; r < g.nrun; ++r) {
            const DRun run = ka.runs[g.run0 + r];
            __syncthreads();
            if (tid < MF_TILE) {
                if (tid < mlen) sm.ra[tid] = make_rec(ka.ap + run.ap0, run.nap, m0 + tid);
            } else if (tid < 2 * MF_TILE) {
                const int32_t j = tid - MF_TILE;
                if (j < nlen) sm.rb[j] = make_rec(ka.bp + run.bp0, run.nbp, n0 + j);
            }
            __syncthreads();
            const int32_t va = (run.flags & R_A_WS) ? 1 : ka.vec_a, vb = (run.flags & R_B_WS) ? 1 : ka.vec_b;
            const MfCtx<T> oa = mf_ctx<T>(ka.ap + run.ap0, run.nap, R_A_KUNIT, R_A_FUNIT, run.flags, m0, mlen, run.K,
                                          run_a<T>(ka, run.flags), va, sm.ra);
            const MfCtx<T> ob = mf_ctx<T>(ka.bp + run.bp0, run.nbp, R_B_KUNIT, R_B_FUNIT, run.flags, n0, nlen, run.K,
                                          run_b<T>(ka, run.flags), vb, sm.rb);
            mf_kloop_any<T>(oa, ob, (run.flags & R_A_WS) ? ka.w_bytes : ka.a_bytes,
                            (run.flags & R_B_WS) ? ka.w_bytes : ka.b_bytes, run.K, sm, acc);
        }
    }

    // epilogue: straight from the accumulators through the C pieces (or the
    // record); the 16 lanes of a row write 16 consecutive columns
    const bool cn = !dense && (g.flags & G_C_ALONG_N) != 0;
    if (!dense) {
        if (tid < MF_TILE) {
            if (!cn && tid < mlen) sm.ra[tid] = make_rec(ka.cp + g.cp0, g.ncp, m0 + tid);
            if (cn && tid < nlen) sm.ra[tid] = make_rec(ka.cp + g.cp0, g.ncp, n0 + tid);
        }
        __syncthreads();
    }
    T *Cp = static_cast<T *>(ka.C);
    const bool accum = ((dense ? fd.flags : g.flags) & G_ACCUMULATE) != 0;
    const int32_t lane = tid & 63, w = tid >> 6;
    const int32_t wm = w & 1, wn = w >> 1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int32_t col = wn * 32 + j * 16 + (lane & 15);
            if (col >= nlen) continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int32_t row = wm * 32 + i * 16 + mf_row(T(0), lane, r);
                if (row >= mlen) continue;
                const int64_t ad = dense ? fd.c_base + static_cast<int64_t>(row) * fd.c_rs + static_cast<int64_t>(col) * fd.c_cs
                                         : (cn ? along(sm.ra[col], m0 + row) : along(sm.ra[row], n0 + col));
                T v = acc[i][j][r];
                if (accum) v += Cp[ad];
                Cp[ad] = v;
            }
        }
    __syncthreads();
}

}  // namespace bsc
