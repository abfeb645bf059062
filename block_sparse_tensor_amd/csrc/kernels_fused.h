// The fused two-stage kernel (fused_internal.h).  Every wave owns one part of
// one task (a task: a 16 x 16 tile of one group and up to NO of the group's
// outputs; its part: every S-th stage-1 block of the group).
//
//  * The wave reads its part record (one 128-byte scalar load), which holds
//    the part's first product, and issues that product's first operand loads
//    at once.  It then loads, one entry per lane, the records of the part's
//    first 64 products, the task's weights W[widx] (stage-1 block x output)
//    and the output views; entries are taken from these lanes by readlane
//    when needed, so the product stream waits on no further scalar load.
//  * Products are walked in order through a ring of D register chunks of
//    FUSED_KC contracted indices: while one chunk runs on the matrix cores
//    (v_mfma_f64_16x16x4_f64 / v_mfma_f32_16x16x4_f32), the next D - 1 are in
//    flight (D = 2 for fp64; for fp32 D = 1, the refill issued after each
//    chunk, and the latency hidden by the other waves: the smaller ring
//    leaves room for five waves per SIMD, which measured faster than four
//    waves with four or two chunks each).  Lane l supplies A_p(i0 + (l & 15), k) and B_p(k, j0 + (l & 15))
//    for k = k0 + 4 s + (l >> 4), read through raw buffer descriptors over the
//    product's operand blocks (consecutive lanes read consecutive rows of A_p
//    and columns of B_p, the operands' contiguous axes in the environment
//    update); a masked element (outside the tile or past K) reads as zero.
//  * After the last product of a stage-1 block, its tile (four values per
//    lane) is added, weighted by the block's W entries, into the accumulators
//    of the task's outputs.
//  * The parts of a task share a workgroup: the part-0 wave adds the other
//    parts' accumulators (through shared memory, in part order) and writes
//    (or accumulates) the outputs through their M x N views.  A
//    group whose outputs run down their rows forms its tiles transposed
//    (operands swapped in the matrix-core call), so that consecutive lanes
//    write consecutive addresses.
//
// The stage-1 blocks never leave the registers, and every output element has
// one owner and a fixed summation order, so repeats are bit-identical.
#pragma once

#include <hip/hip_runtime.h>

#include "fused_internal.h"
#include "kernels_common.h"

namespace bsc {

struct FArgs {
    const FChan *pchans;            // the parts' product lists
    const FOut *outs;
    const int32_t *widx;
    const FPart *parts;             // four per workgroup (one per wave)
    int32_t nwg, no;
    const void *A, *B, *W;
    void *C;
};

typedef float fu_f32x4 __attribute__((ext_vector_type(4)));
typedef double fu_f64x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct FuTraits;
template <>
struct FuTraits<float> {
    typedef fu_f32x4 acc_t;
    static constexpr int D = 1;     // register chunks in the ring
    // tile row of accumulator element v of lane l (column l & 15)
    static __device__ __forceinline__ int32_t row(int32_t l, int32_t v) { return (l >> 4) * 4 + v; }
    static __device__ __forceinline__ acc_t mma(float a, float b, acc_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
};
template <>
struct FuTraits<double> {
    typedef fu_f64x4 acc_t;
    static constexpr int D = 2;
    static __device__ __forceinline__ int32_t row(int32_t l, int32_t v) { return (l >> 4) + 4 * v; }
    static __device__ __forceinline__ acc_t mma(double a, double b, acc_t c) {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
};

constexpr int FUSED_STEPS = FUSED_KC / 4;   // matrix-core steps per chunk

// one chunk of a product's operands in registers: for each of the wave's TW
// row blocks of A and column blocks of B, one value per step
template <typename T, int TW>
struct FuChunk {
    T a[TW][FUSED_STEPS], b[TW][FUSED_STEPS];
};

// A product's operands as raw buffers: each block's range in scalar registers
// (the planner keeps every block range below 2 GiB), one 32-bit lane offset
// per operand, and the bytes per contracted index.  A masked element reads
// through an offset beyond the range, for which the hardware returns zero.
constexpr uint32_t FU_OOB = 0x80000000u;
constexpr int32_t FU_RAW = 0x00020000;   // raw 32-bit buffer (gfx9 descriptor word 3)

struct FuProd {
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t la, lb;        // lane byte offsets at k = 0 (row x of A, column x of B)
    uint32_t a16, b16;      // bytes from one 16-row (16-column) block of the tile to the next
    uint32_t ka, kb;        // bytes per contracted index
    int32_t K, wrow, last;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t fu_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t ua = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(a >> 32))) << 32) |
                        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(a)));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ua), 0,
                                             __builtin_amdgcn_readfirstlane(static_cast<int32_t>(bytes)), FU_RAW);
}

template <typename T>
__device__ __forceinline__ FuProd fu_prod(const T *A, const T *B, const FChan &ch, int32_t M, int32_t N, int32_t i,
                                          int32_t j) {
    constexpr int64_t SZ = sizeof(T);
    FuProd P;
    P.ra = fu_rsrc(A + ch.a_off, ((M - 1) * ch.a_rs + (ch.K - 1) * ch.a_ks + 1) * SZ);
    P.rb = fu_rsrc(B + ch.b_off, ((ch.K - 1) * ch.b_ks + (N - 1) * ch.b_ns + 1) * SZ);
    P.la = static_cast<uint32_t>(i * ch.a_rs * SZ);
    P.lb = static_cast<uint32_t>(j * ch.b_ns * SZ);
    P.a16 = static_cast<uint32_t>(FUSED_TILE * ch.a_rs * SZ);
    P.b16 = static_cast<uint32_t>(FUSED_TILE * ch.b_ns * SZ);
    P.ka = static_cast<uint32_t>(ch.a_ks * SZ);
    P.kb = static_cast<uint32_t>(ch.b_ks * SZ);
    P.K = ch.K;
    P.wrow = ch.wrow;
    P.last = ch.last;
    return P;
}

__device__ __forceinline__ float fu_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, float) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ double fu_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, double) {
    return __builtin_bit_cast(double, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// chunk k0 of a product: lane (x, q) takes k = k0 + 4 s + q, s < FUSED_STEPS,
// for rows x + 16 i of A and columns x + 16 i of B (i < TW).  The offsets of
// the masked elements (outside the tile, past K) are replaced, never formed
// by adding to another (so they cannot wrap into the range).
template <typename T, int TW>
__device__ __forceinline__ void fu_load(const FuProd &P, int32_t k0, const bool (&arow)[TW], const bool (&bcol)[TW],
                                        int32_t q, FuChunk<T, TW> &v) {
#pragma unroll
    for (int s = 0; s < FUSED_STEPS; ++s) {
        const int32_t k = k0 + 4 * s + q;
        const bool ok = k < P.K;
        const uint32_t uk = static_cast<uint32_t>(k);
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            v.a[i][s] = fu_buf(P.ra, (arow[i] && ok) ? P.la + i * P.a16 + uk * P.ka : FU_OOB, T(0));
            v.b[i][s] = fu_buf(P.rb, (bcol[i] && ok) ? P.lb + i * P.b16 + uk * P.kb : FU_OOB, T(0));
        }
    }
}

// readlane of a lane-held value (lane index uniform)
__device__ __forceinline__ int32_t fu_rl(int32_t v, int32_t l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ int64_t fu_rl(int64_t v, int32_t l) {
    const uint32_t lo = static_cast<uint32_t>(fu_rl(static_cast<int32_t>(v), l));
    const uint32_t hi = static_cast<uint32_t>(fu_rl(static_cast<int32_t>(v >> 32), l));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ float fu_rl(float v, int32_t l) {
    return __builtin_bit_cast(float, fu_rl(__builtin_bit_cast(int32_t, v), l));
}
__device__ __forceinline__ double fu_rl(double v, int32_t l) {
    return __builtin_bit_cast(double, fu_rl(__builtin_bit_cast(int64_t, v), l));
}

__device__ __forceinline__ FChan fu_rl(const FChan &c, int32_t l) {
    FChan r;
    r.a_off = fu_rl(c.a_off, l);
    r.a_rs = fu_rl(c.a_rs, l);
    r.a_ks = fu_rl(c.a_ks, l);
    r.b_off = fu_rl(c.b_off, l);
    r.b_ks = fu_rl(c.b_ks, l);
    r.b_ns = fu_rl(c.b_ns, l);
    r.K = fu_rl(c.K, l);
    const int32_t wl =
        fu_rl(static_cast<int32_t>(static_cast<uint16_t>(c.wrow)) | (static_cast<int32_t>(c.last) << 16), l);
    r.wrow = static_cast<int16_t>(wl & 0xffff);
    r.last = static_cast<int16_t>(wl >> 16);
    return r;
}

// One ring slot: the chunk and what the compute step needs to know about it.
template <typename T, int TW>
struct FuSlot {
    FuChunk<T, TW> v;
    int32_t p;              // product index, -1: empty (the stream has ended)
    int32_t k0, K, wrow, last;
};

// One part's product stream (record pr) through the matrix cores, weighted
// into acc.  The loop body is branch-free where the loads are: every slot
// refill issues the same loads (offsets beyond the range once the stream has
// ended, which read zero) and every chunk runs all its matrix-core steps
// (zeros past K add nothing), so the compiler's wait counts stay exact:
// computing a slot waits for that slot's loads only, never for the D - 1
// chunks behind it.
template <typename T, int NO, int TW>
__device__ __forceinline__ void fused_stream(const FArgs &fa, const FPart &pr, int32_t lane,
                                             typename FuTraits<T>::acc_t (&acc)[NO][TW][TW]) {
    typedef typename FuTraits<T>::acc_t acc_t;
    constexpr int D = TW == 1 ? FuTraits<T>::D : 2;   // chunks in the ring (registers: TW^2 more per chunk)
    const T *A = static_cast<const T *>(fa.A);
    const T *B = static_cast<const T *>(fa.B);
    const T *W = static_cast<const T *>(fa.W);
    const bool tr = (pr.flags & G_FTRANS) != 0;
    const int32_t x = lane & 15, q = lane >> 4;
    bool arow[TW], bcol[TW];
#pragma unroll
    for (int i = 0; i < TW; ++i) {
        arow[i] = x + FUSED_TILE * i < pr.ml;
        bcol[i] = x + FUSED_TILE * i < pr.nl;
    }
    const int32_t ia = pr.i0 + x, jb = pr.j0 + x;   // masked where out of the tile
    const FChan *chans = fa.pchans + pr.chan0;

    FuSlot<T, TW> ring[D];
    // the issue cursor: product ip (operands P), next chunk offset ik
    int32_t ip = 0, ik = 0;
    FuProd P = fu_prod(A, B, pr.first, pr.M, pr.N, ia, jb);
    FChan myrec{};
    // the next chunk of the stream into slot sl; past the end the slot is
    // marked empty and its loads read zero
    auto issue = [&](FuSlot<T, TW> &sl) {
        if (ik >= P.K && ip < pr.nchan) {
            ++ip;
            ik = 0;
            if (ip < pr.nchan) {
                if ((ip & (FUSED_LANE_RECS - 1)) == 0) {
                    // the next batch of lane-held records (rare: parts of more than 64 products)
                    myrec = ip + lane < pr.nchan ? chans[ip + lane] : FChan{};
                    __builtin_amdgcn_s_waitcnt(0);
                }
                P = fu_prod(A, B, fu_rl(myrec, ip & (FUSED_LANE_RECS - 1)), pr.M, pr.N, ia, jb);
            }
        }
        const bool live = ip < pr.nchan;
        bool ar[TW], bc[TW];
#pragma unroll
        for (int i = 0; i < TW; ++i) {
            ar[i] = arow[i] && live;
            bc[i] = bcol[i] && live;
        }
        fu_load(P, ik, ar, bc, q, sl.v);
        sl.p = live ? ip : -1;
        sl.k0 = ik;
        sl.K = P.K;
        sl.wrow = P.wrow;
        sl.last = P.last;
        ik += FUSED_KC;
    };
    issue(ring[0]);   // the first chunk waits on the part record alone

    // product records, one per lane (the first batch of 64)
    if (lane < pr.nchan) myrec = chans[lane];
    // weights of (block r, output o) at entry r * NO + o, FUSED_WREG per lane
    // (all index loads first, then all value loads: two round trips in all)
    T wv[FUSED_WREG];
    int32_t wi[FUSED_WREG];
    const int32_t nw = pr.nblk * NO;
#pragma unroll
    for (int m = 0; m < FUSED_WREG; ++m) {
        const int32_t e = lane + 64 * m;
        const int32_t r = e / NO, o = e - r * NO;
        wi[m] = (e < nw && o < pr.no) ? fa.widx[pr.wbase + static_cast<int64_t>(r) * pr.wstride + o] : -1;
    }
#pragma unroll
    for (int m = 0; m < FUSED_WREG; ++m) wv[m] = wi[m] >= 0 ? W[wi[m]] : T(0);
    // the lane-held tables complete before the stream starts (together with the
    // first chunk, issued before them): inside the loop the compiler then knows
    // they are ready and never waits for outstanding chunk loads to read them
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int u = 1; u < D; ++u) issue(ring[u]);

    acc_t t1[TW][TW];
#pragma unroll
    for (int i = 0; i < TW; ++i)
#pragma unroll
        for (int j = 0; j < TW; ++j) t1[i][j] = acc_t{0, 0, 0, 0};
    while (true) {
#pragma unroll
        for (int u = 0; u < D; ++u) {
            FuSlot<T, TW> &sl = ring[u];
            // all steps, operands swapped for a transposed tile by selects
#pragma unroll
            for (int s = 0; s < FUSED_STEPS; ++s)
#pragma unroll
                for (int i = 0; i < TW; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) {
                        const T xa = tr ? sl.v.b[j][s] : sl.v.a[i][s];
                        const T xb = tr ? sl.v.a[i][s] : sl.v.b[j][s];
                        t1[i][j] = FuTraits<T>::mma(xa, xb, t1[i][j]);
                    }
            if (sl.p >= 0 && sl.k0 + FUSED_KC >= sl.K && sl.last) {
                // the stage-1 block is complete: weighted into every output of the task
#pragma unroll
                for (int o = 0; o < NO; ++o) {
                    if (o < pr.no) {
                        const int32_t e = sl.wrow * NO + o, m = e >> 6, l = e & 63;
                        T wgt = fu_rl(wv[0], l);
#pragma unroll
                        for (int mm = 1; mm < FUSED_WREG; ++mm)
                            if (m == mm) wgt = fu_rl(wv[mm], l);
#pragma unroll
                        for (int i = 0; i < TW; ++i)
#pragma unroll
                            for (int j = 0; j < TW; ++j)
#pragma unroll
                                for (int v = 0; v < 4; ++v) acc[o][i][j][v] = fma(wgt, t1[i][j][v], acc[o][i][j][v]);
                    }
                }
#pragma unroll
                for (int i = 0; i < TW; ++i)
#pragma unroll
                    for (int j = 0; j < TW; ++j) t1[i][j] = acc_t{0, 0, 0, 0};
            }
            issue(sl);   // refill the slot
        }
        // slots hold consecutive chunks: slot 0 empty means the stream has ended
        if (ring[0].p < 0) break;
    }
}

template <typename T, int TW>
struct FusedSmem {
    T red[4][4][4 * TW * TW][64];   // [wave][output of the pass][accumulator element][lane]
};

// Four slots per workgroup, one per wave: each wave runs its part; the parts
// of a task are then added in part order by the part-0 wave, four outputs per
// pass through shared memory, and written through the outputs' views.
template <typename T, int NO, int TW>
__global__ __launch_bounds__(256) void fused_contract(FArgs fa) {
    typedef typename FuTraits<T>::acc_t acc_t;
    __shared__ FusedSmem<T, TW> sm;
    const int32_t w = __builtin_amdgcn_readfirstlane(tid_x() >> 6);
    const int32_t lane = tid_x() & 63;
    const FPart pr = fa.parts[static_cast<int64_t>(blockIdx.x) * 4 + w];
    acc_t acc[NO][TW][TW];
#pragma unroll
    for (int o = 0; o < NO; ++o)
#pragma unroll
        for (int i = 0; i < TW; ++i)
#pragma unroll
            for (int j = 0; j < TW; ++j) acc[o][i][j] = acc_t{0, 0, 0, 0};
    // output views, one per lane (the part-0 wave writes)
    FOut myout{};
    if (pr.nparts > 0 && pr.part == 0 && lane < pr.no) myout = fa.outs[pr.out0 + lane];
    if (pr.nparts > 0 && pr.nchan > 0) fused_stream<T, NO, TW>(fa, pr, lane, acc);

    T *Cp = static_cast<T *>(fa.C);
    const bool tr = (pr.flags & G_FTRANS) != 0, accum = (pr.flags & G_ACCUMULATE) != 0;
    const int32_t x = lane & 15;
    // the part-0 wave's outputs (sum: the task's total for output o) through their views
    auto write_out = [&](int32_t o, const acc_t (&sum)[TW][TW]) {
        const int64_t c_off = fu_rl(myout.c_off, o), c_rs = fu_rl(myout.c_rs, o), c_cs = fu_rl(myout.c_cs, o);
#pragma unroll
        for (int bi = 0; bi < TW; ++bi)
#pragma unroll
            for (int bj = 0; bj < TW; ++bj)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int32_t r = FuTraits<T>::row(lane, v);
                    const int32_t i = FUSED_TILE * bi + (tr ? x : r), j = FUSED_TILE * bj + (tr ? r : x);
                    if (i < pr.ml && j < pr.nl) {
                        const int64_t ad =
                            c_off + static_cast<int64_t>(pr.i0 + i) * c_rs + static_cast<int64_t>(pr.j0 + j) * c_cs;
                        T val = sum[bi][bj][v];
                        if (accum) val += Cp[ad];
                        Cp[ad] = val;
                    }
                }
    };
    if (!pr.reduce) {
        // no task of this workgroup is split (the same for all its waves): no barriers
        if (pr.nparts > 0) {
#pragma unroll
            for (int o = 0; o < NO; ++o)
                if (o < pr.no) write_out(o, acc[o]);
        }
        return;
    }
#pragma unroll
    for (int pass = 0; pass < (NO + 3) / 4; ++pass) {
        if (pass < pr.npass) {   // the same for every wave of the workgroup: all join both barriers
            const bool reduce = pr.nparts > 1;   // the same for every wave of a task
            if (reduce && pr.part > 0) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (pass * 4 + u < NO)   // (a one-output instance has one accumulator set)
#pragma unroll
                        for (int i = 0; i < TW; ++i)
#pragma unroll
                            for (int j = 0; j < TW; ++j)
#pragma unroll
                                for (int v = 0; v < 4; ++v)
                                    sm.red[w][u][(i * TW + j) * 4 + v][lane] = acc[pass * 4 + u][i][j][v];
            }
            __syncthreads();
            if (pr.nparts > 0 && pr.part == 0) {
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int32_t o = pass * 4 + u;
                    if (pass * 4 + u < NO && o < pr.no) {
                        acc_t sum[TW][TW];
#pragma unroll
                        for (int i = 0; i < TW; ++i)
#pragma unroll
                            for (int j = 0; j < TW; ++j) sum[i][j] = acc[pass * 4 + u][i][j];
                        for (int32_t pp = 1; pp < pr.nparts; ++pp) {
#pragma unroll
                            for (int i = 0; i < TW; ++i)
#pragma unroll
                                for (int j = 0; j < TW; ++j)
#pragma unroll
                                    for (int v = 0; v < 4; ++v) sum[i][j][v] += sm.red[w + pp][u][(i * TW + j) * 4 + v][lane];
                        }
                        write_out(o, sum);
                    }
                }
            }
            __syncthreads();
        }
    }
}

}  // namespace bsc
