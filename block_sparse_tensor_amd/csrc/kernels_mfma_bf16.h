// Matrix-core tile for bf16 inputs with fp32 accumulation (gfx950).
//
// A 256-thread workgroup (4 waves) computes a 128 x 128 output tile of one
// coalesced group GEMM with v_mfma_f32_32x32x16_bf16: wave w owns the 64 x 64
// quadrant (w & 1, w >> 1) as 2 x 2 MFMA tiles.  Operand chunks of 128 x 32
// (K-contiguous in LDS, so each lane's fragment is one 16-byte LDS read) are
// double-buffered: the global loads of chunk c+1 are in flight while chunk c
// feeds the matrix cores, with one barrier per chunk.
//
// Global loads follow the operand's memory order:
//   K-contiguous rows   -> 16-byte loads along K, stored as-is;
//   free-axis-contiguous -> 16-byte loads along M (or N) for two K rows,
//                          interleaved into K-pairs while storing (transpose);
//   anything else        -> element loads through the per-row address records.
// The 16-byte loads need only element alignment: the HSA code object runs in
// unaligned-access mode, so a row that starts at an odd element still takes
// one vector load per 8 elements (rows of odd length, as sectors are stored
// when nothing pads them, made every other row fall back to 8 element loads).
// LDS rows are padded to 40 elements and skewed by 8 more every 8 rows so the
// fragment reads and the transposing stores spread over all banks.
#pragma once

#include "kernels_common.h"

namespace bsc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int MB_BM = 128;
constexpr int MB_BN = 128;
constexpr int MB_BK = 32;
constexpr int MB_TILE_ELEMS = 128 * 40 + 16 * 8;
constexpr int MB_SLAB = 132;   // fp32 row pitch of the epilogue slab (64 x 128 tile rows)

// LDS row start (in elements) of tile row x: 32 K-values + 8 padding per row,
// plus 8 more every 8 rows, so both the fragment reads (8 rows at a time) and
// the transposing stores (rows 8 apart) land in distinct banks.
__host__ __device__ constexpr int32_t mb_row(int32_t x) { return x * 40 + (x >> 3) * 8; }

constexpr bool mb_rows_disjoint() {
    for (int32_t x = 0; x + 1 < MB_BM; ++x)
        if (mb_row(x) + MB_BK > mb_row(x + 1)) return false;
    return mb_row(MB_BM - 1) + MB_BK <= MB_TILE_ELEMS && (mb_row(1) * 2) % 16 == 0 && (mb_row(8) * 2) % 16 == 0;
}
static_assert(mb_rows_disjoint(), "LDS operand rows must not overlap and must stay 16-byte aligned");

struct MfmaSmemBf16 {
    union {
        struct {
            uint16_t a[2][MB_TILE_ELEMS];   // double-buffered operand chunks, [row][k]
            uint16_t b[2][MB_TILE_ELEMS];
        } op;
        float slab[64 * MB_SLAB];           // epilogue staging
    } u;
    Rec ra[128];
    Rec rb[128];
};

enum : int32_t { LD_KCONTIG = 0, LD_FCONTIG = 1, LD_GENERIC = 2 };

struct OpCtx {
    int32_t mode;
    int32_t x0, xlen;     // tile origin along the free axis (group coordinates) and valid extent
    int32_t K;            // run length
    int32_t vec;          // base pointer 16-byte aligned
    const uint16_t *P;
    int64_t off, sk;      // LD_FCONTIG: element (x, k) at off + x + k * sk, x in group coordinates
    const Rec *rec;       // per-row records (LD_KCONTIG, LD_GENERIC)
};

struct MbStage {
    uint4 v[2];
};

__device__ __forceinline__ uint16_t u4_get(const uint4 &v, int i) {
    const uint32_t d = (i >> 1) == 0 ? v.x : ((i >> 1) == 1 ? v.y : ((i >> 1) == 2 ? v.z : v.w));
    return static_cast<uint16_t>((i & 1) ? (d >> 16) : (d & 0xFFFFu));
}

__device__ __forceinline__ uint4 u4_from(const uint16_t e[8]) {
    uint4 v;
    v.x = static_cast<uint32_t>(e[0]) | (static_cast<uint32_t>(e[1]) << 16);
    v.y = static_cast<uint32_t>(e[2]) | (static_cast<uint32_t>(e[3]) << 16);
    v.z = static_cast<uint32_t>(e[4]) | (static_cast<uint32_t>(e[5]) << 16);
    v.w = static_cast<uint32_t>(e[6]) | (static_cast<uint32_t>(e[7]) << 16);
    return v;
}

// 8 consecutive bf16 values from any element address (one 16-byte load)
__device__ __forceinline__ uint4 ld8_bf16(const uint16_t *p) {
    uint4 v;
    __builtin_memcpy(&v, p, sizeof(v));
    return v;
}

__device__ __forceinline__ void mb_load(const OpCtx &o, int32_t k0, MbStage &st) {
    const int32_t tid = tid_x();
    if (o.mode == LD_KCONTIG) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int32_t u = tid + 256 * q;
            const int32_t x = u >> 2, k = k0 + 8 * (u & 3);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (x < o.xlen && k < o.K) {
                const int64_t ad = o.rec[x].base + k;
                if (k + 8 <= o.K) {
                    v = ld8_bf16(o.P + ad);
                } else {
                    uint16_t e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = (k + j < o.K) ? o.P[ad + j] : uint16_t(0);
                    v = u4_from(e);
                }
            }
            st.v[q] = v;
        }
    } else if (o.mode == LD_FCONTIG) {
        const int32_t x = 8 * (tid & 15), kp = tid >> 4;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int32_t k = k0 + 2 * kp + q;
            uint4 v = make_uint4(0, 0, 0, 0);
            if (k < o.K && x < o.xlen) {
                const int64_t ad = o.off + static_cast<int64_t>(o.x0 + x) + static_cast<int64_t>(k) * o.sk;
                if (x + 8 <= o.xlen) {
                    v = ld8_bf16(o.P + ad);
                } else {
                    uint16_t e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = (x + j < o.xlen) ? o.P[ad + j] : uint16_t(0);
                    v = u4_from(e);
                }
            }
            st.v[q] = v;
        }
    }
    // LD_GENERIC loads in mb_store (element-wise slow path, no prefetch)
}

__device__ __forceinline__ void mb_store(const OpCtx &o, const MbStage &st, uint16_t *lds, int32_t k0) {
    const int32_t tid = tid_x();
    if (o.mode == LD_KCONTIG) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int32_t u = tid + 256 * q;
            *reinterpret_cast<uint4 *>(lds + mb_row(u >> 2) + 8 * (u & 3)) = st.v[q];
        }
    } else if (o.mode == LD_FCONTIG) {
        const int32_t x = 8 * (tid & 15), kp = tid >> 4;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t w = static_cast<uint32_t>(u4_get(st.v[0], i)) | (static_cast<uint32_t>(u4_get(st.v[1], i)) << 16);
            *reinterpret_cast<uint32_t *>(lds + mb_row(x + i) + 2 * kp) = w;
        }
    } else {
        const int32_t kk = tid & 31, k = k0 + kk;
#pragma unroll 2
        for (int q = 0; q < 16; ++q) {
            const int32_t x = (tid >> 5) + 8 * q;
            lds[mb_row(x) + kk] = (x < o.xlen && k < o.K) ? o.P[along(o.rec[x], k)] : uint16_t(0);
        }
    }
}

__device__ __forceinline__ void mb_compute(const uint16_t *la, const uint16_t *lb, f32x16_t (&acc)[2][2]) {
    const int32_t lane = tid_x() & 63, w = tid_x() >> 6;
    const int32_t wm = w & 1, wn = w >> 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        bf16x8_t fa[2], fb[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            fa[f] = *reinterpret_cast<const bf16x8_t *>(la + mb_row(wm * 64 + f * 32 + (lane & 31)) + ks * 16 + (lane >> 5) * 8);
            fb[f] = *reinterpret_cast<const bf16x8_t *>(lb + mb_row(wn * 64 + f * 32 + (lane & 31)) + ks * 16 + (lane >> 5) * 8);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
}

__device__ __forceinline__ OpCtx mb_ctx(const DView *pieces, int32_t np, int32_t flags_k, int32_t flags_f,
                                        int32_t run_flags, int32_t x0, int32_t xlen, int32_t K, const uint16_t *P,
                                        int32_t vec, const Rec *rec) {
    OpCtx o;
    o.x0 = x0;
    o.xlen = xlen;
    o.K = K;
    o.vec = vec;
    o.P = P;
    o.rec = rec;
    o.off = 0;
    o.sk = 0;
    if (run_flags & flags_k) {
        o.mode = LD_KCONTIG;
    } else if ((run_flags & flags_f) && np == 1 && pieces[0].ib == 1) {
        o.mode = LD_FCONTIG;
        o.off = pieces[0].off - pieces[0].begin;
        o.sk = pieces[0].sb0;
    } else {
        o.mode = LD_GENERIC;
    }
    return o;
}

template <typename TC>
__device__ __forceinline__ void mfma_tile_bf16(const KArgs &ka, const DTask &task, MfmaSmemBf16 &sm) {
    // a dense-tile task (its direct-to-LDS body not compiled into this launch) names its group through its record
    const DGroup g = ka.groups[task.cls == T_MFMA ? task.group : ka.fast[task.group].group];
    const int32_t tid = tid_x();
    const int32_t m0 = task.m0, n0 = task.n0;
    const int32_t mlen = min(MB_BM, g.M - m0), nlen = min(MB_BN, g.N - n0);

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    for (int32_t r = 0; r < g.nrun; ++r) {
        const DRun run = ka.runs[g.run0 + r];
        __syncthreads();
        if (tid < 128) {
            if (tid < mlen) sm.ra[tid] = make_rec(ka.ap + run.ap0, run.nap, m0 + tid);
        } else {
            const int32_t j = tid - 128;
            if (j < nlen) sm.rb[j] = make_rec(ka.bp + run.bp0, run.nbp, n0 + j);
        }
        __syncthreads();
        const int32_t va = (run.flags & R_A_WS) ? 1 : ka.vec_a, vb = (run.flags & R_B_WS) ? 1 : ka.vec_b;
        const OpCtx oa = mb_ctx(ka.ap + run.ap0, run.nap, R_A_KUNIT, R_A_FUNIT, run.flags, m0, mlen, run.K,
                                run_a<uint16_t>(ka, run.flags), va, sm.ra);
        const OpCtx ob = mb_ctx(ka.bp + run.bp0, run.nbp, R_B_KUNIT, R_B_FUNIT, run.flags, n0, nlen, run.K,
                                run_b<uint16_t>(ka, run.flags), vb, sm.rb);
        const int32_t nchunks = (run.K + MB_BK - 1) / MB_BK;
        MbStage sa, sb;
        mb_load(oa, 0, sa);
        mb_load(ob, 0, sb);
        mb_store(oa, sa, sm.u.op.a[0], 0);
        mb_store(ob, sb, sm.u.op.b[0], 0);
        __syncthreads();
        for (int32_t c = 0; c < nchunks; ++c) {
            const bool more = c + 1 < nchunks;
            if (more) {
                mb_load(oa, (c + 1) * MB_BK, sa);
                mb_load(ob, (c + 1) * MB_BK, sb);
            }
            mb_compute(sm.u.op.a[c & 1], sm.u.op.b[c & 1], acc);
            if (more) {
                mb_store(oa, sa, sm.u.op.a[(c + 1) & 1], (c + 1) * MB_BK);
                mb_store(ob, sb, sm.u.op.b[(c + 1) & 1], (c + 1) * MB_BK);
            }
            __syncthreads();
        }
    }

    // epilogue: stage 64-row slabs of the fp32 tile in LDS (the operand buffers
    // are free now), then write rows out through the C pieces (the per-block
    // views), four consecutive columns per thread.
    const bool cn = (g.flags & G_C_ALONG_N) != 0;
    if (tid < 128) {
        if (!cn && tid < mlen) sm.ra[tid] = make_rec(ka.cp + g.cp0, g.ncp, m0 + tid);
        if (cn && tid < nlen) sm.ra[tid] = make_rec(ka.cp + g.cp0, g.ncp, n0 + tid);
    }
    float *slab = sm.u.slab;   // [64][MB_SLAB] floats
    TC *Cp = static_cast<TC *>(ka.C);
    const bool accum = (g.flags & G_ACCUMULATE) != 0;
    const int32_t lane = tid & 63, w = tid >> 6;
    const int32_t wm = w & 1, wn = w >> 1;
#pragma unroll
    for (int fi = 0; fi < 2; ++fi) {
        // slab row sr holds tile row (sr / 32) * 64 + fi * 32 + sr % 32
#pragma unroll
        for (int fj = 0; fj < 2; ++fj)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int32_t sr = wm * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                slab[sr * MB_SLAB + wn * 64 + fj * 32 + (lane & 31)] = acc[fi][fj][r];
            }
        __syncthreads();
        const int32_t c4 = (tid & 31) * 4;
#pragma unroll 1
        for (int q = 0; q < 8; ++q) {
            const int32_t sr = (tid >> 5) + 8 * q;
            const int32_t i = (sr >> 5) * 64 + fi * 32 + (sr & 31);
            if (i >= mlen || c4 >= nlen) continue;
            const float4 v = *reinterpret_cast<const float4 *>(slab + sr * MB_SLAB + c4);
            const float vv[4] = {v.x, v.y, v.z, v.w};
            if (!cn) {
                const Rec rc = sm.ra[i];
                const int64_t ad = along(rc, n0 + c4);
                if (sizeof(TC) == 4 && rc.in == 1 && rc.s0 == 1 && c4 + 4 <= nlen) {
                    // four consecutive fp32 outputs, one 16-byte access at any element address
                    float4 o = v;
                    if (accum) {
                        float4 c;
                        __builtin_memcpy(&c, Cp + ad, sizeof(c));
                        o.x += c.x;
                        o.y += c.y;
                        o.z += c.z;
                        o.w += c.w;
                    }
                    __builtin_memcpy(Cp + ad, &o, sizeof(o));
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (c4 + j >= nlen) break;
                        const int64_t aj = along(rc, n0 + c4 + j);
                        float o = vv[j];
                        if (accum) o += static_cast<float>(Cp[aj]);
                        Cp[aj] = static_cast<TC>(o);
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (c4 + j >= nlen) break;
                    const int64_t aj = along(sm.ra[c4 + j], m0 + i);
                    float o = vv[j];
                    if (accum) o += static_cast<float>(Cp[aj]);
                    Cp[aj] = static_cast<TC>(o);
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace bsc
