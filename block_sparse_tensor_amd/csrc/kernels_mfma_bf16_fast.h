// Dense matrix-core tile for bf16 inputs / fp32 accumulation.
//
// For a coalesced group that is one run of single strided views with
// 16-byte aligned rows (the planner's R_A_VEC and R_B_VECN / R_B_VECK
// conditions), the whole tile is described by a host-computed record (DFast):
// operand bases and strides, extents, K.  On top of the wave layout of the
// general tile (128 x 128 output, four 64 x 64 quadrants of
// v_mfma_f32_32x32x16_bf16):
//
//  * K chunks of 64 are copied global -> LDS with 16-byte direct-to-LDS loads
//    (no register staging); each wave instruction fills 1 KB of LDS in lane
//    order and the lane -> global mapping applies an XOR swizzle so the
//    fragment reads hit distinct banks;
//  * A (and B when it is K-contiguous) lives in LDS as [row][k] (128 B rows,
//    16-byte granules swizzled by row); fragments are single 16-byte reads;
//  * B that is N-contiguous (row-major B) lives in LDS as [k][n] (256 B rows,
//    64-byte granules swizzled by k) and each MFMA B fragment comes from two
//    transposing LDS reads (ds_read_b64_tr_b16), so no ALU transpose;
//  * STAGES LDS stages in a ring: while chunk c feeds the matrix cores the
//    copies of the next STAGES - 1 chunks are in flight; each wave waits
//    (vmcnt) only for its own copies of chunk c, then one barrier per chunk;
//  * the last, partial K chunk goes through masked register loads so every
//    element with k >= K is an exact zero in both operands; rows (columns)
//    past the tile edge are clamped to a valid row and their results dropped;
//  * results go straight from the accumulators to C (no staging).
#pragma once

#include "kernels_mfma_bf16.h"

namespace bsc {

typedef short v4i16_t __attribute__((ext_vector_type(4)));

constexpr int FB_BK = 64;
constexpr int FB_STAGE = 128 * 64;       // bf16 elements per operand per stage (16 KB)
constexpr int FB_STAGES = 2;             // LDS ring depth (FB_STAGES * 32 KB of LDS)

#define BSC_LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

struct FastSmemBf16 {
    uint16_t op[FB_STAGES][2][FB_STAGE];   // [stage][A=0,B=1][...]
};

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_vm_chunks(int32_t chunks_after) {
    // each chunk is 8 copies per wave (4 for A, 4 for B)
    switch (chunks_after) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<8>(); break;
        case 2: wait_vm<16>(); break;
        case 3: wait_vm<24>(); break;
        case 4: wait_vm<32>(); break;
        case 5: wait_vm<40>(); break;
        default: wait_vm<48>(); break;
    }
}
static_assert(FB_STAGES - 1 <= 6, "vmcnt table covers at most 6 chunks ahead");

// Workgroup barrier for handing LDS stages between waves.  Each wave first
// waits for its own LDS writes (lgkmcnt) — its direct-to-LDS copies were
// already waited for by count — so, unlike __syncthreads(), copies of later
// chunks stay in flight across it.  The empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16-byte granule (of 8) holding k-granule g in A-layout row r
__device__ __forceinline__ int32_t fa_slot(int32_t r, int32_t g) { return g ^ ((r ^ (r >> 3)) & 7); }
// 64-byte granule (of 4) holding n-granule G in B-layout row k
__device__ __forceinline__ int32_t fb_pos(int32_t k, int32_t G) { return G ^ (k & 3); }

struct FastOp {
    const uint16_t *p[4];   // per-instruction global pointers at chunk 0
    int64_t step;           // elements to advance per chunk
};

// K-contiguous operand ([x][k] layout), element (x, k) at base + x * xs + k:
// wave w instruction j covers rows 32w + 8j .. +8, lane l row 8j + l/8, slot l%8.
__device__ __forceinline__ FastOp dense_setup_kcontig(int64_t base, int64_t xs, int32_t xlen, const uint16_t *P) {
    FastOp f;
    const int32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int32_t r = 32 * w + 8 * j + (lane >> 3);
        const int32_t rr = r < xlen ? r : 0;                      // rows past the edge: a valid row
        f.p[j] = P + base + static_cast<int64_t>(rr) * xs + 8 * fa_slot(r, lane & 7);
    }
    f.step = FB_BK;
    return f;
}

// N-contiguous operand ([k][n] layout), element (k, n) at base + k * ks + n:
// instruction j covers k rows 16w + 4j .. +4, lane l row 4j + l/16, 16-byte slot l%16.
__device__ __forceinline__ FastOp dense_setup_ncontig(int64_t base, int64_t ks, int32_t nlen, const uint16_t *P) {
    FastOp f;
    const int32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int32_t s = lane & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int32_t kr = 16 * w + 4 * j + (lane >> 4);
        const int32_t G = fb_pos(kr, s >> 2);                     // global n-granule for this LDS position
        int32_t n = 32 * G + 8 * (s & 3);
        if (n >= nlen) n = 0;                                      // columns past the edge: a valid column
        f.p[j] = P + base + n + static_cast<int64_t>(kr) * ks;
    }
    f.step = static_cast<int64_t>(FB_BK) * ks;
    return f;
}

__device__ __forceinline__ void fast_issue(const FastOp &f, int32_t c, uint16_t *lds_stage) {
    const int32_t w = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint16_t *src = f.p[j] + static_cast<int64_t>(c) * f.step;
        uint16_t *dst = lds_stage + (4 * w + j) * 512;               // 1 KB per wave instruction
        __builtin_amdgcn_global_load_lds(src, BSC_LDS_PTR(void, dst), 16, 0, 0);
    }
}

// Masked fills of a partial chunk (k0 .. K-1 valid) through registers.
__device__ __forceinline__ void dense_fill_kcontig(int64_t base, int64_t xs, int32_t xlen, int32_t k0, int32_t K,
                                                   const uint16_t *P, uint16_t *lds) {
    const int32_t tid = threadIdx.x;
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
        const int32_t u = tid + 256 * q;         // 1024 granules: row u >> 3, k-granule u & 7
        const int32_t r = u >> 3, g = u & 7;
        const int32_t k = k0 + 8 * g;
        uint16_t e[8];
        const uint16_t *row = P + base + static_cast<int64_t>(r) * xs;
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = (r < xlen && k + t < K) ? row[k + t] : uint16_t(0);
        *reinterpret_cast<uint4 *>(lds + r * 64 + 8 * fa_slot(r, g)) = u4_from(e);
    }
}

__device__ __forceinline__ void dense_fill_ncontig(int64_t base, int64_t ks, int32_t nlen, int32_t k0, int32_t K,
                                                   const uint16_t *P, uint16_t *lds) {
    const int32_t tid = threadIdx.x;
#pragma unroll 1
    for (int q = 0; q < 4; ++q) {
        const int32_t u = tid + 256 * q;         // 1024 granules: k row u >> 4, 8-column piece u & 15
        const int32_t kr = u >> 4, s = u & 15;
        const int32_t n = 8 * s, k = k0 + kr;
        uint16_t e[8];
        const uint16_t *row = P + base + static_cast<int64_t>(k) * ks;
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = (k < K && n + t < nlen) ? row[n + t] : uint16_t(0);
        *reinterpret_cast<uint4 *>(lds + kr * 128 + 32 * fb_pos(kr, n >> 5) + 8 * ((n >> 3) & 3)) = u4_from(e);
    }
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(BSC_LDS_PTR(const void, p)));
}

// Fragment reads are issued from asm.  This keeps the compiler from treating
// them as possible readers of an in-flight direct-to-LDS copy (it would wait
// for that copy first), and, with scheduling barriers around the MFMAs, keeps
// the reads of K-step s+1 in flight while step s runs on the matrix cores.
// frag_wait waits for all LDS reads; naming the fragments as its outputs keeps
// every use after it.
typedef int v4i32_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void lds_read_b128(uint32_t ad, v4i32_t &r) {
    asm volatile("ds_read_b128 %0, %1" : "=&v"(r) : "v"(ad) : "memory");
}

__device__ __forceinline__ void lds_read_tr4(uint32_t a0, uint32_t a1, uint32_t a2, uint32_t a3, v4i16_t &r0,
                                             v4i16_t &r1, v4i16_t &r2, v4i16_t &r3) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %5\n\t"
        "ds_read_b64_tr_b16 %2, %6\n\t"
        "ds_read_b64_tr_b16 %3, %7"
        : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
        : "v"(a0), "v"(a1), "v"(a2), "v"(a3)
        : "memory");
}

// Operand fragments of one K-step (16) for the 2 x 2 MFMA tiles.
struct Frags {
    v4i32_t a[2];
    v4i32_t b[2];     // K-contiguous B
    v4i16_t t[4];     // N-contiguous B: transposed halves
};

template <bool BN>
__device__ __forceinline__ void frag_issue(const uint16_t *la, const uint16_t *lb, int32_t ks, Frags &fr) {
    const int32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int32_t wm = w & 1, wn = w >> 1;
    if constexpr (BN) {
        const int32_t hh = lane >> 4, p = lane & 15;
        const int32_t gk = hh >> 1, noff = 16 * (hh & 1);
        uint32_t ad[4];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int32_t n = wn * 64 + f * 32 + noff + 4 * (p & 3);
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const int32_t k = ks * 16 + 8 * gk + 4 * h2 + (p >> 2);
                ad[2 * f + h2] = lds_addr(lb + k * 128 + 32 * fb_pos(k, n >> 5) + (n & 31));
            }
        }
        lds_read_tr4(ad[0], ad[1], ad[2], ad[3], fr.t[0], fr.t[1], fr.t[2], fr.t[3]);
    } else {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int32_t r = wn * 64 + f * 32 + (lane & 31);
            lds_read_b128(lds_addr(lb + r * 64 + 8 * fa_slot(r, 2 * ks + (lane >> 5))), fr.b[f]);
        }
    }
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int32_t r = wm * 64 + f * 32 + (lane & 31);
        lds_read_b128(lds_addr(la + r * 64 + 8 * fa_slot(r, 2 * ks + (lane >> 5))), fr.a[f]);
    }
}

template <bool BN>
__device__ __forceinline__ void frag_wait(Frags &fr) {
    if constexpr (BN)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(fr.a[0]), "+v"(fr.a[1]), "+v"(fr.t[0]), "+v"(fr.t[1]), "+v"(fr.t[2]), "+v"(fr.t[3])
                     :
                     : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(fr.a[0]), "+v"(fr.a[1]), "+v"(fr.b[0]), "+v"(fr.b[1]) : : "memory");
}

template <bool BN>
__device__ __forceinline__ void frag_mfma(const Frags &fr, f32x16_t (&acc)[2][2]) {
    bf16x8_t fa[2], fb[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        fa[f] = __builtin_bit_cast(bf16x8_t, fr.a[f]);
        if constexpr (BN) {
            const v4i16_t lo = fr.t[2 * f], hi = fr.t[2 * f + 1];
            short e8 __attribute__((ext_vector_type(8))) = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            fb[f] = __builtin_bit_cast(bf16x8_t, e8);
        } else {
            fb[f] = __builtin_bit_cast(bf16x8_t, fr.b[f]);
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// One K chunk (4 steps of 16) with the fragment reads of step s+1 in flight
// while the matrix cores run step s.
template <bool BN>
__device__ __forceinline__ void fast_chunk(const uint16_t *la, const uint16_t *lb, f32x16_t (&acc)[2][2]) {
    Frags cur, nxt;
    frag_issue<BN>(la, lb, 0, cur);
    frag_wait<BN>(cur);
#pragma unroll
    for (int32_t ks = 0; ks < 4; ++ks) {
        if (ks < 3) frag_issue<BN>(la, lb, ks + 1, nxt);
        __builtin_amdgcn_sched_barrier(0);
        frag_mfma<BN>(cur, acc);
        __builtin_amdgcn_sched_barrier(0);
        if (ks < 3) {
            frag_wait<BN>(nxt);
            cur = nxt;
        }
    }
}

template <typename TC, bool BN>
__device__ __forceinline__ void fast_tile_bf16(const KArgs &ka, const DFast &fd_ref, FastSmemBf16 &sm) {
    const DFast fd = fd_ref;   // one read of the record
    const uint16_t *A = static_cast<const uint16_t *>((fd.flags & F_A_WS) ? ka.W : ka.A);
    const uint16_t *B = static_cast<const uint16_t *>((fd.flags & F_B_WS) ? ka.W : ka.B);
    const int32_t mlen = fd.mlen, nlen = fd.nlen, K = fd.K;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const FastOp fa = dense_setup_kcontig(fd.a_base, fd.a_rs, mlen, A);
    const int64_t b_s = BN ? fd.b_ks : fd.b_ns;   // stride of B's non-contiguous axis
    const FastOp fb = BN ? dense_setup_ncontig(fd.b_base, b_s, nlen, B) : dense_setup_kcontig(fd.b_base, b_s, nlen, B);
    const int32_t nfull = K / FB_BK;
    const int32_t ntot = (K + FB_BK - 1) / FB_BK;
    auto fill_partial = [&](int32_t stage) {
        dense_fill_kcontig(fd.a_base, fd.a_rs, mlen, nfull * FB_BK, K, A, sm.op[stage][0]);
        if (BN) dense_fill_ncontig(fd.b_base, b_s, nlen, nfull * FB_BK, K, B, sm.op[stage][1]);
        else dense_fill_kcontig(fd.b_base, b_s, nlen, nfull * FB_BK, K, B, sm.op[stage][1]);
    };
    wait_vm<0>();      // nothing else outstanding: the counted waits below see only this tile's copies
    __syncthreads();   // previous users of the LDS ring are done
    int32_t issued = 0;
#pragma unroll
    for (int32_t p = 0; p < FB_STAGES - 1; ++p) {
        if (p < nfull) {
            fast_issue(fa, p, sm.op[p][0]);
            fast_issue(fb, p, sm.op[p][1]);
            ++issued;
        }
    }
    if (nfull < ntot && nfull <= FB_STAGES - 2) fill_partial(nfull);
    for (int32_t c = 0; c < ntot; ++c) {
        if (c < nfull) wait_vm_chunks(issued - c - 1);   // this wave's copies of chunk c have landed
        lds_barrier();                                  // ... and every other wave's
        const int32_t nx = c + FB_STAGES - 1;           // refill the stage chunk c-1 used
        const int32_t st = nx % FB_STAGES;
        if (nx < nfull) {
            fast_issue(fa, nx, sm.op[st][0]);
            fast_issue(fb, nx, sm.op[st][1]);
            ++issued;
        } else if (nx == nfull && nfull < ntot) {
            fill_partial(st);
        }
        const int32_t cs = c % FB_STAGES;
        fast_chunk<BN>(sm.op[cs][0], sm.op[cs][1], acc);
    }

    // epilogue: straight from the accumulators, 32 consecutive columns per row
    TC *Cp = static_cast<TC *>(ka.C);
    const bool accum = (fd.flags & G_ACCUMULATE) != 0;
    const int32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int32_t wm = w & 1, wn = w >> 1;
#pragma unroll
    for (int fj = 0; fj < 2; ++fj) {
        const int32_t j = wn * 64 + fj * 32 + (lane & 31);
        if (j >= nlen) continue;
        TC *col = Cp + fd.c_base + static_cast<int64_t>(j) * fd.c_cs;
#pragma unroll
        for (int fi = 0; fi < 2; ++fi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int32_t i = wm * 64 + fi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (i >= mlen) continue;
                TC *dst = col + static_cast<int64_t>(i) * fd.c_rs;
                float v = acc[fi][fj][r];
                if (accum) v += static_cast<float>(*dst);
                *dst = static_cast<TC>(v);
            }
    }
}

}  // namespace bsc
