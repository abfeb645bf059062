// Dense matrix-core tile for bf16 inputs / fp32 accumulation.
//
// For a coalesced group that is one run of single strided views with
// 16-byte aligned rows (the planner's R_A_VEC and R_B_VECN / R_B_VECK
// conditions), the whole tile is described by a host-computed record (DFast):
// operand bases and strides, extents, K.  The tile is 256 x 128, computed by
// four waves in a 2 x 2 arrangement; each wave owns 128 x 64 as 4 x 2 tiles
// of v_mfma_f32_32x32x16_bf16.  Two workgroups share a CU, so every SIMD holds
// two waves and one wave's LDS fragment reads overlap the other's MFMAs.
//
// Why this shape: with a 64 x 64 wave tile the LDS fragment reads (1 KB per
// MFMA) take as long as the MFMAs themselves; a 128 x 64 wave tile reads
// 0.75 KB per MFMA, which two waves per SIMD hide behind the matrix cores.  A
// 256 x 128 tile also fetches 25 % fewer operand bytes per flop than 128 x 128.
//
//  * K is cut into chunks of 32 (24 KB per stage: A 256 x 32, B 32 x 128)
//    held in a ring of FB_STAGES stages (72 KB per workgroup, two per CU);
//    FB_STAGES - 1 chunks are in flight while one feeds the matrix cores;
//  * chunks are copied global -> LDS with 16-byte direct-to-LDS loads (no
//    register staging); each wave instruction fills 1 KB of LDS in lane order
//    and the lane -> global mapping applies an XOR swizzle so the fragment
//    reads hit distinct banks;
//  * A (and B when it is K-contiguous) lives in LDS as [row][k], 64-byte rows
//    of four 16-byte granules, granule g of row r in slot g ^ fa_perm(r): the
//    eight rows one LDS cycle serves sit in distinct 16-byte bank groups;
//  * B that is N-contiguous (row-major B) lives in LDS as [k][n] (256 B rows,
//    64-byte granules swizzled by k) and each MFMA B fragment comes from two
//    transposing LDS reads (ds_read_b64_tr_b16), so no ALU transpose;
//  * each wave waits (vmcnt) only for its own copies of chunk c, then one
//    barrier per chunk hands the stage over; a wave whose A rows all lie past
//    the tile edge copies no A (the rows it would fill only feed results that
//    are dropped);
//  * the last, partial K chunk goes through masked register loads so every
//    element with k >= K is an exact zero in both operands; rows (columns)
//    past the tile edge are clamped to a valid row and their results dropped;
//  * results go straight from the accumulators to C (no staging).
#pragma once

#include <type_traits>

#include "kernels_mfma_bf16.h"

namespace bsc {

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int FB_BM = 256;                      // tile rows
constexpr int FB_BN = 128;                      // tile columns
constexpr int FB_BK = 32;                       // contracted indices per chunk
constexpr int FB_A_STAGE = FB_BM * FB_BK;       // bf16 elements of A per full stage (16 KB)
constexpr int FB_B_STAGE = FB_BN * FB_BK;       // bf16 elements of B per stage (8 KB)
constexpr int FB_NIA = FB_A_STAGE * 2 / 1024 / 4;   // 1 KB copies of A per wave and chunk (4)
constexpr int FB_NIB = FB_B_STAGE * 2 / 1024 / 4;   // 1 KB copies of B per wave and chunk (2)
constexpr int FB_FM = FB_BM / 2 / 32;               // row fragments per wave (4)
static_assert(FB_BM == TILE_MFMA_DENSE_M && FB_BN == TILE_MFMA, "tile shape the planner cuts");

#define BSC_LDS_PTR(T, p) ((__attribute__((address_space(3))) T *)(p))

// The LDS ring: three 24 KB stages (A 256 x 32, then B 32 x 128).  A task of
// at most 128 rows runs in the same 80 KB as a 128 x 128 tile of four 64 x 64
// waves with five 16 KB stages (HalfTile, kernels_mfma_bf16_wide.h).
struct Ring {
    static constexpr int STAGES = 3;
    static constexpr int A_ELEMS = FB_BM * FB_BK;   // A part of a stage
    static constexpr int STAGE_ELEMS = A_ELEMS + FB_B_STAGE;
};
constexpr int FB_RING_ELEMS = 40960;   // 80 KB: two workgroups per CU
static_assert(Ring::STAGES * Ring::STAGE_ELEMS <= FB_RING_ELEMS, "full ring");

struct FastSmemBf16 {
    uint16_t op[FB_RING_ELEMS];
};

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding; expcnt and lgkmcnt left unconstrained).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until this wave's copies of the chunk that has `chunks_after` newer
// chunks in flight have landed (PER copies per chunk and wave).
template <int PER>
__device__ __forceinline__ void wait_vm_chunks(int32_t chunks_after) {
    switch (chunks_after) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<PER>(); break;
        case 2: wait_vm<2 * PER>(); break;
        default: wait_vm<3 * PER>(); break;
    }
}
static_assert(Ring::STAGES - 2 <= 3 && 3 * (FB_NIA + FB_NIB) < 64, "wait table: at most three newer chunks");

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

// Row permutation of the A-layout swizzle (values 0..3, period 16): the four
// rows of one parity among any eight consecutive rows get distinct values.
__device__ __forceinline__ int32_t fa_perm(int32_t r) { return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1); }
// 16-byte slot (of 4) holding k-granule g in A-layout row r
__device__ __forceinline__ int32_t fa_slot(int32_t r, int32_t g) { return g ^ fa_perm(r); }
// 64-byte granule (of 4) holding n-granule G in B-layout row k
__device__ __forceinline__ int32_t fb_pos(int32_t k, int32_t G) { return G ^ (k & 3); }

// Copies go through buffer descriptors: the tile's range of the operand in
// scalar registers, one 32-bit lane offset per copy instruction, and the chunk
// advance as the scalar offset (the planner keeps every tile range below
// 2 GiB).  The hardware range check of a raw buffer covers the lane offset
// only, not the scalar offset, so no copy may address a chunk past the last
// full one: the partial last chunk goes through the masked register fill.
constexpr int32_t BUF_DWORD3 = 0x00020000;   // raw 32-bit buffer (gfx9 descriptor word 3)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void *base, int64_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint64_t ua = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(a >> 32))) << 32) |
                        static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(a)));
    const int32_t n = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(bytes));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ua), 0, n, BUF_DWORD3);
}

template <int NI>
struct FastOp {
    __amdgpu_buffer_rsrc_t rs;   // the operand's range for this tile
    uint32_t off[NI];            // per-instruction lane byte offsets at chunk 0
    uint32_t step;               // bytes to advance per chunk
};

// K-contiguous operand ([x][k] layout), element (x, k) at base + x * xs + k:
// copy block w (a wave's share) instruction j fills rows 16 (NI w + j) .. +16
// (1 KB); lane l fills row l / 4, slot l % 4, so it copies k-granule
// (l % 4) ^ fa_perm(row).
template <int NI>
__device__ __forceinline__ FastOp<NI> dense_setup_kcontig(int64_t base, int64_t xs, int32_t xlen, int32_t K,
                                                          const uint16_t *P, int32_t w) {
    FastOp<NI> f;
    const int32_t lane = tid_x() & 63;
    f.rs = wave_rsrc(P + base, 2 * (static_cast<int64_t>(xlen - 1) * xs + K) + 16);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int32_t r = 16 * (NI * w + j) + (lane >> 2);
        const int32_t rr = r < xlen ? r : 0;                      // rows past the edge: a valid row
        f.off[j] = static_cast<uint32_t>(2 * (static_cast<int64_t>(rr) * xs + 8 * ((lane & 3) ^ fa_perm(r))));
    }
    f.step = 2 * FB_BK;
    return f;
}

// N-contiguous operand ([k][n] layout), element (k, n) at base + k * ks + n:
// instruction j fills k rows 4 (NI w + j) .. +4; lane l fills row l / 16,
// 16-byte slot l % 16.
template <int NI>
__device__ __forceinline__ FastOp<NI> dense_setup_ncontig(int64_t base, int64_t ks, int32_t nlen, int32_t K,
                                                          const uint16_t *P, int32_t w) {
    FastOp<NI> f;
    const int32_t lane = tid_x() & 63;
    const int32_t s = lane & 15;
    f.rs = wave_rsrc(P + base, 2 * (static_cast<int64_t>(K - 1) * ks + FB_BN) + 16);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int32_t kr = 4 * (NI * w + j) + (lane >> 4);
        const int32_t G = fb_pos(kr, s >> 2);                     // global n-granule for this LDS position
        int32_t n = 32 * G + 8 * (s & 3);
        if (n >= nlen) n = 0;                                      // columns past the edge: a valid column
        f.off[j] = static_cast<uint32_t>(2 * (n + static_cast<int64_t>(kr) * ks));
    }
    f.step = static_cast<uint32_t>(2 * FB_BK * ks);
    return f;
}

template <bool BN>
__device__ __forceinline__ FastOp<FB_NIB> dense_setup_b(int64_t base, int64_t s, int32_t nlen, int32_t K,
                                                        const uint16_t *P, int32_t w) {
    if constexpr (BN) return dense_setup_ncontig<FB_NIB>(base, s, nlen, K, P, w);
    else return dense_setup_kcontig<FB_NIB>(base, s, nlen, K, P, w);
}

// w: the copy block (a wave's share), wave-uniform (the LDS destination goes through M0)
template <int NI>
__device__ __forceinline__ void fast_issue(const FastOp<NI> &f, int32_t c, uint16_t *lds_op, int32_t w) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        uint16_t *dst = lds_op + (NI * w + j) * 512;                 // 1 KB per wave instruction
        // (a non-const descriptor and int offsets: the form this compiler's host
        // pass accepts when the kernel template is instantiated from host code)
        __amdgpu_buffer_rsrc_t rs = f.rs;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, BSC_LDS_PTR(void, dst), 16, static_cast<int>(f.off[j]),
                                                 static_cast<int>(static_cast<uint32_t>(c) * f.step), 0, 0);
    }
}

// Masked fill of a partial chunk (k0 .. K-1 valid) of a K-contiguous operand
// through registers: ROWS rows of four 16-byte granules.
template <int ROWS, int NT = 256>
__device__ __forceinline__ void dense_fill_kcontig(int64_t base, int64_t xs, int32_t xlen, int32_t k0, int32_t K,
                                                   const uint16_t *P, uint16_t *lds) {
    const int32_t tid = tid_x();
#pragma unroll 1
    for (int q = 0; q < ROWS * 4 / NT; ++q) {
        const int32_t u = tid + NT * q;         // row u / 4, k-granule u % 4
        const int32_t r = u >> 2, g = u & 3;
        const int32_t k = k0 + 8 * g;
        uint16_t e[8];
        const uint16_t *row = P + base + static_cast<int64_t>(r) * xs;
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = (r < xlen && k + t < K) ? row[k + t] : uint16_t(0);
        *reinterpret_cast<uint4 *>(lds + r * FB_BK + 8 * fa_slot(r, g)) = u4_from(e);
    }
}

__device__ __forceinline__ void dense_fill_ncontig(int64_t base, int64_t ks, int32_t nlen, int32_t k0, int32_t K,
                                                   const uint16_t *P, uint16_t *lds) {
    const int32_t tid = tid_x();
#pragma unroll 1
    for (int q = 0; q < FB_BK * 16 / 256; ++q) {
        const int32_t u = tid + 256 * q;         // k row u / 16, 8-column piece u % 16
        const int32_t kr = u >> 4, s = u & 15;
        const int32_t n = 8 * s, k = k0 + kr;
        uint16_t e[8];
        const uint16_t *row = P + base + static_cast<int64_t>(k) * ks;
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = (k < K && n + t < nlen) ? row[n + t] : uint16_t(0);
        *reinterpret_cast<uint4 *>(lds + kr * FB_BN + 32 * fb_pos(kr, n >> 5) + 8 * ((n >> 3) & 3)) = u4_from(e);
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
// every use after it.  Every read is a per-chunk base address plus an
// immediate offset, so the addresses cost a few registers per wave.
typedef int v4i32_t __attribute__((ext_vector_type(4)));

template <int OFF>
__device__ __forceinline__ void lds_read_b128(uint32_t ad, v4i32_t &r) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=&v"(r) : "v"(ad), "i"(OFF) : "memory");
}

template <int OFF>
__device__ __forceinline__ void lds_read_tr(uint32_t ad, v4i16_t &r) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=&v"(r) : "v"(ad), "i"(OFF) : "memory");
}

// Per-lane byte offsets of a wave's fragment reads within a stage, fixed for
// the whole tile.  A rows wm*128 + f*32 + (lane % 32) read k-granule
// 2 ks + lane / 32; the row swizzle has period 16, so f moves the address by
// f * 2 KB and ks flips bit 5 of it.  N-contiguous B: lane (gk, half, p) reads
// k rows 16 ks + 8 gk + 4 h2 + p / 4 (h2 and ks move the address by 1 KB and
// 4 KB), columns wn*64 + f*32 + 16 half + 4 (p % 4); f flips bit 6.
struct FragOff {
    uint32_t a[2];   // A, by K-step
    uint32_t b[2];   // K-contiguous B by K-step; N-contiguous B by column fragment
};

template <bool BN>
__device__ __forceinline__ FragOff frag_offsets() {
    const int32_t lane = tid_x() & 63, w = tid_x() >> 6;
    const int32_t wm = w & 1, wn = w >> 1;
    FragOff o;
    const int32_t ra = wm * (FB_BM / 2) + (lane & 31);
    o.a[0] = 2 * (ra * FB_BK + 8 * fa_slot(ra, lane >> 5));
    o.a[1] = o.a[0] ^ 32;
    if constexpr (BN) {
        const int32_t hh = lane >> 4, p = lane & 15;
        const int32_t k = 8 * (hh >> 1) + (p >> 2);
        const int32_t n = wn * 64 + 16 * (hh & 1) + 4 * (p & 3);
        o.b[0] = 2 * (k * FB_BN + 32 * fb_pos(k, n >> 5) + (n & 31));
        o.b[1] = o.b[0] ^ 64;
    } else {
        const int32_t rb = wn * 64 + (lane & 31);
        o.b[0] = 2 * (rb * FB_BK + 8 * fa_slot(rb, lane >> 5));
        o.b[1] = o.b[0] ^ 32;
    }
    return o;
}

// Operand fragments of one K-step (16) of one wave: four row fragments of A,
// two column fragments of B.
struct Frags {
    v4i32_t a[FB_FM];
    v4i32_t b[2];     // K-contiguous B
    v4i16_t t[4];     // N-contiguous B: transposed halves
};

// stage: LDS byte address of the stage; va / vb: its per-lane read bases
template <bool BN, int KS>
__device__ __forceinline__ void frag_issue(uint32_t va, uint32_t vb0, uint32_t vb1, Frags &fr) {
    if constexpr (BN) {
        constexpr int KO = 2 * 16 * KS * FB_BN;   // 16 k rows per step
        constexpr int HO = 2 * 4 * FB_BN;         // 4 k rows per half
        lds_read_tr<KO>(vb0, fr.t[0]);
        lds_read_tr<KO + HO>(vb0, fr.t[1]);
        lds_read_tr<KO>(vb1, fr.t[2]);
        lds_read_tr<KO + HO>(vb1, fr.t[3]);
    } else {
        lds_read_b128<0>(vb0, fr.b[0]);
        lds_read_b128<2 * 32 * FB_BK>(vb0, fr.b[1]);
    }
    lds_read_b128<0>(va, fr.a[0]);
    lds_read_b128<1 * 2 * 32 * FB_BK>(va, fr.a[1]);
    lds_read_b128<2 * 2 * 32 * FB_BK>(va, fr.a[2]);
    lds_read_b128<3 * 2 * 32 * FB_BK>(va, fr.a[3]);
}

template <bool BN>
__device__ __forceinline__ void frag_wait(Frags &fr) {
    static_assert(FB_FM == 4, "four row fragments per wave");
    if constexpr (BN)
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(fr.a[0]), "+v"(fr.a[1]), "+v"(fr.a[2]), "+v"(fr.a[3]), "+v"(fr.t[0]), "+v"(fr.t[1]),
                       "+v"(fr.t[2]), "+v"(fr.t[3])
                     :
                     : "memory");
    else
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(fr.a[0]), "+v"(fr.a[1]), "+v"(fr.a[2]), "+v"(fr.a[3]), "+v"(fr.b[0]), "+v"(fr.b[1])
                     :
                     : "memory");
}

// The MFMAs of one K-step.  Fragments past the tile edge are computed too
// (their rows were loaded clamped to a valid row): conditional MFMAs would make
// the accumulators merge across branches, which costs far more than the work.
template <bool BN>
__device__ __forceinline__ void frag_mfma(const Frags &fr, f32x16_t (&acc)[FB_FM][2]) {
    bf16x8_t fa[FB_FM], fb[2];
#pragma unroll
    for (int f = 0; f < FB_FM; ++f) fa[f] = __builtin_bit_cast(bf16x8_t, fr.a[f]);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        if constexpr (BN) {
            const v4i16_t lo = fr.t[2 * f], hi = fr.t[2 * f + 1];
            short e8 __attribute__((ext_vector_type(8))) = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            fb[f] = __builtin_bit_cast(bf16x8_t, e8);
        } else {
            fb[f] = __builtin_bit_cast(bf16x8_t, fr.b[f]);
        }
    }
#pragma unroll
    for (int i = 0; i < FB_FM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// One fragment read (index r of the K-step's reads: B first, then A).
template <bool BN, int KS>
__device__ __forceinline__ void read_one(int r, uint32_t va, uint32_t vb0, uint32_t vb1, Frags &fr) {
    constexpr int KO = 2 * 16 * KS * FB_BN, HO = 2 * 4 * FB_BN, AR = 2 * 32 * FB_BK;
    if constexpr (BN) {
        switch (r) {
            case 0: lds_read_tr<KO>(vb0, fr.t[0]); break;
            case 1: lds_read_tr<KO + HO>(vb0, fr.t[1]); break;
            case 2: lds_read_tr<KO>(vb1, fr.t[2]); break;
            case 3: lds_read_tr<KO + HO>(vb1, fr.t[3]); break;
            case 4: lds_read_b128<0>(va, fr.a[0]); break;
            case 5: lds_read_b128<AR>(va, fr.a[1]); break;
            case 6: lds_read_b128<2 * AR>(va, fr.a[2]); break;
            default: lds_read_b128<3 * AR>(va, fr.a[3]); break;
        }
    } else {
        switch (r) {
            case 0: lds_read_b128<0>(vb0, fr.b[0]); break;
            case 1: lds_read_b128<AR>(vb0, fr.b[1]); break;
            case 2: lds_read_b128<0>(va, fr.a[0]); break;
            case 3: lds_read_b128<AR>(va, fr.a[1]); break;
            case 4: lds_read_b128<2 * AR>(va, fr.a[2]); break;
            default: lds_read_b128<3 * AR>(va, fr.a[3]); break;
        }
    }
}

// The eight MFMAs of one K-step (fragments `cur`) with the reads of the next
// K-step's fragments (`nxt`, K-step KS at the given bases) issued between
// them, so a single wave keeps its matrix core fed while the reads go out:
// reads start after the first PRE MFMAs (a gap between the last MFMA that
// read `nxt`'s registers and the first read that overwrites them), and
// `mid` runs right before MFMA PRE (the chunk hand-over: waits, barrier,
// copies), while the first MFMAs execute.
template <bool BN, int KS, int PRE, typename Mid>
__device__ __forceinline__ void mfma_interleaved(const Frags &cur, Frags &nxt, uint32_t va, uint32_t vb0, uint32_t vb1,
                                                 f32x16_t (&acc)[FB_FM][2], Mid &&mid) {
    constexpr int NR = BN ? 8 : 6;   // reads per K-step
    bf16x8_t fa[FB_FM], fb[2];
#pragma unroll
    for (int f = 0; f < FB_FM; ++f) fa[f] = __builtin_bit_cast(bf16x8_t, cur.a[f]);
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        if constexpr (BN) {
            const v4i16_t lo = cur.t[2 * f], hi = cur.t[2 * f + 1];
            short e8 __attribute__((ext_vector_type(8))) = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            fb[f] = __builtin_bit_cast(bf16x8_t, e8);
        } else {
            fb[f] = __builtin_bit_cast(bf16x8_t, cur.b[f]);
        }
    }
    // reads per MFMA slot from PRE on, the remainder after the last MFMA
    constexpr int SLOTS = 2 * FB_FM - PRE;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < 2 * FB_FM; ++k) {
        if (k == PRE) {
            mid();
            __builtin_amdgcn_sched_barrier(0);
        }
        acc[k / 2][k % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k / 2], fb[k % 2], acc[k / 2][k % 2], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (k >= PRE) {
            const int slot = k - PRE;
            // spread NR reads over SLOTS slots, front-loaded
            const int r0 = slot * NR / SLOTS, r1 = (slot + 1) * NR / SLOTS;
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (r >= r0 && r < r1) read_one<BN, KS>(r, va, vb0, vb1, nxt);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // keep `cur` allocated until every read into `nxt` is issued: a read must
    // not land in registers an MFMA issued just before it may still be reading
    if constexpr (BN)
        asm volatile("" ::"v"(cur.a[0]), "v"(cur.a[1]), "v"(cur.a[2]), "v"(cur.a[3]), "v"(cur.t[0]), "v"(cur.t[1]),
                     "v"(cur.t[2]), "v"(cur.t[3]));
    else
        asm volatile("" ::"v"(cur.a[0]), "v"(cur.a[1]), "v"(cur.a[2]), "v"(cur.a[3]), "v"(cur.b[0]), "v"(cur.b[1]));
}

// Fragment reads of one K-step (0 or 1) of the chunk whose stage starts at
// LDS byte address `stage`.
// stage: LDS byte address of the stage (its A part); bstage: of its B part
template <bool BN, int KS>
__device__ __forceinline__ void frag_step(uint32_t stage, uint32_t bstage, const FragOff &o, Frags &fr) {
    static_assert(FB_BK == 32, "two K-steps per chunk");
    // K-contiguous B: one base per K-step; N-contiguous B: one per column fragment
    const uint32_t vb0 = bstage + o.b[0], vb1 = bstage + o.b[1];
    if constexpr (BN) frag_issue<BN, KS>(stage + o.a[KS], vb0, vb1, fr);
    else frag_issue<BN, KS>(stage + o.a[KS], KS ? vb1 : vb0, vb1, fr);
}

// K split: one slice of the tile is done.  The slice stores its partial tile
// (lane-contiguous: 16-byte group q of lane l at q * 64 + l within the wave's
// block), waits until the stores are complete, then counts itself in the
// tile's counter.  Returns false for every slice but the last; the last resets
// the counter for the next launch and forms p0 + p1 + ... + p(S-1), added left
// to right, so the result does not depend on which slice finishes last.
//
// Slices may run on different chiplets, whose L2 caches are not kept coherent
// with each other.  The partials are therefore written and read with
// device-coherent buffer accesses (the sc1 cache policy that device-scope
// atomic loads and stores use, here without their one-at-a-time waits), and
// the counter is a device-scope atomic; no device-scope fence, whose
// whole-cache write-back and invalidation would stall every other workgroup on
// the chiplet.  A pair's last slice adds the other's partial to the one it
// holds (a + b and b + a are the same float); more slices reload all partials
// in slice order.  The buffer descriptor covers exactly the tile's partials,
// so the hardware drops any access outside them.
constexpr int32_t CPOL_SC1 = 16;             // device-coherent cache policy

__device__ __forceinline__ bool split_arrive(const KArgs &ka, const DFast &fd, f32x16_t (&acc)[FB_FM][2], int32_t w,
                                             int32_t lane, int32_t &last) {
    constexpr int SPLIT_BYTES = FB_BM * FB_BN * 4;   // one partial tile
    constexpr int NQ = FB_FM * 2 * 4;                 // 16-byte groups per lane (32)
    // the record is wave-uniform: build the descriptor in scalar registers
    const uint64_t base = reinterpret_cast<uint64_t>(ka.P + fd.part);
    const uint64_t ubase = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(base >> 32))) << 32) |
                           static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(base)));
    const int32_t nsplit = __builtin_amdgcn_readfirstlane(fd.nsplit);
    const int32_t me = __builtin_amdgcn_readfirstlane(fd.split);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ubase), 0, nsplit * SPLIT_BYTES, BUF_DWORD3);
    const int32_t lane_off = (w * NQ * 64 + lane) * 16;
    const int32_t mine = me * SPLIT_BYTES + lane_off;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const f32x16_t &a = acc[q / 8][(q / 4) & 1];
        const int r = 4 * (q & 3);
        const f32x4_t v = {a[r], a[r + 1], a[r + 2], a[r + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i32_t, v), rs, mine + q * 1024, 0, CPOL_SC1);
    }
    wait_vm<0>();   // this wave's partial stores are complete
    __syncthreads();
    if (tid_x() == 0) {
        const int32_t before = __hip_atomic_fetch_add(ka.cnt + fd.counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = before == fd.nsplit - 1;
        if (last) __hip_atomic_store(ka.cnt + fd.counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return false;
    constexpr int SPLIT_BATCH = 16;
    // A pair's last slice keeps its own partial and adds the other's; with
    // more slices, slice 0 replaces the accumulators and slices 1.. are added
    // in order.  (One add loop serves both: a second copy of it made the
    // compiler spill the whole kernel to scratch.)
    const bool pair = nsplit == 2;
    if (!pair) {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            f32x16_t &a = acc[q / 8][(q / 4) & 1];
            const int r = 4 * (q & 3);
            // (the whole vector is reinterpreted at once: extracting single lanes of
            // the loaded integer vector through bit casts is narrowed to a
            // one-dword load by this compiler)
            const f32x4_t x =
                __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off + q * 1024, 0, CPOL_SC1));
#pragma unroll
            for (int e = 0; e < 4; ++e) a[r + e] = x[e];
        }
    }
    for (int32_t s = pair ? 0 : 1; s < nsplit; ++s) {
        if (pair && s == me) continue;
        const int32_t src = s * SPLIT_BYTES + lane_off;
#pragma unroll
        for (int h = 0; h < NQ; h += SPLIT_BATCH) {
            // a batch of loads issued before any is added (one by one, each
            // would wait out a full memory round trip)
            v4i32_t t[SPLIT_BATCH];
#pragma unroll
            for (int u = 0; u < SPLIT_BATCH; ++u)
                t[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, src + (h + u) * 1024, 0, CPOL_SC1);
#pragma unroll
            for (int u = 0; u < SPLIT_BATCH; ++u) {
                const int q = h + u;
                f32x16_t &a = acc[q / 8][(q / 4) & 1];
                const int r = 4 * (q & 3);
                const f32x4_t x = __builtin_bit_cast(f32x4_t, t[u]);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[r + e] += x[e];
            }
        }
    }
    return true;
}

template <typename TC, bool BN>
__device__ __forceinline__ void fast_tile_bf16(const KArgs &ka, const DFast &fd_ref, FastSmemBf16 &sm) {
    const DFast fd = fd_ref;   // one read of the record
    const uint16_t *A = static_cast<const uint16_t *>((fd.flags & F_A_WS) ? ka.W : ka.A);
    const uint16_t *B = static_cast<const uint16_t *>((fd.flags & F_B_WS) ? ka.W : ka.B);
    const int32_t mlen = fd.mlen, nlen = fd.nlen, K = fd.K;
    // the wave index through a scalar register, so tests on it are scalar branches
    const int32_t w = __builtin_amdgcn_readfirstlane(tid_x() >> 6);

    f32x16_t acc[FB_FM][2];
#pragma unroll
    for (int i = 0; i < FB_FM; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Wave roles.  Wave (wm, wn) computes rows wm*128 .. +128 and columns
    // wn*64 .. +64 of the tile and copies A rows wm*128 + wn*64 .. +64; a wave
    // whose rows (or columns) lie wholly past the tile edge computes nothing,
    // and one whose A rows do copies no A (only tiles of more than 128 rows
    // come here, so every wave computes unless the tile is narrow).  Every
    // wave copies its share of B.  The roles are wave-uniform, so each wave
    // runs one instantiation of the K loop below; all of them meet at the same
    // barriers.
    const int32_t wm = w & 1, wn = w >> 1;
    const bool compute = wm * (FB_BM / 2) < mlen && wn * (FB_BN / 2) < nlen;
    const bool acopy = wm * (FB_BM / 2) + wn * (FB_BM / 4) < mlen;
    const FastOp<FB_NIA> fa = dense_setup_kcontig<FB_NIA>(fd.a_base, fd.a_rs, mlen, K, A, 2 * wm + wn);
    const int64_t b_s = BN ? fd.b_ks : fd.b_ns;   // stride of B's non-contiguous axis
    const FastOp<FB_NIB> fb = dense_setup_b<BN>(fd.b_base, b_s, nlen, K, B, w);
    const int32_t nfull = K / FB_BK;
    const int32_t ntot = (K + FB_BK - 1) / FB_BK;
    const FragOff fo = frag_offsets<BN>();
    wait_vm<0>();      // nothing else outstanding: the counted waits below see only this tile's copies
    __syncthreads();   // previous users of the LDS ring are done

    auto kloop = [&](auto compute_c, auto acopy_c) {
        constexpr bool COMPUTE = decltype(compute_c)::value, ACOPY = decltype(acopy_c)::value;
        using R = Ring;
        constexpr int STAGES = R::STAGES;
        constexpr int PER = (ACOPY ? FB_NIA : 0) + FB_NIB;   // copies per chunk and wave
        uint16_t *const ops = sm.op;
        auto fill_partial = [&](int32_t stage) {
            uint16_t *at = ops + stage * R::STAGE_ELEMS;
            dense_fill_kcontig<FB_BM>(fd.a_base, fd.a_rs, mlen, nfull * FB_BK, K, A, at);
            if constexpr (BN) dense_fill_ncontig(fd.b_base, b_s, nlen, nfull * FB_BK, K, B, at + R::A_ELEMS);
            else dense_fill_kcontig<FB_BN>(fd.b_base, b_s, nlen, nfull * FB_BK, K, B, at + R::A_ELEMS);
        };
        auto issue = [&](int32_t c, int32_t stage) {
            uint16_t *at = ops + stage * R::STAGE_ELEMS;
            if constexpr (ACOPY) fast_issue<FB_NIA>(fa, c, at, 2 * wm + wn);
            fast_issue<FB_NIB>(fb, c, at + R::A_ELEMS, w);
        };
        int32_t issued = 0;
#pragma unroll
        for (int32_t p = 0; p < STAGES - 1; ++p) {
            if (p < nfull) {
                issue(p, p);
                ++issued;
            }
        }
        if (nfull < ntot && nfull <= STAGES - 2) fill_partial(nfull);
        // Make chunk cn readable: this wave's copies of it have landed, then the
        // barrier (every wave's have, and every wave is done reading chunk cn - 1,
        // whose stage is refilled with chunk cn + STAGES - 1).
        auto advance = [&](int32_t cn) {
            if (cn < nfull) wait_vm_chunks<PER>(issued - cn - 1);
            lds_barrier();
            const int32_t nx = cn + STAGES - 1;
            const int32_t st = nx % STAGES;
            if (nx < nfull) {
                issue(nx, st);
                ++issued;
            } else if (nx == nfull && nfull < ntot) {
                fill_partial(st);
            }
        };
        const uint32_t ring = lds_addr(ops);
        constexpr uint32_t STAGE_BYTES = R::STAGE_ELEMS * 2, B_OFF = R::A_ELEMS * 2;
        auto stage_addr = [&](int32_t c) { return ring + (c % STAGES) * STAGE_BYTES; };
        // software-pipelined across chunks: the reads of step 1 of chunk c
        // overlap the MFMAs of step 0, and the reads of step 0 of chunk c + 1
        // (after the hand-over barrier) overlap the MFMAs of step 1
        Frags s0, s1;
        auto reads = [&](auto ks_c, uint32_t stage, Frags &fr) {
            if constexpr (COMPUTE) frag_step<BN, decltype(ks_c)::value>(stage, stage + B_OFF, fo, fr);
        };
        auto mfmas = [&](const Frags &fr) {
            if constexpr (COMPUTE) {
                __builtin_amdgcn_sched_barrier(0);
                frag_mfma<BN>(fr, acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto settle = [&](Frags &fr) {
            if constexpr (COMPUTE) frag_wait<BN>(fr);
        };
        using K0 = std::integral_constant<int, 0>;
        using K1 = std::integral_constant<int, 1>;
        advance(0);
        reads(K0(), stage_addr(0), s0);
        settle(s0);
        // Steady state, without branches: while chunk c + STAGES is a full
        // chunk, iteration c waits for chunk c + 1 with STAGES - 2 newer chunks
        // still in flight and refills chunk c's stage with chunk c + STAGES.
        // The stage rotates through scalar selects.
        int32_t c = 0, st = 0;
        const int32_t nsteady = nfull - STAGES;   // iterations whose refill is a full chunk
        for (; c < nsteady; ++c) {
            const int32_t sn = st == STAGES - 1 ? 0 : st + 1;
            if constexpr (COMPUTE) {
                // MFMAs of step 0 with the reads of step 1 (same stage) between them;
                // then the MFMAs of step 1 with the hand-over (wait, barrier, refill)
                // after the first two and the reads of chunk c + 1's step 0 after it
                const uint32_t here = ring + st * STAGE_BYTES, next = ring + sn * STAGE_BYTES;
                mfma_interleaved<BN, 1, 2>(s0, s1, here + fo.a[1], here + B_OFF + fo.b[BN ? 0 : 1],
                                           here + B_OFF + fo.b[1], acc, [] {});
                settle(s1);
                mfma_interleaved<BN, 0, 2>(s1, s0, next + fo.a[0], next + B_OFF + fo.b[0], next + B_OFF + fo.b[1], acc,
                                           [&] {
                                               wait_vm<PER * (STAGES - 2)>();
                                               lds_barrier();
                                               issue(c + STAGES, st);
                                           });
                settle(s0);
            } else {
                wait_vm<PER * (STAGES - 2)>();
                lds_barrier();
                issue(c + STAGES, st);
            }
            st = sn;
        }
        issued = c + STAGES < nfull ? c + STAGES : nfull;   // chunks 0 .. c + STAGES - 1 are issued
        for (; c < ntot; ++c) {
            reads(K1(), stage_addr(c), s1);
            mfmas(s0);
            settle(s1);
            const bool more = c + 1 < ntot;
            if (more) {
                advance(c + 1);
                reads(K0(), stage_addr(c + 1), s0);
            }
            mfmas(s1);
            if (more) settle(s0);
        }
    };
    using T = std::true_type;
    using F = std::false_type;
    if (compute) {
        if (acopy) kloop(T(), T());
        else kloop(T(), F());
    } else {
        if (acopy) kloop(F(), T());
        else kloop(F(), F());
    }

    const int32_t lane = tid_x() & 63;
    // (the ring is idle from here on: the K-split flag may alias its first word)
    if (fd.nsplit > 1 && !split_arrive(ka, fd, acc, w, lane, *reinterpret_cast<int32_t *>(sm.op))) return;

    // epilogue: straight from the accumulators, 32 consecutive columns per row
    TC *Cp = static_cast<TC *>(ka.C);
    const bool accum = (fd.flags & G_ACCUMULATE) != 0;
#pragma unroll
    for (int fj = 0; fj < 2; ++fj) {
        const int32_t j = wn * 64 + fj * 32 + (lane & 31);
        if (j >= nlen) continue;
        TC *col = Cp + fd.c_base + static_cast<int64_t>(j) * fd.c_cs;
#pragma unroll
        for (int fi = 0; fi < FB_FM; ++fi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int32_t i = wm * (FB_BM / 2) + fi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (i >= mlen) continue;
                TC *dst = col + static_cast<int64_t>(i) * fd.c_rs;
                float v = acc[fi][fj][r];
                if (accum) v += static_cast<float>(*dst);
                *dst = static_cast<TC>(v);
            }
    }
}

}  // namespace bsc
