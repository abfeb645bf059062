// Wide dense matrix-core tile for bf16 inputs / fp32 accumulation: one
// workgroup per CU.  Two forms: four waves (below), and eight waves of
// 128 x 64 (wide8_tile_bf16, a launch of wide tiles only).  The same loop,
// with two row fragments per wave, also computes the 256 x 128 tile's tasks of
// at most 128 rows as 128 x 128 tiles of four 64 x 64 waves (HalfTile).
//
// Same record-addressed groups as the 256 x 128 direct-to-LDS tile
// (kernels_mfma_bf16_fast.h: one run of single strided views, 16-byte aligned
// rows), but the workgroup owns the CU's whole LDS and computes a 256 x 256
// output tile with four waves (one per SIMD), each 128 x 128 as 4 x 4
// v_mfma_f32_32x32x16_bf16 (accumulators in the accumulation registers).  A
// tile of at most 128 columns runs the same loop with 128 x 64 per wave.
//
// Why this shape.  Under full-chip load a chunk's copies take about 2 us to
// land, so what a CU computes per microsecond is the work of the chunks it has
// in flight divided by that latency.  Two 256 x 128 workgroups per CU keep four
// 24 KB chunks (8.4 MFLOP of tile work) in flight; one 256 x 256 workgroup with
// a five-stage ring of 32 KB chunks keeps four (16.8 MFLOP), twice the work per
// byte in flight, and a 128 x 128 wave tile reads half a KB of LDS per MFMA
// instead of 0.75, so one wave per SIMD keeps its matrix core fed (16 MFMAs
// per K-step of 16, 8 to 12 fragment reads).
//
//  * K is cut into chunks of 32; stage = A 256 x 32 + B 32 x 256 (32 KB), five
//    stages (160 KB); with 128 columns, 24 KB stages, six of them;
//  * copies, swizzles, the partial last chunk and the transposing reads of an
//    N-contiguous B are those of the 256 x 128 tile, with B rows twice as long
//    (512-byte [k][n] rows: 32 slots of 16 bytes, the 64-byte granules
//    swizzled by k as before);
//  * the K loop is software-pipelined as in the 256 x 128 tile: the fragment
//    reads of the next K-step go out between the MFMAs of this one, and the
//    chunk hand-over (wait for this wave's copies, barrier, refill) sits after
//    the first MFMAs of a chunk's second K-step;
//  * results go straight from the accumulators to C; a K-split tile stores its
//    partial tile and the last slice adds the partials in slice order (as the
//    256 x 128 tile does).
#pragma once

#include <type_traits>

#include "kernels_mfma_bf16_fast.h"

namespace bsc {

constexpr int WB_RING_ELEMS = 81920;   // 160 KB: the CU's whole LDS

// Geometry of a direct-to-LDS tile computed by NW waves in a 2 x (NW / 2)
// arrangement, each wave 32 FM rows by WN columns (FM row and WN / 32 column
// fragments of 32 x 32), with a ring of RING bf16 elements.  The wide tile:
// FM = 4 (256 rows), WN = 128 or 64, NW = 4 or 8, the CU's whole LDS.  The
// 128 x 128 tile of four 64 x 64 waves: FM = 2, in the 80 KB ring of the
// 256 x 128 tile's launch (kernels_mfma_bf16_fast.h).  The copies of a chunk
// are shared out over the NW waves.
template <int WN, int NW = 4, int FM = 4, int RING = WB_RING_ELEMS>
struct Wide {
    static constexpr int WC = WN;                       // columns per wave
    static constexpr int NWV = NW;                      // waves
    static constexpr int FR = FM;                       // row fragments per wave
    static constexpr int TM = 2 * 32 * FM;              // tile rows
    static constexpr int NT = 64 * NW;                  // threads
    static constexpr int BN = (NW / 2) * WN;            // tile columns
    static constexpr int FN = WN / 32;                  // column fragments per wave
    static constexpr int A_ELEMS = TM * FB_BK;          // A part of a stage
    static constexpr int B_ELEMS = BN * FB_BK;          // B part of a stage
    static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
    static constexpr int STAGES = RING / STAGE_ELEMS < 6 ? RING / STAGE_ELEMS : 6;
    static constexpr int NIA = A_ELEMS * 2 / 1024 / NW;   // 1 KB copies of A per wave and chunk
    static constexpr int NIB = B_ELEMS * 2 / 1024 / NW;   // of B
    static constexpr int SLOTS = BN * 2 / 16;            // 16-byte slots per N-contiguous B row
    static constexpr int ROWS_PER = 64 / SLOTS;          // B k-rows one copy instruction fills
    // the first MFMAs of a K-step before its reads of the next one go out
    static constexpr int PRE = FM * (WN / 32) >= 8 ? 2 : 1;
    static_assert(STAGES * STAGE_ELEMS <= RING && STAGES >= 3, "ring fits the LDS");
    static_assert(FN * 32 == WN && (WN == 128 || WN == 64), "wave tile width");
    static_assert((FM == 4 || FM == 2) && NIA >= 1 && NIB >= 1, "tile shape");
};
static_assert(Wide<128>::STAGES == 5 && Wide<64>::STAGES == 6, "ring depths");
using HalfTile = Wide<64, 4, 2, FB_RING_ELEMS>;   // 128 x 128, four 64 x 64 waves, 80 KB ring
static_assert(HalfTile::STAGES == 5, "four chunks of copies in flight");

struct WideSmemBf16 {
    uint16_t op[WB_RING_ELEMS];
};

// Wait until this wave's copies of the chunk with `after` newer chunks in flight
// have landed (PER copies per chunk and wave).
template <int PER>
__device__ __forceinline__ void wide_wait_chunks(int32_t after) {
    switch (after) {
        case 0: wait_vm<0>(); break;
        case 1: wait_vm<PER>(); break;
        case 2: wait_vm<2 * PER>(); break;
        case 3: wait_vm<3 * PER>(); break;
        default: wait_vm<4 * PER>(); break;
    }
}
static_assert(4 * (Wide<128>::NIA + Wide<128>::NIB) < 64 && 4 * (Wide<64>::NIA + Wide<64>::NIB) < 64,
              "vmcnt range: at most four newer chunks");

// N-contiguous B operand ([k][n] layout, element (k, n) at base + k * ks + n)
// into BN-wide LDS rows: instruction j fills k rows ROWS_PER (NI w + j) ..;
// lane l fills row l / SLOTS, 16-byte slot l % SLOTS, i.e. 64-byte position
// (l % SLOTS) / 4, which holds n-granule position ^ (k & 3).
template <typename G, int NI>
__device__ __forceinline__ FastOp<NI> wide_setup_ncontig(int64_t base, int64_t ks, int32_t nlen, int32_t K,
                                                         const uint16_t *P, int32_t w) {
    FastOp<NI> f;
    const int32_t lane = tid_x() & 63;
    const int32_t s = lane % G::SLOTS;
    f.rs = wave_rsrc(P + base, 2 * (static_cast<int64_t>(K - 1) * ks + G::BN) + 16);
#pragma unroll
    for (int j = 0; j < NI; ++j) {
        const int32_t kr = G::ROWS_PER * (NI * w + j) + lane / G::SLOTS;
        int32_t n = 32 * fb_pos(kr, s >> 2) + 8 * (s & 3);
        if (n >= nlen) n = 0;                                      // columns past the edge: a valid column
        f.off[j] = static_cast<uint32_t>(2 * (n + static_cast<int64_t>(kr) * ks));
    }
    f.step = static_cast<uint32_t>(2 * FB_BK * ks);
    return f;
}

// Masked fill of a partial chunk (k0 .. K-1 valid) of an N-contiguous B into BN-wide rows.
template <typename G>
__device__ __forceinline__ void wide_fill_ncontig(int64_t base, int64_t ks, int32_t nlen, int32_t k0, int32_t K,
                                                  const uint16_t *P, uint16_t *lds) {
    const int32_t tid = tid_x();
#pragma unroll 1
    for (int q = 0; q < FB_BK * G::SLOTS / G::NT; ++q) {
        const int32_t u = tid + G::NT * q;         // k row u / SLOTS, 8-column piece u % SLOTS
        const int32_t kr = u / G::SLOTS, s = u % G::SLOTS;
        const int32_t n = 8 * s, k = k0 + kr;
        uint16_t e[8];
        const uint16_t *row = P + base + static_cast<int64_t>(k) * ks;
#pragma unroll
        for (int t = 0; t < 8; ++t) e[t] = (k < K && n + t < nlen) ? row[n + t] : uint16_t(0);
        *reinterpret_cast<uint4 *>(lds + kr * G::BN + 32 * fb_pos(kr, n >> 5) + 8 * ((n >> 3) & 3)) = u4_from(e);
    }
}

// Per-lane byte offsets of a wave's fragment reads within a stage.  A as in
// the 256 x 128 tile (rows wm * 128 + 32 f + lane % 32, k-granule
// 2 ks + lane / 32; the next K-step flips bit 5).  N-contiguous B: lane
// (hh, p) reads k rows 16 ks + 8 (hh / 2) + p / 4 (+4 for the second half),
// columns wn * WN + 32 f + 16 (hh % 2) + 4 (p % 4); column fragment f lies in
// 64-byte position (4 wn + f) ^ (k & 3) (for WN = 64: (2 wn + f) ^ (k & 3)),
// so fragment f is fragment 0 with f * 64 XORed into the address.  K-contiguous
// B: like A with rows wn * WN + 32 f + lane % 32.
struct WideOff {
    uint32_t a[2];   // A, by K-step
    uint32_t b[4];   // K-contiguous B: by K-step (b[0], b[1]); N-contiguous B: by column fragment
};

template <typename G, bool BN>
__device__ __forceinline__ WideOff wide_offsets() {
    constexpr int WN = G::WC;
    const int32_t lane = tid_x() & 63, w = tid_x() >> 6;
    const int32_t wm = w & 1, wn = w >> 1;
    WideOff o;
    const int32_t ra = wm * (G::TM / 2) + (lane & 31);
    o.a[0] = 2 * (ra * FB_BK + 8 * fa_slot(ra, lane >> 5));
    o.a[1] = o.a[0] ^ 32;
    if constexpr (BN) {
        const int32_t hh = lane >> 4, p = lane & 15;
        const int32_t k = 8 * (hh >> 1) + (p >> 2);
        const int32_t n = wn * WN + 16 * (hh & 1) + 4 * (p & 3);
        o.b[0] = 2 * (k * G::BN + 32 * fb_pos(k, n >> 5) + (n & 31));
        // fragment f: 64-byte position (G + f) ^ (k & 3) with G a multiple of FN
#pragma unroll
        for (int f = 1; f < 4; ++f) o.b[f] = f < G::FN ? (o.b[0] ^ static_cast<uint32_t>(64 * f)) : o.b[0];
    } else {
        const int32_t rb = wn * WN + (lane & 31);
        o.b[0] = 2 * (rb * FB_BK + 8 * fa_slot(rb, lane >> 5));
        o.b[1] = o.b[0] ^ 32;
        o.b[2] = o.b[3] = 0;
    }
    return o;
}

// 16-byte fragment read i (0..3) at byte offset i * STEP from ad (the immediate
// offset field); i is a constant once the callers' loops are unrolled.
template <int STEP>
__device__ __forceinline__ void lds_read_b128_at(int i, uint32_t ad, v4i32_t &r) {
    switch (i) {
        case 0: lds_read_b128<0>(ad, r); break;
        case 1: lds_read_b128<STEP>(ad, r); break;
        case 2: lds_read_b128<2 * STEP>(ad, r); break;
        default: lds_read_b128<3 * STEP>(ad, r); break;
    }
}

template <typename G>
struct WideFrags {
    v4i32_t a[G::FR];
    v4i32_t b[G::FN];        // K-contiguous B
    v4i16_t t[2 * G::FN];    // N-contiguous B: transposed halves
};

// Fragment read r of a K-step (B reads first, then A).  va: the stage's A base
// plus this wave's A offset for the K-step; vb: K-contiguous B: the stage's B
// base plus the B offset of the K-step; N-contiguous B: the stage's B base,
// to which each fragment adds its own lane offset o.b[f].
template <typename G, bool BN, int KS>
__device__ __forceinline__ void wide_read_one(int r, uint32_t va, uint32_t vb, const WideOff &o, WideFrags<G> &fr) {
    constexpr int FN = G::FN;
    constexpr int AR = 2 * 32 * FB_BK;               // bytes between row fragments
    if constexpr (BN) {
        constexpr int KO = 2 * 16 * KS * G::BN, HO = 2 * 4 * G::BN;
        if (r < 2 * FN) {
#pragma unroll
            for (int ff = 0; ff < FN; ++ff) {
                if (ff != (r >> 1)) continue;
                const uint32_t ad = vb + o.b[ff];
                if (r & 1) lds_read_tr<KO + HO>(ad, fr.t[2 * ff + 1]);
                else lds_read_tr<KO>(ad, fr.t[2 * ff]);
            }
            return;
        }
    } else {
        if (r < FN) {
#pragma unroll
            for (int ff = 0; ff < FN; ++ff)
                if (ff == r) lds_read_b128_at<AR>(ff, vb, fr.b[ff]);
            return;
        }
    }
    const int ra = r - (BN ? 2 * FN : FN);
#pragma unroll
    for (int fi = 0; fi < G::FR; ++fi)
        if (fi == ra) lds_read_b128_at<AR>(fi, va, fr.a[fi]);
}

template <typename G, bool BN>
constexpr int wide_reads() { return (BN ? 2 * G::FN : G::FN) + G::FR; }

template <typename G, bool BN, int KS>
__device__ __forceinline__ void wide_read_all(uint32_t va, uint32_t vb, const WideOff &o, WideFrags<G> &fr) {
#pragma unroll
    for (int r = 0; r < wide_reads<G, BN>(); ++r) wide_read_one<G, BN, KS>(r, va, vb, o, fr);
}

template <typename G, bool BN>
__device__ __forceinline__ void wide_wait(WideFrags<G> &fr) {
    // every fragment register is an output, so no use moves above the wait
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int f = 0; f < G::FR; ++f) asm volatile("" : "+v"(fr.a[f]));
    if constexpr (BN) {
#pragma unroll
        for (int f = 0; f < 2 * G::FN; ++f) asm volatile("" : "+v"(fr.t[f]));
    } else {
#pragma unroll
        for (int f = 0; f < G::FN; ++f) asm volatile("" : "+v"(fr.b[f]));
    }
}

template <typename G, bool BN>
__device__ __forceinline__ bf16x8_t wide_bfrag(const WideFrags<G> &fr, int f) {
    if constexpr (BN) {
        const v4i16_t lo = fr.t[2 * f], hi = fr.t[2 * f + 1];
        short e8 __attribute__((ext_vector_type(8))) = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(bf16x8_t, e8);
    } else {
        return __builtin_bit_cast(bf16x8_t, fr.b[f]);
    }
}

// The MFMAs of one K-step (fragments `cur`, FM x FN of them) with the reads of
// the next K-step's fragments (`nxt`, K-step KS at bases va, vb) issued between
// them after the first PRE MFMAs; `mid` runs right before MFMA PRE.
template <typename G, bool BN, int KS, int PRE, typename Mid>
__device__ __forceinline__ void wide_mfma_interleaved(const WideFrags<G> &cur, WideFrags<G> &nxt,
                                                      uint32_t va, uint32_t vb, const WideOff &o,
                                                      f32x16_t (&acc)[G::FR][G::FN], Mid &&mid) {
    constexpr int FN = G::FN, FM = G::FR;
    constexpr int NM = FM * FN;                    // MFMAs per K-step
    constexpr int NR = wide_reads<G, BN>();        // reads per K-step
    static_assert(PRE + (NR + 1) / 2 <= NM, "every read issued within the K-step");
    bf16x8_t fa[FM], fb[FN];
#pragma unroll
    for (int f = 0; f < FM; ++f) fa[f] = __builtin_bit_cast(bf16x8_t, cur.a[f]);
#pragma unroll
    for (int f = 0; f < FN; ++f) fb[f] = wide_bfrag<G, BN>(cur, f);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NM; ++k) {
        if (k == PRE) {
            mid();
            __builtin_amdgcn_sched_barrier(0);
        }
        acc[k / FN][k % FN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k / FN], fb[k % FN], acc[k / FN][k % FN], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (k >= PRE) {
            // two reads after each MFMA from PRE on: with one wave per SIMD nothing
            // else hides a read still in flight when the next K-step starts, so
            // the reads go out early (all of them within the first
            // PRE + NR / 2 MFMAs of the NM)
            const int slot = k - PRE;
#pragma unroll
            for (int r = 0; r < NR; ++r)
                if (r >= 2 * slot && r < 2 * slot + 2) wide_read_one<G, BN, KS>(r, va, vb, o, nxt);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // keep `cur` allocated until every read into `nxt` is issued
#pragma unroll
    for (int f = 0; f < FM; ++f) asm volatile("" ::"v"(cur.a[f]));
    if constexpr (BN) {
#pragma unroll
        for (int f = 0; f < 2 * FN; ++f) asm volatile("" ::"v"(cur.t[f]));
    } else {
#pragma unroll
        for (int f = 0; f < FN; ++f) asm volatile("" ::"v"(cur.b[f]));
    }
}

// MFMAs of one K-step without interleaved reads.
template <typename G, bool BN>
__device__ __forceinline__ void wide_mfma(const WideFrags<G> &fr, f32x16_t (&acc)[G::FR][G::FN]) {
    constexpr int FN = G::FN, FM = G::FR;
    bf16x8_t fa[FM], fb[FN];
#pragma unroll
    for (int f = 0; f < FM; ++f) fa[f] = __builtin_bit_cast(bf16x8_t, fr.a[f]);
#pragma unroll
    for (int f = 0; f < FN; ++f) fb[f] = wide_bfrag<G, BN>(fr, f);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// K split of a wide tile (see split_arrive of the 256 x 128 tile): store this
// slice's partial tile lane-contiguously, count the slice in the tile's
// counter, and let the last slice reload the accumulators as the partials'
// sum in slice order.
template <typename G>
__device__ __forceinline__ bool wide_split_arrive(const KArgs &ka, const DFast &fd, f32x16_t (&acc)[G::FR][G::FN],
                                                  int32_t w, int32_t lane, int32_t &last) {
    constexpr int FN = G::FN;
    constexpr int SPLIT_BYTES = G::TM * G::BN * 4;    // one partial tile
    constexpr int NQ = G::FR * FN * 4;                // 16-byte groups per lane
    const uint64_t base = reinterpret_cast<uint64_t>(ka.P + fd.part);
    const uint64_t ubase = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(base >> 32))) << 32) |
                           static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int32_t>(base)));
    const int32_t nsplit = __builtin_amdgcn_readfirstlane(fd.nsplit);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(ubase), 0, nsplit * SPLIT_BYTES, BUF_DWORD3);
    const int32_t lane_off = (w * NQ * 64 + lane) * 16;
    const int32_t mine = fd.split * SPLIT_BYTES + lane_off;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const f32x16_t &a = acc[q / (4 * FN)][(q / 4) % FN];
        const int r = 4 * (q & 3);
        const f32x4_t v = {a[r], a[r + 1], a[r + 2], a[r + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i32_t, v), rs, mine + q * 1024, 0, CPOL_SC1);
    }
    wait_vm<0>();
    __syncthreads();
    if (tid_x() == 0) {
        const int32_t before = __hip_atomic_fetch_add(ka.cnt + fd.counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last = before == fd.nsplit - 1;
        if (last) __hip_atomic_store(ka.cnt + fd.counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!last) return false;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        f32x16_t &a = acc[q / (4 * FN)][(q / 4) % FN];
        const int r = 4 * (q & 3);
        const f32x4_t x = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, lane_off + q * 1024, 0, CPOL_SC1));
#pragma unroll
        for (int e = 0; e < 4; ++e) a[r + e] = x[e];
    }
    constexpr int BATCH = 16;
    for (int32_t s = 1; s < nsplit; ++s) {
        const int32_t src = s * SPLIT_BYTES + lane_off;
#pragma unroll
        for (int h = 0; h < NQ; h += BATCH) {
            v4i32_t t[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) t[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, src + (h + u) * 1024, 0, CPOL_SC1);
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const int q = h + u;
                f32x16_t &a = acc[q / (4 * FN)][(q / 4) % FN];
                const int r = 4 * (q & 3);
                const f32x4_t x = __builtin_bit_cast(f32x4_t, t[u]);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[r + e] += x[e];
            }
        }
    }
    return true;
}

// ring_lds: the LDS ring (G::STAGES stages of G::STAGE_ELEMS elements)
template <typename TC, bool BN, typename G>
__device__ __forceinline__ void wide_tile_body(const KArgs &ka, const DFast &fd, uint16_t *ring_lds) {
    constexpr int FN = G::FN, FM = G::FR, WN = G::WC, NW = G::NWV;
    const uint16_t *A = static_cast<const uint16_t *>((fd.flags & F_A_WS) ? ka.W : ka.A);
    const uint16_t *B = static_cast<const uint16_t *>((fd.flags & F_B_WS) ? ka.W : ka.B);
    const int32_t mlen = fd.mlen, nlen = fd.nlen, K = fd.K;
    const int32_t w = __builtin_amdgcn_readfirstlane(tid_x() >> 6);

    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Wave (wm, wn) computes rows wm*TM/2 .. +TM/2 and columns wn*WN .. +WN and
    // copies A rows TM/NW w .. +TM/NW; a wave whose rows (or columns) lie wholly past
    // the tile edge computes nothing, one whose A rows do copies no A.  Every
    // wave copies its share of B.  Roles are wave-uniform; all waves meet at
    // the same barriers.
    const int32_t wm = w & 1, wn = w >> 1;
    const bool compute = wm * (G::TM / 2) < mlen && wn * WN < nlen;
    const bool acopy = (G::TM / NW) * w < mlen;
    const FastOp<G::NIA> fa = dense_setup_kcontig<G::NIA>(fd.a_base, fd.a_rs, mlen, K, A, w);
    FastOp<G::NIB> fb;
    if constexpr (BN) fb = wide_setup_ncontig<G, G::NIB>(fd.b_base, fd.b_ks, nlen, K, B, w);
    else fb = dense_setup_kcontig<G::NIB>(fd.b_base, fd.b_ns, nlen, K, B, w);
    const int64_t b_s = BN ? fd.b_ks : fd.b_ns;
    const int32_t nfull = K / FB_BK;
    const int32_t ntot = (K + FB_BK - 1) / FB_BK;
    const WideOff fo = wide_offsets<G, BN>();
    wait_vm<0>();      // nothing else outstanding: the counted waits below see only this tile's copies
    __syncthreads();   // previous users of the LDS ring are done

    auto kloop = [&](auto compute_c, auto acopy_c) {
        constexpr bool COMPUTE = decltype(compute_c)::value, ACOPY = decltype(acopy_c)::value;
        constexpr int STAGES = G::STAGES;
        constexpr int PER = (ACOPY ? G::NIA : 0) + G::NIB;   // copies per chunk and wave
        uint16_t *const ops = ring_lds;
        auto fill_partial = [&](int32_t stage) {
            uint16_t *at = ops + stage * G::STAGE_ELEMS;
            dense_fill_kcontig<G::TM, G::NT>(fd.a_base, fd.a_rs, mlen, nfull * FB_BK, K, A, at);
            if constexpr (BN) wide_fill_ncontig<G>(fd.b_base, b_s, nlen, nfull * FB_BK, K, B, at + G::A_ELEMS);
            else dense_fill_kcontig<G::BN, G::NT>(fd.b_base, b_s, nlen, nfull * FB_BK, K, B, at + G::A_ELEMS);
        };
        auto issue = [&](int32_t c, int32_t stage) {
            uint16_t *at = ops + stage * G::STAGE_ELEMS;
            if constexpr (ACOPY) fast_issue<G::NIA>(fa, c, at, w);
            fast_issue<G::NIB>(fb, c, at + G::A_ELEMS, w);
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
        auto advance = [&](int32_t cn) {
            if (cn < nfull) wide_wait_chunks<PER>(issued - cn - 1);
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
        constexpr uint32_t STAGE_BYTES = G::STAGE_ELEMS * 2, B_OFF = G::A_ELEMS * 2;
        auto stage_addr = [&](int32_t c) { return ring + (c % STAGES) * STAGE_BYTES; };
        WideFrags<G> s0, s1;
        // B base of a stage for K-step ks: N-contiguous B adds per-fragment offsets later
        auto bbase = [&](uint32_t stage, int ks) { return stage + B_OFF + (BN ? 0u : fo.b[ks]); };
        auto reads0 = [&](uint32_t stage, WideFrags<G> &fr) {
            if constexpr (COMPUTE) wide_read_all<G, BN, 0>(stage + fo.a[0], bbase(stage, 0), fo, fr);
        };
        auto reads1 = [&](uint32_t stage, WideFrags<G> &fr) {
            if constexpr (COMPUTE) wide_read_all<G, BN, 1>(stage + fo.a[1], bbase(stage, 1), fo, fr);
        };
        auto mfmas = [&](const WideFrags<G> &fr) {
            if constexpr (COMPUTE) {
                __builtin_amdgcn_sched_barrier(0);
                wide_mfma<G, BN>(fr, acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        auto settle = [&](WideFrags<G> &fr) {
            if constexpr (COMPUTE) wide_wait<G, BN>(fr);
        };
        advance(0);
        reads0(stage_addr(0), s0);
        settle(s0);
        // steady state, without branches (as in the 256 x 128 tile)
        int32_t c = 0, st = 0;
        const int32_t nsteady = nfull - STAGES;
        for (; c < nsteady; ++c) {
            const int32_t sn = st == STAGES - 1 ? 0 : st + 1;
            if constexpr (COMPUTE) {
                const uint32_t here = ring + st * STAGE_BYTES, next = ring + sn * STAGE_BYTES;
                wide_mfma_interleaved<G, BN, 1, G::PRE>(s0, s1, here + fo.a[1], bbase(here, 1), fo, acc, [] {});
                settle(s1);
                wide_mfma_interleaved<G, BN, 0, G::PRE>(s1, s0, next + fo.a[0], bbase(next, 0), fo, acc, [&] {
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
        issued = c + STAGES < nfull ? c + STAGES : nfull;
        for (; c < ntot; ++c) {
            reads1(stage_addr(c), s1);
            mfmas(s0);
            settle(s1);
            const bool more = c + 1 < ntot;
            if (more) {
                advance(c + 1);
                reads0(stage_addr(c + 1), s0);
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
    if (fd.nsplit > 1 && !wide_split_arrive<G>(ka, fd, acc, w, lane, *reinterpret_cast<int32_t *>(ring_lds))) return;

    // epilogue: straight from the accumulators, 32 consecutive columns per row
    TC *Cp = static_cast<TC *>(ka.C);
    const bool accum = (fd.flags & G_ACCUMULATE) != 0;
#pragma unroll
    for (int fj = 0; fj < FN; ++fj) {
        const int32_t j = wn * WN + fj * 32 + (lane & 31);
        if (j >= nlen) continue;
        TC *col = Cp + fd.c_base + static_cast<int64_t>(j) * fd.c_cs;
#pragma unroll
        for (int fi = 0; fi < FM; ++fi)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int32_t i = wm * (G::TM / 2) + fi * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
                if (i >= mlen) continue;
                TC *dst = col + static_cast<int64_t>(i) * fd.c_rs;
                float v = acc[fi][fj][r];
                if (accum) v += static_cast<float>(*dst);
                *dst = static_cast<TC>(v);
            }
    }
}

// A wide tile: the 128 x 128 wave tile when the tile has more than 128
// columns, else the 128 x 64 one.
template <typename TC, bool BN>
__device__ __forceinline__ void wide_tile_bf16(const KArgs &ka, const DFast &fd_ref, WideSmemBf16 &sm) {
    const DFast fd = fd_ref;   // one read of the record
    if (fd.nlen > 128) wide_tile_body<TC, BN, Wide<128>>(ka, fd, sm.op);
    else wide_tile_body<TC, BN, Wide<64>>(ka, fd, sm.op);
}

// The same tile on eight waves (a 512-thread workgroup, two waves per SIMD):
// 2 x 4 waves of 128 x 64, so one wave's fragment reads overlap the other's
// MFMAs on every SIMD, which four waves of 128 x 128 cannot do.  A tile of at
// most 128 columns runs the same loop; the waves whose columns lie past its
// edge copy their share of B (clamped to a valid column) and compute nothing.
// A tile of at most 128 rows (the planner's cut of long-K groups) runs as
// 128 x 256 with 2 x 4 waves of 64 x 64: half the K chain's work per chunk.
template <typename TC, bool BN>
__device__ __forceinline__ void wide8_tile_bf16(const KArgs &ka, const DFast &fd_ref, WideSmemBf16 &sm) {
    const DFast fd = fd_ref;
    if (fd.mlen <= 128) wide_tile_body<TC, BN, Wide<64, 8, 2>>(ka, fd, sm.op);
    else wide_tile_body<TC, BN, Wide<64, 8>>(ka, fd, sm.op);
}

}  // namespace bsc
