// Fused two-stage plan: a contraction followed by one whose right operand is
// a sparse matrix of scalars (1 x 1 blocks) applied to the first stage's
// output blocks, computed without materialising the intermediate.
//
// In the R/A/B/C environment update (uni20 "block coalescing", Open questions:
// the "A.Y accumulate" stage) stage 1 forms T1 = E^T A block by block and
// stage 2 forms T2 = T1 W, where every W block is a single matrix element: each
// T2 block is a weighted sum of whole T1 blocks.  The W stage has almost no
// arithmetic (0.4 flop/B) and its cost is the T1 round trip through memory
// (the memory-wall argument of the "Sparse Operator Fusion" page), so the fused
// plan computes every T1 tile where it is needed and adds it, weighted, into
// the T2 tiles it feeds.
//
// Device records (read verbatim by kernels_fused.h):
//   FGroup — one per stage-2 output row key: the M x N shape shared by its
//            outputs and stage-1 blocks, its product and output ranges, and
//            the base of its weight table (one row of nout indices into W per
//            stage-1 block, -1 = no term);
//   FChan  — one stage-1 block product A_p B_p: A_p(i, k) at
//            a_off + i a_rs + k a_ks of the stage-1 A buffer, B_p(k, j) at
//            b_off + k b_ks + j b_ns of the stage-1 B buffer, K contracted.
//            The products of one stage-1 C block are consecutive and carry
//            that block's weight row (wrow); the last of them is flagged;
//   FOut   — one stage-2 output block viewed as M x N: C_o(i, j) at
//            c_off + i c_rs + j c_cs of the stage-2 C buffer;
//   FTask  — one 16 x 16 tile (i0, j0) of one group and the group's outputs
//            oc * no .. oc * no + no - 1 (no = the plan's outputs per task);
//   FPart  — the kernel's per-wave record: one part of one task with
//            everything its wave needs to start (see below).  A task whose
//            group has much work is split into S <= min(4, nblk) parts, part p
//            taking the stage-1 blocks r = p, p + S, ...; the parts of a task
//            sit in consecutive slots of one workgroup (four slots), whose
//            part-0 wave adds the others' partial sums in part order through
//            shared memory;
//   pchans — per group and split S, each part's products as one contiguous
//            list (copies of FChan records), which the part record points to.
// With T1_r the r-th stage-1 block of group g (the sum of its products),
// output o of g receives sum over r of W[widx[g.wbase + r * g.nout + o]] * T1_r
// (terms with index -1 skipped).
#pragma once

#include <cstdint>
#include <vector>

#include "bsc_internal.h"

namespace bsc {

constexpr int FUSED_TILE = 16;      // matrix-core block edge (16 x 16)
// A wave's output tile is TW x TW matrix-core blocks (TW = 1 or 2): with
// TW = 2 a wave loads two rows of A and two columns of B per contracted
// index for four matrix-core operations instead of one of each for one,
// halving the operand loads per flop.  Chosen per plan (fp32 plans whose
// accumulators fit, see fused.cpp).
constexpr int FUSED_MAX_OUT = 16;   // outputs per task (larger groups are split over several tasks)
constexpr int FUSED_KC = 32;        // contracted indices per register chunk (8 matrix-core steps)
// Splitting: a task with more register chunks than a share is split into up to
// min(4, nblk) parts.  The planner takes the smallest share (most splitting)
// whose workgroups fit the device at once, give or take a quarter: FUSED_CUS
// compute units, each holding as many workgroups as the kernel instance's
// register use allows (one wave per SIMD per workgroup).
constexpr int FUSED_CUS = 256;
// A stream plan is preferred over the grouped tiles when no wave's product
// stream is longer than this many register chunks (32 contracted indices
// each); measured on MI355X over 22 f32 / f64 contractions, longer streams
// (long K per C block: 43-52 chunks) ran 10-35 % slower than the grouped
// 64 x 64 tiles, shorter ones up to 4.5x faster.
constexpr int64_t STREAM_MAX_CHUNKS = 32;
constexpr int32_t STREAM_SPLIT_PRODUCTS = 8;   // products from which a stream plan's C block may be split
constexpr int64_t FUSED_WIDE_TASKS = 1024;   // 32 x 32 tiles only with at least this many tasks (4 per CU)
constexpr int FUSED_MIN_PART = 4;
inline int fused_wgs_per_cu(bsc_dtype dt, int no, int tile_blocks) {
    // every workgroup puts one wave on each SIMD, so this is the instance's
    // waves per SIMD as compiled (register counts from the compiler's report)
    if (dt == BSC_F64) return no <= 4 ? 3 : 2;      // 124 / 146 / 176 / 240 VGPRs at 1 / 4 / 8 / 16 outputs
    if (tile_blocks == 2) return 2;                 // 32 x 32 tiles: 120 / 185 VGPRs + 24 accumulation registers
    return no <= 1 ? 7 : no <= 4 ? 5 : (no <= 8 ? 4 : 3);   // 61 / 78 / 96 / 129 VGPRs
}

struct FGroup {
    int32_t M, N;
    int32_t nchan, chan0;           // products (FChan) of the group
    int32_t nout, out0;
    int32_t wbase, flags;           // flags: G_ACCUMULATE, G_FTRANS
    int32_t nblk;                   // stage-1 blocks (weight rows)
    int32_t pad0, pad1, pad2;
};
static_assert(sizeof(FGroup) == 48, "FGroup layout");

struct FChan {
    int64_t a_off, a_rs, a_ks;
    int64_t b_off, b_ks, b_ns;
    int32_t K;
    int16_t wrow, last;             // the block's weight row; last: the block's last product
};
static_assert(sizeof(FChan) == 56, "FChan layout");

struct FOut {
    int64_t c_off, c_rs, c_cs;
};
static_assert(sizeof(FOut) == 24, "FOut layout");

struct FTask {
    int32_t group, i0, j0, oc;
};

// FPart — one part as its wave reads it, in one record: the tile, the group's
// shape and flags, the part's products (in pchans), the task's outputs and
// weight rows, the split, the workgroup's output passes, and the part's first
// product (so the first operand loads wait on this record alone).  Idle
// slots have nparts = 0.
struct FPart {
    int32_t i0, j0, ml, nl;         // tile origin and valid extent
    int32_t M, N, nchan, chan0;     // group shape; the part's products pchans[chan0 ..]
    int32_t no, out0, wbase, wstride;   // outputs outs[out0 + o], weights widx[wbase + r * wstride + o]
    int32_t nblk, flags, part, nparts;
    FChan first;                    // the part's first product
    int32_t npass;                  // output passes of four (the most any slot of the workgroup needs)
    int32_t reduce;                 // some task of the workgroup is split: outputs go through the reduction
};
static_assert(sizeof(FPart) == 128, "FPart layout");

// Lane-held tables: a wave keeps the records of 64 of its part's products
// (one per lane; the next 64 are loaded when the stream reaches them) and up to
// FUSED_WREG x 64 weights in registers.
constexpr int FUSED_LANE_RECS = 64;   // a power of two
constexpr int FUSED_WREG = 4;
constexpr int FUSED_WCAP = 64 * FUSED_WREG;   // stage-1 blocks x outputs per task

// G_FTRANS: the group's outputs run contiguously down their rows (|c_rs| < |c_cs|),
// so the tile is formed transposed and consecutive lanes write consecutive rows.
constexpr int32_t G_FTRANS = 1 << 8;
static_assert(sizeof(FTask) == 16, "FTask layout");

struct FusedPlan {
    bsc_dtype dtype = BSC_F64;
    std::vector<FGroup> groups;
    std::vector<FChan> chans;
    std::vector<FOut> outs;
    std::vector<int32_t> widx;
    std::vector<FTask> tasks;
    std::vector<FPart> parts;       // four per workgroup, the kernel's input
    std::vector<FChan> pchans;      // the parts' product lists
    int64_t a_elems = 0, b_elems = 0, w_elems = 0, c_elems = 0;
    int64_t useful_flops = 0, alg_bytes = 0, stage1_flops = 0;
    int64_t terms = 0;              // nonzero (stage-1 block, output) weights
    int32_t outs_per_task = FUSED_MAX_OUT;   // 4, 8 or 16: the kernel instance
    int32_t tile_blocks = 1;                 // TW: the wave's tile is TW x TW blocks of 16 x 16
    bool stream = false;                     // one contraction, each C block weighted by the plan's own 1
    int64_t longest_chunks = 0;              // register chunks of the longest part
    // device image
    size_t off_groups = 0, off_chans = 0, off_outs = 0, off_widx = 0, off_tasks = 0, off_parts = 0, off_pchans = 0;
    size_t off_ones = 0;                     // the weight 1 of a stream plan, in the plan's type
    std::vector<unsigned char> image;
    void *dev = nullptr;
    int32_t cu_count = 0;
    int64_t launches_issued = 0;
};

}  // namespace bsc
