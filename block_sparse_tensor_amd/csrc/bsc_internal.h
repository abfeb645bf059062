// Internal plan representation shared by the host planner and the HIP runtime.
//
// The planner turns the caller's sector lists into a device work list:
//   groups  — one coalesced GEMM each (uni20 "block coalescing": "Coalescing is
//             a plan-time transform" — one node per group plus its scatter map);
//   runs    — maximal stretches of a group's contracted axis over which both
//             operands are single strided views (contraction-axis
//             concatenation that needs no copy);
//   pieces  — strided views that cover a run's operand along the stacked free
//             axis (one piece when the members interleave into one view, one
//             per member otherwise), and the C pieces that scatter results back
//             to their sectors ("Expressed as strided views over shared
//             storage");
//   tasks   — workgroup-sized work items in longest-first order.
// The record layouts below are read verbatim by the device code.
#pragma once

#include <array>
#include <cstdint>
#include <string>
#include <vector>

#include "bsc.h"

namespace bsc {

// A strided two-leg view.  Axis "a" is the piece axis (the stacked free axis
// for A and B pieces, the axis C pieces are cut along), axis "b" the other one.
// Element (x, y), x local to the piece, lives at
//   off + (x/ia)*sa0 + (x%ia)*sa1 + (y/ib)*sb0 + (y%ib)*sb1.
struct DView {
    int64_t off;
    int64_t sa0, sa1;
    int64_t sb0, sb1;
    int32_t ia, ib;
    int32_t begin;   // first group row/column this piece covers along axis a
    int32_t len;     // extent along axis a
};
static_assert(sizeof(DView) == 56, "DView layout");

enum : int32_t {
    G_C_ALONG_N = 1,     // C pieces are cut along columns (else along rows)
    G_ACCUMULATE = 2,    // C += A B (else C = A B)
};

struct DGroup {
    int32_t M, N, K;     // coalesced GEMM extents
    int32_t nrun, run0;  // runs (nrun == 0: zero-fill group)
    int32_t ncp, cp0;    // C pieces
    int32_t flags;
};
static_assert(sizeof(DGroup) == 32, "DGroup layout");

enum : int32_t {
    R_A_KUNIT = 1,       // every A piece: single-leg k axis with stride 1
    R_A_FUNIT = 2,       // every A piece: single-leg free axis with stride 1
    R_B_KUNIT = 4,
    R_B_FUNIT = 8,
    R_A_VEC = 16,        // A: K-unit, every row start 16-byte aligned (16-byte loads along K)
    R_B_VECK = 32,       // B: K-unit, every column start 16-byte aligned
    R_B_VECN = 64,       // B: one N-unit piece, K rows 16-byte aligned, rows readable to a multiple of 8
    R_A_WS = 128,        // A pieces address the pack workspace (a gathered copy), not A
    R_B_WS = 256,        // B pieces address the pack workspace, not B
};

struct DRun {
    int32_t K;           // extent along k
    int32_t nap, ap0;    // A pieces (axis a = M)
    int32_t nbp, bp0;    // B pieces (axis a = N)
    int32_t flags;
    int32_t kbase;       // position of the run along the group's K
    int32_t pad;
};
static_assert(sizeof(DRun) == 32, "DRun layout");

enum : int32_t {
    T_GENERIC = 0,       // workgroup tile, any views, vector ALU
    T_MFMA = 1,          // workgroup tile on the matrix cores
    T_TAIL = 2,          // up to four whole small groups, one per wave
    T_ZERO = 3,          // zero fill of a C tile
    T_MFMA_FAST_N = 4,   // dense matrix-core tile, direct-to-LDS loads, N-contiguous B (group = DFast index)
    T_MFMA_FAST_K = 5,   // dense matrix-core tile, direct-to-LDS loads, K-contiguous B (group = DFast index)
    T_NOP = 6,           // placeholder keeping the task -> XCD mapping (no work)
    T_SKINNY_M = 7,      // at most 16 output columns: 256 R rows x all columns, R rows per thread
    T_SKINNY_N = 8,      // at most 16 output rows: all rows x 256 R columns, R columns per thread
    T_MFMA_DENSE = 9,    // fp32 / fp64 matrix-core tile addressed through a DFast record (group = DFast index)
    T_SKINNY_DENSE_M = 10,   // skinny tile, long axis M, addressed through a DFast record
    T_SKINNY_DENSE_N = 11,   // skinny tile, long axis N, addressed through a DFast record
    T_MFMA_WIDE_N = 12,  // wide dense tile (one workgroup per CU, up to 256 x 256), N-contiguous B (DFast record)
    T_MFMA_WIDE_K = 13,  // wide dense tile, K-contiguous B (DFast record)
    T_NCLASS = 14,
};

// Workgroups of a launch are dispatched round-robin over the chiplets (XCDs),
// each with its own L2: task t of a grouped launch runs on XCD t % BSC_XCDS
// when the grid is a multiple of BSC_XCDS.
constexpr int BSC_XCDS = 8;
// Compute units per XCD on MI355X.  While every workgroup of a launch is
// resident, the k-th workgroup an XCD receives lands on CU k mod
// BSC_CUS_PER_XCD of it (one per CU first, then a second round on the same CUs
// in the same order), so workgroups k and k + BSC_CUS_PER_XCD of an XCD share
// a CU.  The planner uses this only to choose which tiles share a CU.
constexpr int BSC_CUS_PER_XCD = 32;

// kernel feature sets: which tile bodies a grouped launch contains (a plan
// uses either the 256 x 128 direct-to-LDS tiles or the wide ones, never both)
enum : int32_t { FEAT_MFMA = 1, FEAT_FAST_N = 2, FEAT_FAST_K = 4, FEAT_WIDE = 8 };

// Per-tile record of a dense matrix-core tile: the tile's rows of A, columns of
// B and block of C each lie inside one single-leg strided view, so the tile's
// addressing reduces to bases and strides the planner computes once (the
// per-element decode is paid at plan time, not per element or per tile).
// Element addresses (tile-local i, j; run-local k):
//   A(i, k) = a_base + i * a_rs + k * a_ks
//   B(k, j) = b_base + k * b_ks + j * b_ns
//   C(i, j) = c_base + i * c_rs + j * c_cs
struct DFast {
    int64_t a_base, a_rs, a_ks;
    int64_t b_base, b_ks, b_ns;
    int64_t c_base, c_rs, c_cs;
    int32_t mlen, nlen, K, flags;   // flags: G_ACCUMULATE, F_A_WS, F_B_WS
    int32_t group;                  // the tile's group (for the general tile when this one is not compiled in)
    // K split (bf16 direct-to-LDS tile only): the output tile is summed over
    // `nsplit` K-slices, each a task of its own; this record covers slice
    // `split` (its bases and K are the slice's).  Every slice stores its fp32
    // partial tile at part + split * (the tile body's rows x columns: 256 x 128,
    // or for the wide tile 256 x 256, 256 x 128 when nlen <= 128) and counts
    // itself in counter `counter`; the last to arrive adds the partials in
    // slice order and writes C.  nsplit = 1: no split.
    int32_t split, nsplit, counter;
    int64_t part;
};
static_assert(sizeof(DFast) == 112, "DFast layout");
enum : int32_t {
    F_A_WS = 4,          // DFast: A read from the pack workspace
    F_B_WS = 8,          // DFast: B read from the pack workspace
};

// One gather of the pack kernel (uni20 "block coalescing", section
// "Interleaved vs contiguous — the real tradeoff is a copy": members that do not
// line up are copied once into a contiguous operand with a constant leading
// dimension).  `rows` x `cols` elements of a strided source view — axis a = the
// group's free axis, axis b = k — land in the workspace at
//   dst + x * ld + y   (k-major destination, dmode 0)  or
//   dst + y * ld + x   (free-major destination, dmode 1).
struct DPack {
    int64_t off, sa0, sa1, sb0, sb1;   // source view, element (x, y) as in DView
    int64_t dst;                        // workspace element of (0, 0)
    int32_t ia, ib;
    int32_t rows, cols;                 // extents along a and b
    int32_t ld;                         // workspace leading dimension (elements)
    int32_t src;                        // 0: the A buffer, 1: the B buffer
    int32_t dmode;                      // 0: k-major, 1: free-major destination
    int32_t pad;
};
static_assert(sizeof(DPack) == 80, "DPack layout");

// How a gather's pieces are copied: straight along k (source and destination
// both unit-stride along k), straight along the free axis, or through LDS
// (the unit axes differ: read along the source's, written along the
// destination's).
enum : int32_t { PACK_VIA_LDS = 0, PACK_ALONG_K = 1, PACK_ALONG_FREE = 2 };
constexpr int32_t pack_mode(const DPack &d) {
    const bool s_k = d.ib == 1 && (d.sb0 == 1 || d.cols == 1);
    const bool s_f = d.ia == 1 && (d.sa0 == 1 || d.rows == 1);
    return d.dmode == 0 ? (s_k ? PACK_ALONG_K : PACK_VIA_LDS) : (s_f ? PACK_ALONG_FREE : PACK_VIA_LDS);
}
// Piece of a gather one pack task copies, tr rows (free axis) by tc columns
// (k), tc a power of two: up to 4096 elements of at most 64 columns, so thin
// gathers (a few k) still move whole runs of rows per task.  A straight bf16
// gather (the alignment gathers of unpadded bf16 blocks: long lines) takes
// pieces of up to 16384 elements with lines of up to 1024, each lane moving
// several 16-byte vectors per task.  Measured on MI355X: the unpadded bf16
// workload 51.4 -> 48.9-49.4 us per contraction; the same for the fp32
// gathers of the U(1)xU(1) update (short lines) was slower, so fp32 and fp64
// keep the small pieces.
constexpr int PACK_TILE_ELEMS = 4096;
constexpr int PACK_TILE_MAXROWS = 1024;
constexpr int PACK_STRAIGHT_ELEMS = 16384;
constexpr int PACK_LDS_ELEMS = 5120;    // max over tc of tr * (tc + 1)
constexpr bool pack_big(int32_t elem_bytes, int32_t mode) { return elem_bytes == 2 && mode != PACK_VIA_LDS; }
constexpr void pack_tile(int32_t rows, int32_t cols, int32_t mode, bool big, int32_t &tr, int32_t &tc) {
    tc = 1;
    if (big && mode == PACK_ALONG_K) {
        while (tc < cols && tc < 1024) tc *= 2;
        tr = PACK_STRAIGHT_ELEMS / tc;
    } else if (big && mode == PACK_ALONG_FREE) {
        int32_t lr = 1;   // line length along the free axis
        while (lr < rows && lr < 1024) lr *= 2;
        while (tc < cols && tc * lr < PACK_STRAIGHT_ELEMS) tc *= 2;
        tr = PACK_STRAIGHT_ELEMS / tc < 4096 ? PACK_STRAIGHT_ELEMS / tc : 4096;
    } else {
        while (tc < cols && tc < 64) tc *= 2;
        tr = PACK_TILE_ELEMS / tc < PACK_TILE_MAXROWS ? PACK_TILE_ELEMS / tc : PACK_TILE_MAXROWS;
    }
}
// Output tiles in flight at once on MI355X (256 CUs x two resident 256-thread
// workgroups); the planner's cost model divides per-tile costs by it.
constexpr double CONCURRENT_TILES = 512.0;
// Wide tiles: a group whose K chain exceeds this many times one CU's share of
// the launch's chunks is cut into 128-row wide tiles.
constexpr double WIDE_HALF_SHARE = 2.0;

struct DTask {
    int32_t cls;
    int32_t group;       // T_TAIL: first tail entry; group of the tile otherwise
    int32_t m0, n0;      // T_TAIL: m0 = number of tail entries in the bundle
};
static_assert(sizeof(DTask) == 16, "DTask layout");

constexpr int TILE_GENERIC = 64;   // generic tile edge
constexpr int TILE_MFMA = 128;     // bf16 matrix-core tile edge
constexpr int TILE_MFMA_DENSE_M = 256;   // rows of the dense (direct-to-LDS) bf16 tile; 128 columns
constexpr int TILE_MFMA_F = 64;    // fp32 / fp64 matrix-core tile edge
constexpr int TILE_WIDE = 256;     // rows and (at most) columns of the wide bf16 tile

// task classes addressed through a DFast record (task t's record is record t)
constexpr bool is_wide(int32_t cls) { return cls == T_MFMA_WIDE_N || cls == T_MFMA_WIDE_K; }
// bf16 dense tiles with direct-to-LDS copies (256 x 128 or wide)
constexpr bool is_direct(int32_t cls) {
    return cls == T_MFMA_FAST_N || cls == T_MFMA_FAST_K || is_wide(cls);
}
constexpr bool has_record(int32_t cls) {
    return is_direct(cls) || cls == T_MFMA_DENSE || cls == T_SKINNY_DENSE_M || cls == T_SKINNY_DENSE_N;
}
constexpr bool is_mfma(int32_t cls) { return cls == T_MFMA || cls == T_MFMA_DENSE || is_direct(cls); }
constexpr int TILE_SKINNY_SHORT = 16;   // largest short extent of a skinny group
// Slot time a 32-wide K chunk of the register-staged general bf16 tile costs
// beyond the direct-to-LDS tile's, for the alignment gathers (microseconds
// per chunk of a 128 x 128 tile): measured on MI355X on the block-diagonal
// bf16 workload with every row misaligned (64 sectors, 609 general tiles of
// 11,622 chunks in all), whose grouped kernel took 79.5 us on the general
// tile and 30.7 us after gathering every operand into 16-byte rows:
// 48.8 us x 512 concurrent tiles / 11,622 chunks.
constexpr double ALIGN_CHUNK_US = 2.15;
constexpr int32_t ALIGN_CHUNK_K = 32;   // K chunk of the general bf16 tile

// Tail bundles (T_TAIL): up to four whole tiny groups per workgroup, one per
// wave.  A tail group is one run of single views with near-zero flops
// (2 M N K <= TAIL_MAX_FLOPS), at most TAIL_MAX_OUT outputs (TAIL_PER_LANE per
// lane), at most TAIL_MAX_K contracted indices and at most TAIL_LANE_WORK
// multiply-adds per lane (outputs per lane x K / lanes per output); each wave
// stages its group's operands through TAIL_STAGE elements of LDS (accumulation
// type) in K-chunks, addressed through the group's DFast record (bases and
// strides of A, B and C, nsplit = 1).
constexpr int TAIL_MAX_OUT = 256;
constexpr int TAIL_PER_LANE = TAIL_MAX_OUT / 64;
constexpr int TAIL_MAX_K = 512;
constexpr int TAIL_LANE_WORK = 64;
constexpr int TAIL_STAGE = 1024;
constexpr int TAIL_BUNDLE = 4;
constexpr int64_t TAIL_MAX_FLOPS = 1024;
// lanes per output of a tail group with mn outputs (a power of two, lanes * mn <= 64)
constexpr int32_t tail_lanes_host(int32_t mn) {
    int32_t p = 1;
    while (2 * p * mn <= 64) p *= 2;
    return p;
}

// Skinny tile extent along its long axis: 256 threads x R lines, where R times
// the short extent rounded up to 4, 8 or 16 is the accumulator budget per
// thread (32).
inline int32_t skinny_long(bsc_dtype, int32_t short_ext) {
    const int32_t yb = short_ext <= 4 ? 4 : (short_ext <= 8 ? 8 : 16);
    return 256 * (32 / yb);
}

// output tile extents (rows, columns) of a task class for a plan dtype and group shape
inline void tile_extents(bsc_dtype dt, int32_t cls, int32_t M, int32_t N, int32_t &tm, int32_t &tn) {
    if (cls == T_SKINNY_M) {
        tm = skinny_long(dt, N);
        tn = N > 0 ? N : 1;
    } else if (cls == T_SKINNY_N) {
        tm = M > 0 ? M : 1;
        tn = skinny_long(dt, M);
    } else if (cls == T_MFMA_FAST_N || cls == T_MFMA_FAST_K) {
        tm = TILE_MFMA_DENSE_M;
        tn = TILE_MFMA;
    } else if (is_wide(cls)) {
        tm = tn = TILE_WIDE;
    } else {
        tm = tn = is_mfma(cls) ? (dt == BSC_BF16_F32 ? TILE_MFMA : TILE_MFMA_F) : TILE_GENERIC;
    }
}

struct Blk {
    int32_t r, c;
    int64_t off;
    int64_t rs0, rs1, cs0, cs1;
    int32_t ri, ci;      // canonical inner extents of the view (1 = single leg)
};

struct Plan {
    bsc_dtype dtype = BSC_F64;
    bsc_options opt{};
    int32_t axis = BSC_AXIS_AUTO;
    int32_t nq = 1;
    std::vector<int64_t> dm, dk, dn;
    std::vector<Blk> A, B, C;
    int64_t a_elems = 0, b_elems = 0, c_elems = 0;

    std::vector<std::array<int32_t, 3>> triples;  // (m, k, n), sorted by (m, n, k)
    std::vector<int32_t> group_of_triple;
    std::vector<std::array<int32_t, 3>> group_mode;

    std::vector<DGroup> groups;   // work groups first, then zero-fill groups
    int32_t n_work_groups = 0;
    std::vector<DRun> runs;
    std::vector<DView> apieces, bpieces, cpieces;
    std::vector<DTask> tasks;
    std::vector<DFast> fast;      // records of dense matrix-core tiles
    std::vector<DFast> tail;      // tail entries: record of each wave's group (bundles consecutive)
    std::vector<DPack> packs;     // gathers into the pack workspace
    std::vector<DTask> pack_tasks;   // 64 x 64 pieces of the gathers (group = gather index)
    int64_t ws_elems = 0;         // pack workspace size (operand elements)
    int32_t n_counters = 0;       // K-split arrival counters (one per split tile, zero between launches)
    int64_t part_elems = 0;       // K-split partial tiles (fp32 elements)
    int32_t split_tiles = 0;      // output tiles cut along K
    // pack-cost model terms summed over the gathered operands (microseconds)
    double gain_seg_us = 0, gain_pad_us = 0, gain_align_us = 0, pack_cost_us = 0;
    std::vector<std::array<int32_t, 2>> launches;  // per-sector mode: task ranges, one launch each

    // device binding
    void *dev = nullptr;
    size_t dev_bytes = 0;
    size_t off_groups = 0, off_runs = 0, off_ap = 0, off_bp = 0, off_cp = 0, off_tasks = 0, off_fast = 0, off_tail = 0;
    size_t off_packs = 0, off_ptasks = 0, off_ws = 0;   // gathers, their tasks, the workspace
    size_t off_cnt = 0, off_part = 0;                    // K-split counters (in the image), partials
    std::vector<unsigned char> image;   // host copy of the device tables
    int32_t cu_count = 0;
    int32_t grid = 0;
    int32_t features = 0;             // FEAT_* bits over all tasks
    bool only_wide = false;           // every task is a wide tile, a tail bundle or a no-op

    bsc_stats stats{};
};

// host planner (planner.cpp); returns BSC_OK or an error with set_error() called
bsc_status build_plan(Plan &p, const bsc_index *m, const bsc_index *k, const bsc_index *n,
                      const bsc_operand *A, const bsc_operand *B, const bsc_operand *C);

void set_error(const std::string &msg);

}  // namespace bsc
