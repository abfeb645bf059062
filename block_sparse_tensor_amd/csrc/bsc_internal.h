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

#include "../../include/bsc.h"

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
};

struct DTask {
    int32_t cls;
    int32_t group;       // T_TAIL: first tail entry; group of the tile otherwise
    int32_t m0, n0;      // T_TAIL: m0 = number of tail entries in the bundle
};
static_assert(sizeof(DTask) == 16, "DTask layout");

constexpr int TILE_GENERIC = 64;   // generic tile edge
constexpr int TILE_MFMA = 128;     // matrix-core tile edge

inline int32_t tile_m(int32_t cls) { return cls == T_MFMA ? TILE_MFMA : TILE_GENERIC; }
inline int32_t tile_n(int32_t cls) { return cls == T_MFMA ? TILE_MFMA : TILE_GENERIC; }

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
    std::vector<std::array<int32_t, 2>> launches;  // per-sector mode: task ranges, one launch each

    // device binding
    void *dev = nullptr;
    size_t dev_bytes = 0;
    size_t off_groups = 0, off_runs = 0, off_ap = 0, off_bp = 0, off_cp = 0, off_tasks = 0;
    std::vector<unsigned char> image;   // host copy of the device tables
    int32_t cu_count = 0;
    int32_t grid = 0;

    bsc_stats stats{};
};

// host planner (planner.cpp); returns BSC_OK or an error with set_error() called
bsc_status build_plan(Plan &p, const bsc_index *m, const bsc_index *k, const bsc_index *n,
                      const bsc_operand *A, const bsc_operand *B, const bsc_operand *C);

void set_error(const std::string &msg);

}  // namespace bsc
