/*
 * bsc.h — block-sparse contraction engine for AMD Instinct MI355X (gfx950).
 *
 * Computes the block GEMM over symmetry sectors
 *
 *     C[m,n] = sum_k A[m,k] * B[k,n]
 *
 * where every index is a list of keys (sectors) and every operand is a list of
 * blocks, each a strided view into one flat device buffer.  This is the
 * contraction of the uni20 design note "block coalescing" (section "Why
 * single-axis coalescing is hole-free").  The planner groups the per-sector
 * GEMMs along ONE axis only — stacking output blocks that share the other
 * output key and the contracted-key list (free-axis grouping), or
 * concatenating the contracted keys of one output block (contraction-axis
 * grouping) — so the coalesced operands have no structural zeros (same
 * section).  Each block keeps its sector identity through its own
 * (offset, stride) view (section "Expressed as strided views over shared
 * storage"), and grouping happens once, at plan time (section "Coalescing is a
 * plan-time transform").  A contraction then runs as one persistent
 * grouped-GEMM launch, plus one gather launch when some group is packed
 * (section "Interleaved vs contiguous — the real tradeoff is a copy").
 *
 * Conventions
 * -----------
 * Charges.  Key r of an index carries an integer charge vector of length nq
 * (1 for U(1), 2 for U(1)xU(1)).  A block (r, c) of operand X may exist only if
 * q_row(r) - q_col(c) == flux_X componentwise, and flux_C must equal
 * flux_A + flux_B.
 *
 * Views.  A key may be a fused pair of legs: dim = outer * inner.  Element
 * (r, c) of a block lives at buffer element
 *     offset + (r / Ri)*rs[0] + (r % Ri)*rs[1] + (c / Ci)*cs[0] + (c % Ci)*cs[1]
 * with Ri, Ci the inner extents of the row and column keys (1 when `inner` is
 * NULL).  Strides are in elements; a leg of extent > 1 needs a stride >= 1,
 * the stride of a unit leg is ignored.  C blocks must not overlap; A and B
 * blocks may.
 *
 * Semantics.  Overwrite mode (default): every listed C block receives
 * sum over k of A[m,k] B[k,n], or zeros if no k contributes.  Accumulate mode
 * adds to what C holds.  Elements of C's buffer outside every listed C block
 * are never written.  A product sector (m, n) absent from C's block list is an
 * error (BSC_ERR_MISSING_OUTPUT).
 *
 * Types.  BSC_F64: A, B, C double.  BSC_F32: A, B, C float.  BSC_BF16_F32:
 * A, B bfloat16 (16-bit patterns), accumulation and C in float.
 *
 * Ownership.  bsc_plan copies every descriptor array; the caller may free them
 * on return.  A plan owns host memory only.  All device memory — A, B, C and
 * the plan's device region (work list + pack workspace) — belongs to the
 * caller and must outlive every contraction enqueued on it.
 *
 * Streams.  `stream` arguments are hipStream_t values passed as void*
 * (NULL = the null stream).  bsc_contract enqueues its launches and returns
 * without synchronising.  The pack workspace lives in the plan's device
 * region, so one plan must not run on two streams at once.
 *
 * Errors.  Every call returns a bsc_status; nothing throws or aborts across
 * this interface.  bsc_last_error() gives a thread-local message for the last
 * failing call.
 */
#ifndef BSC_H
#define BSC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    BSC_OK = 0,
    BSC_ERR_ARG = -1,            /* NULL pointer, bad enum, size mismatch, unbound plan buffers */
    BSC_ERR_CHARGE = -2,         /* a block breaks the charge rule, or flux_C != flux_A + flux_B */
    BSC_ERR_SHAPE = -3,          /* bad dim / inner extent / stride, duplicate block, key out of range */
    BSC_ERR_BOUNDS = -4,         /* a block reaches outside its buffer, or a negative offset */
    BSC_ERR_OVERLAP = -5,        /* two C elements share a buffer element */
    BSC_ERR_MISSING_OUTPUT = -6, /* a product sector (m,n) has no C block */
    BSC_ERR_UNSUPPORTED = -7,    /* sizes beyond the engine's 32-bit tile indexing, or no device */
    BSC_ERR_NOT_BOUND = -8,      /* bsc_contract before bsc_plan_bind */
    BSC_ERR_DEVICE_BYTES = -9,   /* the device region passed to bind is too small */
    BSC_ERR_HIP = -10            /* a HIP runtime call failed (detail in bsc_last_error) */
} bsc_status;

typedef enum { BSC_F64 = 0, BSC_F32 = 1, BSC_BF16_F32 = 2 } bsc_dtype;

/* Coalescing axis.  NONE = one group per sector GEMM (only meaningful with the
 * per-sector launch mode).  FREE_M: stack output blocks sharing n and the
 * contracted-key list along M.  FREE_N: the same along N.  CONTRACT: one group
 * per output block, contracted keys concatenated along K.  AUTO: CONTRACT if
 * more than a quarter of the non-empty output blocks sum over more than one k,
 * else whichever free axis yields fewer groups (FREE_M on a tie). */
typedef enum {
    BSC_AXIS_NONE = 0, BSC_AXIS_FREE_M = 1, BSC_AXIS_FREE_N = 2,
    BSC_AXIS_CONTRACT = 3, BSC_AXIS_AUTO = 4
} bsc_axis;

typedef enum { BSC_LAUNCH_GROUPED = 0, BSC_LAUNCH_PER_SECTOR = 1 } bsc_launch_mode;

/* Operand arrangement policy per group.  AUTO: the cost model decides between
 * the zero-copy arrangement (VIEW when the members form one strided view,
 * else SEGMENTS: per-member views walked inside the work item) and PACK (a
 * gather into contiguous workspace).  NEVER_PACK and FORCE_PACK pin it. */
typedef enum { BSC_LAYOUT_AUTO = 0, BSC_LAYOUT_NEVER_PACK = 1, BSC_LAYOUT_FORCE_PACK = 2 } bsc_layout_policy;

/* Arrangement of one operand of one group, as reported by bsc_plan_export. */
typedef enum { BSC_MODE_VIEW = 0, BSC_MODE_PACK = 1, BSC_MODE_SEGMENTS = 2 } bsc_mode;

typedef struct {
    int32_t nkeys;          /* number of keys (>= 0) */
    int32_t nq;             /* charge components per key (>= 1, equal for m, k, n) */
    const int32_t *charge;  /* [nkeys * nq], key-major */
    const int64_t *dim;     /* [nkeys], >= 1 */
    const int64_t *inner;   /* [nkeys] inner-leg extents (>= 1, dividing dim), or NULL */
} bsc_index;

typedef struct {
    int64_t nblocks;
    const int32_t *row_key;    /* [nblocks] */
    const int32_t *col_key;    /* [nblocks] */
    const int64_t *offset;     /* [nblocks] first element, in elements */
    const int64_t *row_stride; /* [2 * nblocks]: outer, inner leg of the row key */
    const int64_t *col_stride; /* [2 * nblocks]: outer, inner leg of the column key */
    const int32_t *flux;       /* [nq] */
    int64_t buffer_elems;      /* elements in the operand's flat buffer */
} bsc_operand;

typedef struct {
    int32_t launch_mode;    /* bsc_launch_mode */
    int32_t layout_policy;  /* bsc_layout_policy */
    int32_t accumulate;     /* 0: C = A B ; 1: C += A B */
    int32_t grid_limit;     /* cap on workgroups per grouped launch; 0 = engine default */
    /* Pack-cost model (uni20 "block coalescing", section "Interleaved vs
     * contiguous"): operand X of a group is gathered when
     *   2 * bytes(X) / pack_gbps  <  tiles * (pieces(X) - 1) * t_seg_us / 512
     *                                + padding flops saved / tile_gflops,
     * and the plan keeps its gathers only if their summed net saving exceeds
     * t_launch_us (the extra launch).  Times in microseconds; 512 tiles run
     * at once on MI355X.  0 selects the built-in MI355X defaults. */
    double t_launch_us;     /* cost of one more launch per contraction */
    double t_seg_us;        /* extra cost per piece one tile walks beyond one per k-segment */
    double pack_gbps;       /* gather bandwidth, counting read + write bytes */
    double tile_gflops;     /* sustained whole-GPU rate of the matrix-core tiles */
    /* K split of the bf16 direct-to-LDS tiles (uni20 "block coalescing":
     * enough independent work to fill the machine).  A 256 x 128 output tile
     * whose K chain is much longer than the plan's work per concurrent tile
     * slot is cut into K-slices that run as separate work items; the last
     * slice to finish adds the fp32 partial tiles in slice order (so results
     * do not depend on timing) and writes C.  The partials travel through
     * device-coherent memory, so splitting pays only for very long K chains.
     * 0: automatic (a tile is cut when its K exceeds twice the larger of
     * 64 x 32 and one slot's share of the plan's work, into slices of about
     * that length); -1: never split; n > 0: slices of at most n x 32 K. */
    int32_t split_k;
    /* Rows of the bf16 direct-to-LDS tiles (uni20 "block coalescing": enough
     * independent work to fill the machine): 0 = automatic (when the plan has
     * at most one 256 x 128 tile per CU, 128 for a group whose K chain is at
     * least 16 x 32 and above 1.5x one slot's share of the plan's work; 256
     * otherwise); 128 or 256 to force.  A tile of at most 128 rows runs as
     * four 64 x 64 waves with four K chunks in flight instead of two. */
    int32_t tile_rows;
    /* Columns of the bf16 direct-to-LDS tiles: 0 = automatic, 128 = the
     * 256 x 128 tile (two workgroups per CU), 256 = the wide tile (one
     * workgroup per CU holding the whole LDS: 256 x 256 output, four chunks of
     * copies in flight; eight waves of 128 x 64 when the plan's tasks are wide
     * tiles and tail bundles only, else four waves of 128 x 128, or 128 x 64
     * for groups of at most 128 columns).  tile_rows = 128, or a K chain far
     * above one CU's share of the launch, cuts wide tiles to 128 rows
     * (128 x 256 on eight 64 x 64 waves). */
    int32_t tile_cols;
} bsc_options;

typedef struct {
    int64_t triples;                 /* sector GEMMs (m, k, n) */
    int64_t c_blocks;                /* listed C blocks */
    int64_t zero_blocks;             /* listed C blocks no k contributes to */
    int64_t groups;                  /* coalescing groups with work (zero-fill groups excluded) */
    int64_t zero_groups;             /* zero-fill groups */
    int32_t axis;                    /* resolved bsc_axis */
    int32_t dtype;                   /* bsc_dtype */
    int64_t mode_count[3][3];        /* [operand A,B,C][bsc_mode]: groups per arrangement */
    int64_t runs;                    /* contiguous K-runs over all groups */
    int64_t items;                   /* work items per contraction */
    int64_t items_by_class[6];       /* generic tile, matrix-core tile, wave tail, zero fill,
                                        matrix-core tile with direct-to-LDS loads,
                                        skinny tile (at most 16 output rows or columns) */
    int64_t launches_per_contract;   /* GPU commands bsc_contract enqueues */
    int64_t launches_per_sector;     /* one launch per sector GEMM (+1 zero fill if needed) */
    int64_t useful_flops;            /* sum over triples of 2 M N K */
    int64_t alg_bytes;               /* A and B blocks read once + C blocks written once */
    int64_t pack_bytes;              /* bytes the gather kernel writes per contraction */
    int64_t device_bytes;            /* size of the device region bsc_plan_bind needs */
    int64_t tail_triples;            /* triples with 2 M N K <= 1024 */
    int64_t launches_issued;         /* launches enqueued by this plan so far */
    int32_t grid;                    /* workgroups of the grouped launch */
    int32_t split_tiles;             /* output tiles whose K is cut into slices (see split_k) */
    double predicted_us;             /* cost-model estimate of one contraction */
    /* the pack-cost model's terms over the gathered operands (0 without gathers):
     * saved piece set-ups (t_seg_us), saved K-step padding, gather traffic */
    double pack_gain_seg_us, pack_gain_pad_us, pack_cost_us;
    /* bf16: time saved by gathering misaligned single-view operands into
     * 16-byte rows, which moves their groups onto the direct-to-LDS tile */
    double pack_gain_align_us;
    /* 1 when the tasks are wide tiles (tile_cols = 256), tail bundles and
     * nothing else: with both operand bases 16-byte aligned the launch then
     * runs eight-wave workgroups of 512 threads instead of four-wave ones */
    int64_t wide_only;
} bsc_stats;

typedef struct bsc_plan_s *bsc_plan_t;

/* Fill *opt with defaults (grouped launch, AUTO layout, overwrite, built-in
 * cost constants). */
void bsc_options_default(bsc_options *opt);

/* Validate the descriptors, join sectors on k, build single-axis groups along
 * `axis`, choose each operand's arrangement and build the work list (host
 * only; no device call).  `opt` may be NULL.  On success *out owns a new plan. */
bsc_status bsc_plan(const bsc_index *m, const bsc_index *k, const bsc_index *n,
                    const bsc_operand *A, const bsc_operand *B, const bsc_operand *C,
                    bsc_dtype dtype, bsc_axis axis, const bsc_options *opt, bsc_plan_t *out);

/* Bytes of device memory bsc_plan_bind needs (work list + pack workspace +
 * K-split partial tiles). */
bsc_status bsc_plan_device_bytes(bsc_plan_t plan, size_t *bytes);

/* Upload the work list into the caller's device region `dev` (>= device_bytes,
 * 256-byte aligned) on `stream` and wait for the copy.  Also records the
 * current device's compute-unit count for the launch grid.  May be called
 * again with another region. */
bsc_status bsc_plan_bind(bsc_plan_t plan, void *dev, size_t bytes, void *stream);

/* Enqueue one contraction on `stream`: C (+)= A B.  A, B, C are device
 * pointers to the flat buffers the descriptors index (element types per
 * dtype).  Returns without synchronising. */
bsc_status bsc_contract(bsc_plan_t plan, const void *A, const void *B, void *C, void *stream);

/* bsc_contract for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * plan need not be bound.  Its device region (work-list image, pack
 * workspace, K-split partial tiles and counters: bsc_plan_device_bytes) lives
 * in a fixed array of 64 MiB that the library holds on every GPU it runs on
 * until the process ends; each call first copies the work-list image (counters
 * zero) into the current device's array on `stream`, then enqueues the same
 * launches as bsc_contract.  No device memory is allocated or freed.  Every
 * call on one GPU shares that GPU's array, which keeps the last call's
 * contents: calls that overlap in time on one GPU (different streams, or a
 * stream and a graph replay) race and give undefined results.
 * Errors: BSC_ERR_ARG (NULL plan or operand buffer), BSC_ERR_DEVICE_BYTES
 * (bsc_plan_device_bytes above 64 MiB; nothing is enqueued), BSC_ERR_HIP. */
bsc_status bsc_contract_noalloc(bsc_plan_t plan, const void *A, const void *B, void *C, void *stream);

/* Plan statistics (host only). */
bsc_status bsc_plan_stats(bsc_plan_t plan, bsc_stats *out);

/* Export the sector map for bit-exact checks: triples [3*T] as (m, k, n) key
 * ids sorted by (m, n, k); group_of_triple [T] (canonical group order; zero-fill
 * groups are not numbered); group_mode [3*G] the bsc_mode of A, B, C per group.
 * Any pointer may be NULL.  Sizes come from bsc_plan_stats (T = triples,
 * G = groups). */
bsc_status bsc_plan_export(bsc_plan_t plan, int32_t *triples, int32_t *group_of_triple, int32_t *group_mode);

/* Layout of the device work list (for inspection tools and host-side checks of
 * the kernels' addressing).  Counts are records; offsets are bytes into the
 * device region.  The record formats are internal to this library version. */
typedef struct {
    int64_t n_groups, n_runs, n_apieces, n_bpieces, n_cpieces, n_tasks, n_dense;
    int64_t off_groups, off_runs, off_apieces, off_bpieces, off_cpieces, off_tasks, off_dense;
    int64_t n_packs, n_pack_tasks;   /* gathers into the pack workspace and their work items */
    int64_t off_packs, off_pack_tasks;
    int64_t off_workspace;   /* byte offset of the pack workspace in the device region (after the image) */
    int64_t workspace_elems; /* pack workspace size in operand elements */
    int64_t bytes;           /* size of the work-list image */
    int64_t n_launches;      /* launches per contraction */
    int64_t n_counters, off_counters;   /* K-split arrival counters (int32, in the image, zero) */
    int64_t off_partials, partial_elems; /* K-split partial tiles (fp32, after the workspace) */
    int64_t n_tail, off_tail;            /* tail entries (one dense-tile record per wave of the tail bundles) */
} bsc_worklist_info;

/* Fill *info and, if image != NULL and bytes >= info->bytes, copy the host
 * image of the device work list (what bsc_plan_bind uploads) into image. */
bsc_status bsc_plan_worklist(bsc_plan_t plan, bsc_worklist_info *info, void *image, size_t bytes);

void bsc_plan_destroy(bsc_plan_t plan);

/* Plan cache (uni20 "block coalescing", "Open questions": keeping the
 * coalescing groups across DMRG sweeps once a site's block structure is
 * stable).  Planning costs milliseconds of host time; a sweep that contracts
 * the same block structure again should not pay it again.
 *
 * bsc_plan_cache_create makes an empty cache holding at most `capacity`
 * (>= 1) plans; the least recently used plan is dropped beyond that.
 *
 * bsc_plan_cached takes bsc_plan's arguments and returns the same result.
 * When every input (index tables, operand descriptors including offsets,
 * strides, flux and buffer lengths, dtype, axis and every option; opt NULL
 * means the defaults) equals that of a plan in the cache, *out is a copy of
 * the cached plan and no planning is done (*hit = 1); otherwise the call plans
 * as bsc_plan does, stores a copy and sets *hit = 0 (`hit` may be NULL).
 * Either way *out is a new, unbound plan owned by the caller (bind it, destroy
 * it with bsc_plan_destroy); the cache keeps its own copy and owns no device
 * memory.  Inputs are compared in full.  Errors are those of bsc_plan, plus
 * BSC_ERR_ARG for a NULL cache or out; a failed plan is not cached.  The cache
 * is internally locked, so threads may share one.
 *
 * bsc_plan_cache_stats reports hits, misses and stored plans (any pointer may
 * be NULL).  bsc_plan_cache_destroy frees the cache and its stored plans;
 * plans handed out stay valid. */
typedef struct bsc_plan_cache_s *bsc_plan_cache_t;
bsc_status bsc_plan_cache_create(int32_t capacity, bsc_plan_cache_t *out);
bsc_status bsc_plan_cached(bsc_plan_cache_t cache, const bsc_index *m, const bsc_index *k, const bsc_index *n,
                           const bsc_operand *A, const bsc_operand *B, const bsc_operand *C, bsc_dtype dtype,
                           bsc_axis axis, const bsc_options *opt, bsc_plan_t *out, int32_t *hit);
bsc_status bsc_plan_cache_stats(bsc_plan_cache_t cache, int64_t *hits, int64_t *misses, int64_t *entries);
void bsc_plan_cache_destroy(bsc_plan_cache_t cache);

/* Layout planning for chains of contractions (uni20 "block coalescing",
 * "Interleaved vs contiguous — the real tradeoff is a copy": the zero-copy
 * arrangement needs the axis to be coalesced laid out interleaved; "Open
 * questions": the coalescing axis may differ per stage).  Returns a block
 * layout for operand `which` (0 = A, 1 = B, 2 = C) of the contraction given
 * by the other arguments (as for bsc_plan), chosen so that the groups this
 * contraction forms see their members of that operand as one strided view.
 * The producer of an intermediate then writes it through these views and the
 * consumer needs neither a gather nor a per-member walk.
 *
 * Only the block keys (row_key, col_key, nblocks) and flux of the selected
 * operand are read; its offset, strides and buffer_elems are ignored.  The
 * other operands must be valid descriptors.  Grouping follows `axis` and
 * `opt` exactly as bsc_plan would (it depends on keys only).  Blocks go into
 * one panel per key of the non-coalesced axis (free-m grouping: A per k and
 * C per n, stacked down the rows; free-n: B per k and C per m, side by side;
 * contraction-axis: A per m side by side, B per n stacked down the rows; the
 * remaining operand one block per panel).  Within a panel each group's
 * members are consecutive in ascending key order, larger groups first; a
 * member already placed by an earlier group stays, and that group walks its
 * members one by one.  Every block is row-major inside its panel
 * (row_stride = {Ri*ld, ld}, col_stride = {Ci, 1}, with Ri, Ci the inner
 * extents); panel starts and leading dimensions are multiples of `align`
 * (>= 1) elements.
 *
 * Outputs, in the operand's block order: offset [nblocks], row_stride
 * [2*nblocks], col_stride [2*nblocks], and *buffer_elems, the buffer length
 * the layout needs (their contents are unspecified on failure).  Errors: BSC_ERR_ARG
 * (bad `which` or `align`, a NULL argument), BSC_ERR_SHAPE (a block key out
 * of range or a dimension < 1), and any error of bsc_plan on the keys. */
bsc_status bsc_plan_layout(const bsc_index *m, const bsc_index *k, const bsc_index *n,
                           const bsc_operand *A, const bsc_operand *B, const bsc_operand *C,
                           bsc_dtype dtype, bsc_axis axis, const bsc_options *opt, int32_t which, int64_t align,
                           int64_t *offset, int64_t *row_stride, int64_t *col_stride, int64_t *buffer_elems);

/* A fixed sequence of contractions (e.g. the stages of one environment
 * update) replayed as one HIP graph launch instead of one launch per stage
 * from the host (uni20 "block coalescing", "Open questions": deferred
 * synchronisation and reuse of a captured graph per site).
 *
 * bsc_chain_create records bsc_contract(plans[i], A[i], B[i], C[i]) for
 * i = 0 .. n-1, in that order, on a private stream into a graph and
 * instantiates it; nothing runs.  A, B, C are device pointers as for
 * bsc_contract; the graph holds these addresses and the plans' device
 * regions, so the buffers must stay allocated at the same addresses and the
 * plans must stay alive and bound to the same region while the chain exists.
 * On success *out owns a new chain.  Errors: BSC_ERR_ARG (a NULL pointer or
 * n < 1, or a NULL operand buffer), BSC_ERR_NOT_BOUND (an unbound plan),
 * BSC_ERR_HIP (stream, capture or instantiation failure; detail in
 * bsc_last_error).
 *
 * bsc_chain_launch enqueues one replay on `stream` (any stream, including the
 * default one) and returns without synchronising.  Replays of one chain, and a
 * replay and a direct bsc_contract of one of its plans, share the plans'
 * workspaces and must not overlap in time (use one stream).  A plan's
 * launches_issued statistic counts the capture only, not replays. */
typedef struct bsc_chain_s *bsc_chain_t;
bsc_status bsc_chain_create(const bsc_plan_t *plans, const void *const *A, const void *const *B, void *const *C,
                            int32_t n, bsc_chain_t *out);
bsc_status bsc_chain_launch(bsc_chain_t chain, void *stream);
void bsc_chain_destroy(bsc_chain_t chain);

/* Fused two-stage plan (uni20 "block coalescing", Open questions: the
 * "A.Y accumulate" stage of the R/A/B/C update; the memory-wall argument of
 * the "Sparse Operator Fusion" glossary page): stage 1 is a block-sparse
 * contraction C1 = A1 B1 (m1, k1, n1, A1, B1, C1 as for bsc_plan); stage 2
 * contracts C1's blocks with a matrix B2 whose blocks are all 1 x 1
 * (C2 = A2 B2), where every stage-2 A block is one stage-1 C block read
 * through the same buffer with its rows and columns fused into one row index
 * (outer leg = the stage-1 row, inner leg = the stage-1 column; one column).
 * In the environment update this is T1 = E^T A followed by T2 = T1 W.
 *
 * bsc_fused_plan validates both stages as bsc_plan does, matches every stage-2
 * A block to the stage-1 C block with the same elements, and plans one
 * launch that computes C2 directly: each output block of stage-2 row key r,
 * viewed as an M x N matrix (M, N the outer and inner extents of r), receives
 * the sum over the stage-1 products A1(m1, a) B1(a, n1) that make up the
 * stage-2 A blocks (r, k) of row r, each weighted by the B2 element (k, n)
 * of that output (no term where B2 has no block).  C1 is neither read nor
 * written.  Overwrite or accumulate per opt->accumulate; opt->split_k bounds
 * how many waves share one output tile's stage-1 blocks (0: automatic, at
 * most 4; 1: one wave per tile; negative: BSC_ERR_ARG); opt->tile_cols sets
 * a wave's output tile edge (0: automatic; 16; 32, taken for fp32 plans of at
 * most 4 outputs per task and ignored otherwise; anything else: BSC_ERR_ARG);
 * other options are ignored.  Requirements (else BSC_ERR_UNSUPPORTED): dtype BSC_F64 or BSC_F32;
 * every stage-2 B block and output column of dim 1; stage-1 A, B, C blocks and
 * the stage-2 output blocks single strided views (as M x N for the outputs);
 * at most 64 stage-1 blocks per stage-2 row key;
 * C1's buffer length equal to A2's (else BSC_ERR_ARG).  Any error bsc_plan
 * reports for either stage is reported here.
 *
 * bsc_fused_bind uploads the work list into a caller-owned device region of
 * bsc_fused_device_bytes (256-byte aligned) on `stream` and waits for it.
 * bsc_fused_contract enqueues the one launch on `stream`: A1, B1 the stage-1
 * operand buffers, B2 the scalar matrix's buffer, C2 the output buffer.
 * Repeats are bit-identical (fixed summation order, no atomics). */
typedef struct bsc_fused_s *bsc_fused_t;
typedef struct {
    int64_t groups;                 /* stage-2 output row keys (stream plan: C blocks) */
    int64_t channels;               /* stage-1 block products (stream plan: sector GEMMs) */
    int64_t outputs;                /* stage-2 output blocks (stream plan: C blocks) */
    int64_t terms;                  /* nonzero (stage-1 block, output) weights (stream plan: C blocks
                                       some product reaches) */
    int64_t items;                  /* output tiles (16 x 16, or 32 x 32 when tile_blocks is 2) x output chunks */
    int64_t launches_per_contract;
    int64_t useful_flops;           /* stage-1 products (2 M N K each) + weighted adds (2 M N per term);
                                       a stream plan counts its products only */
    int64_t stage1_flops;
    int64_t alg_bytes;              /* stage-1 operands and B2 read once, C2 written once */
    int64_t device_bytes;
    int64_t launches_issued;
    /* byte offsets of the record arrays in the device image (bsc_fused_worklist) */
    int64_t off_groups, off_chans, off_outs, off_widx, off_tasks;
    int64_t outs_per_task;          /* outputs one task accumulates (1, 4, 8 or 16) */
    int64_t off_parts, n_parts;     /* per-wave records, four per workgroup */
    int64_t off_pchans, n_pchans;   /* the parts' product lists */
    int64_t tile_blocks;            /* a wave's tile: tile_blocks^2 blocks of 16 x 16 */
    int64_t stream;                 /* 1: a bsc_stream_plan (one contraction), 0: two stages */
    int64_t off_ones;               /* byte offset of a stream plan's weight 1 in the device image */
    int64_t longest_chunks;         /* 32-index register chunks of the longest wave's product stream */
    int64_t stream_preferred;       /* stream plan expected faster than bsc_plan's grouped tiles: 1 when
                                       longest_chunks <= 32 (measured crossover on MI355X; long K per C
                                       block favours the grouped tiles' operand reuse) */
} bsc_fused_summary;
bsc_status bsc_fused_plan(const bsc_index *m1, const bsc_index *k1, const bsc_index *n1, const bsc_operand *A1,
                          const bsc_operand *B1, const bsc_operand *C1, const bsc_index *m2, const bsc_index *k2,
                          const bsc_index *n2, const bsc_operand *A2, const bsc_operand *B2, const bsc_operand *C2,
                          bsc_dtype dtype, const bsc_options *opt, bsc_fused_t *out);
/* One block-sparse contraction C (+)= A B (the operation of bsc_plan, uni20
 * "block coalescing": every C block the sum over its k sectors of A B block
 * products) planned for the register-stream kernel of the fused plan instead
 * of the grouped tiles: every C block is its own group (one stage-1 block,
 * one output, weight 1) cut into 16 x 16 (or, fp32, 32 x 32) wave tiles, each
 * wave streaming its tile's products through registers and writing the C
 * block directly.  Suits many short-K sector GEMMs in fp32 / fp64, where the
 * grouped tiles wait on their dependent loads.  Arguments as for bsc_plan
 * (dtype BSC_F64 or BSC_F32 only; every A, B and C block a single strided
 * view, else BSC_ERR_UNSUPPORTED); opt->accumulate and opt->tile_cols (0, 16
 * or 32, as for bsc_fused_plan) are used, other options ignored.  C blocks no
 * product reaches are written as zero (overwrite) or left as they are
 * (accumulate).  The result is a bsc_fused_t: bind, contract, stats, worklist
 * and destroy as for a fused plan, with bsc_fused_contract(plan, A, B, NULL,
 * C, stream) (the B2 argument is ignored).  Repeats are bit-identical. */
bsc_status bsc_stream_plan(const bsc_index *m, const bsc_index *k, const bsc_index *n, const bsc_operand *A,
                           const bsc_operand *B, const bsc_operand *C, bsc_dtype dtype, const bsc_options *opt,
                           bsc_fused_t *out);
bsc_status bsc_fused_device_bytes(bsc_fused_t plan, size_t *bytes);
bsc_status bsc_fused_bind(bsc_fused_t plan, void *dev, size_t bytes, void *stream);
bsc_status bsc_fused_contract(bsc_fused_t plan, const void *A1, const void *B1, const void *B2, void *C2, void *stream);
bsc_status bsc_fused_stats(bsc_fused_t plan, bsc_fused_summary *out);
/* Copy of the device image bsc_fused_bind uploads (for inspection and host
 * replay): `bytes` must be at least bsc_fused_device_bytes, else BSC_ERR_ARG. */
bsc_status bsc_fused_worklist(bsc_fused_t plan, void *buf, size_t bytes);
void bsc_fused_destroy(bsc_fused_t plan);

/* Matrix-core issue-rate probe (measurement only, not part of a contraction):
 * enqueues on `stream` one launch of 8 workgroups per CU whose waves run
 * `iters` rounds of independent back-to-back matrix-core operations of the
 * kind the tiles of `dtype` use (v_mfma_f32_32x32x16_bf16 for BSC_BF16_F32,
 * v_mfma_f32_16x16x4_f32 for BSC_F32, v_mfma_f64_16x16x4_f64 for BSC_F64),
 * operands in registers.  *flops receives the launch's floating-point
 * operations; the caller times the launch (events on `stream`) to get the
 * measured peak.  `sink` is a device float the kernel could write but never
 * does.  Errors: BSC_ERR_ARG (NULL sink or flops, iters < 1, unknown dtype),
 * BSC_ERR_HIP. */
bsc_status bsc_probe_mfma(bsc_dtype dtype, int32_t iters, float *sink, void *stream, double *flops);

const char *bsc_status_string(bsc_status s);

/* Thread-local text of the last error raised on this thread ("" if none). */
const char *bsc_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BSC_H */
