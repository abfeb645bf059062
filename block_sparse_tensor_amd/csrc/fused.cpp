// Host planner of the fused two-stage plan (fused_internal.h): stage 1 is a
// block-sparse contraction C1 = A1 B1; stage 2 contracts C1's blocks, each
// viewed as a stage-2 A block (rows: the stage-1 block's rows and columns
// fused, outer and inner leg; one column), with a matrix B2 of 1 x 1 blocks.
// Both stages are validated by the ordinary planner; this file matches stage
// 2's A blocks to stage 1's C blocks by their views of the shared buffer and
// turns every stage-2 output row into a group of weighted block products.
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <map>
#include <new>
#include <stdexcept>
#include <string>
#include <utility>

#include "fused_internal.h"

namespace bsc {

namespace {

struct FFail {
    bsc_status st;
};

[[noreturn]] void ffail(bsc_status st, const std::string &msg) {
    set_error(msg);
    throw FFail{st};
}

// element (x, y) of a validated block
int64_t blk_addr(const Blk &b, int64_t x, int64_t y) {
    return b.off + (x / b.ri) * b.rs0 + (x % b.ri) * b.rs1 + (y / b.ci) * b.cs0 + (y % b.ci) * b.cs1;
}

struct PlanGuard {
    bsc_plan_t p = nullptr;
    ~PlanGuard() { bsc_plan_destroy(p); }
};

bool single(const Blk &b) { return b.ri == 1 && b.ci == 1; }

// Every stage-1 C block's products (A block, B block), ascending k.
std::vector<std::vector<std::pair<size_t, size_t>>> stage1_products(const Plan &s1) {
    std::map<std::pair<int32_t, int32_t>, size_t> a1_at, b1_at, c1_key;
    for (size_t i = 0; i < s1.A.size(); ++i) a1_at[{s1.A[i].r, s1.A[i].c}] = i;
    for (size_t i = 0; i < s1.B.size(); ++i) b1_at[{s1.B[i].r, s1.B[i].c}] = i;
    std::vector<std::vector<std::pair<size_t, size_t>>> prods(s1.C.size());
    for (size_t i = 0; i < s1.C.size(); ++i) c1_key[{s1.C[i].r, s1.C[i].c}] = i;
    for (const auto &t : s1.triples) {   // sorted by (m, n, k): ascending k per C block
        const size_t ci = c1_key.at({t[0], t[2]});
        prods[ci].push_back({a1_at.at({t[0], t[1]}), b1_at.at({t[1], t[2]})});
    }
    return prods;
}

// The product record of one stage-1 product A1 B1 of an M x N block; wrow is
// the block's weight row, last marks the block's last product.
void push_chan(FusedPlan &f, const Plan &s1, const Blk &a1, const Blk &b1, int64_t M, int64_t N, int32_t wrow,
               bool last, const char *who) {
    const int64_t esz = s1.dtype == BSC_F64 ? 8 : 4;
    if (!single(a1) || !single(b1))
        ffail(BSC_ERR_UNSUPPORTED, std::string(who) + ": the A and B blocks must be single-leg views");
    FChan ch{};
    ch.a_off = a1.off;
    ch.a_rs = a1.rs0;
    ch.a_ks = a1.cs0;
    ch.b_off = b1.off;
    ch.b_ks = b1.rs0;
    ch.b_ns = b1.cs0;
    ch.K = (int32_t)s1.dk[(size_t)a1.c];
    // the kernel reads each operand block as one raw buffer of 32-bit range
    const int64_t span_a = ((M - 1) * ch.a_rs + (ch.K - 1) * ch.a_ks + 1) * esz;
    const int64_t span_b = ((int64_t)(ch.K - 1) * ch.b_ks + (N - 1) * ch.b_ns + 1) * esz;
    if (span_a >= ((int64_t)1 << 31) || span_b >= ((int64_t)1 << 31))
        ffail(BSC_ERR_UNSUPPORTED, std::string(who) + ": an operand block spans 2 GiB or more");
    ch.wrow = (int16_t)wrow;
    ch.last = last ? 1 : 0;
    f.chans.push_back(ch);
    f.stage1_flops += 2 * M * N * ch.K;
}

void finish_fused(FusedPlan &f, const Plan &s1, int32_t max_parts, int32_t tile_cols);

// One contraction through the register stream: every C block is a group of
// one stage-1 block whose tile is written (weight 1) to the block itself.
void build_stream(FusedPlan &f, const Plan &s1, bool accumulate, int32_t tile_cols) {
    const char *who = "bsc_stream_plan";
    const auto prods = stage1_products(s1);
    f.stream = true;
    f.a_elems = s1.a_elems;
    f.b_elems = s1.b_elems;
    f.w_elems = 0;
    f.c_elems = s1.c_elems;
    const int64_t esz = s1.dtype == BSC_F64 ? 8 : 4;
    for (size_t ci = 0; ci < s1.C.size(); ++ci) {
        const Blk &c = s1.C[ci];
        if (!single(c)) ffail(BSC_ERR_UNSUPPORTED, std::string(who) + ": the C blocks must be single-leg views");
        const int64_t M = s1.dm[(size_t)c.r], N = s1.dn[(size_t)c.c];
        FGroup g{};
        g.M = (int32_t)M;
        g.N = (int32_t)N;
        g.out0 = (int32_t)f.outs.size();
        g.nout = 1;
        g.chan0 = (int32_t)f.chans.size();
        g.flags = accumulate ? G_ACCUMULATE : 0;
        f.outs.push_back({c.off, c.rs0, c.cs0});
        if (M > 1 && N > 1 && std::llabs(c.rs0) < std::llabs(c.cs0)) g.flags |= G_FTRANS;
        f.alg_bytes += M * N * esz;
        // A C block of many products makes every product a block of its own,
        // weighted by 1 into the output, so its list can be shared by up to
        // four waves (the fused plan's split by blocks, taken when the launch
        // would leave CUs idle), their sums added in part order.  Measured on
        // MI355X: an all-zero-charge chain's stage 3 (16 products per block)
        // 23.0 -> 11.8 us; blocks of a few products ran slower that way (a
        // random structure 10.4 -> 13.4 us), so they stay one block.
        const auto &pl = prods[ci];
        // (at most FUSED_WCAP blocks fit a wave's lane-held weights: longer lists stay one block)
        const bool each = pl.size() >= (size_t)STREAM_SPLIT_PRODUCTS && pl.size() <= (size_t)FUSED_WCAP;
        for (size_t pi = 0; pi < pl.size(); ++pi)
            push_chan(f, s1, s1.A[pl[pi].first], s1.B[pl[pi].second], M, N, each ? (int32_t)pi : 0,
                      each || pi + 1 == pl.size(), who);
        g.nchan = (int32_t)f.chans.size() - g.chan0;
        // a C block without products is written as zero (or left as is)
        g.nblk = pl.empty() ? 0 : (each ? (int32_t)pl.size() : 1);
        g.wbase = (int32_t)f.widx.size();
        for (int32_t b = 0; b < g.nblk; ++b) f.widx.push_back(0);   // the plan's own weight 1
        if (!pl.empty()) f.terms++;
        f.groups.push_back(g);
    }
    finish_fused(f, s1, 4, tile_cols);
}

void build_fused(FusedPlan &f, const Plan &s1, const Plan &s2, const bsc_index *m2idx, bool accumulate,
                 int32_t max_parts, int32_t tile_cols) {
    if (s1.c_elems != s2.a_elems)
        ffail(BSC_ERR_ARG, "bsc_fused_plan: stage 2's A buffer must be stage 1's C buffer (lengths differ)");
    // stage 2's B: scalars only (every contracted and output key of stage 2 has dim 1)
    for (const Blk &b : s2.B)
        if (s2.dk[(size_t)b.r] != 1 || s2.dn[(size_t)b.c] != 1)
            ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: stage 2's B blocks must all be 1 x 1");
    for (const Blk &b : s2.C)
        if (s2.dn[(size_t)b.c] != 1) ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: stage 2's output columns must have dim 1");
    // stage-1 C blocks by offset
    std::map<int64_t, size_t> c1_at;
    for (size_t i = 0; i < s1.C.size(); ++i) {
        if (!single(s1.C[i])) ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: stage 1's C blocks must be single-leg views");
        c1_at[s1.C[i].off] = i;
    }
    const auto prods = stage1_products(s1);
    // stage 2: A blocks and outputs by row key, B blocks by (k, n)
    std::map<int32_t, std::vector<size_t>> a2_rows, c2_rows;
    for (size_t i = 0; i < s2.A.size(); ++i) a2_rows[s2.A[i].r].push_back(i);
    for (size_t i = 0; i < s2.C.size(); ++i) c2_rows[s2.C[i].r].push_back(i);
    std::map<std::pair<int32_t, int32_t>, int64_t> w_at;
    for (const Blk &b : s2.B) w_at[{b.r, b.c}] = b.off;
    f.a_elems = s1.a_elems;
    f.b_elems = s1.b_elems;
    f.w_elems = s2.b_elems;
    f.c_elems = s2.c_elems;
    const int64_t esz = s1.dtype == BSC_F64 ? 8 : 4;
    for (auto &row : c2_rows) {
        const int32_t m2 = row.first;
        std::vector<size_t> &outs = row.second;
        std::sort(outs.begin(), outs.end(), [&](size_t x, size_t y) { return s2.C[x].c < s2.C[y].c; });
        // the row's blocks as M x N matrices: the row key's outer leg down, its inner leg across
        const int64_t N = m2idx->inner ? m2idx->inner[m2] : 1, M = s2.dm[(size_t)m2] / N;
        FGroup g{};
        g.M = (int32_t)M;
        g.N = (int32_t)N;
        g.out0 = (int32_t)f.outs.size();
        g.nout = (int32_t)outs.size();
        g.chan0 = (int32_t)f.chans.size();
        g.flags = accumulate ? G_ACCUMULATE : 0;
        bool trans = true;
        for (size_t oi : outs) {
            const Blk &c = s2.C[oi];
            // element (i, j) of the M x N view is stage-2 row i * N + j (outer leg i, inner leg j);
            // the view must be affine in (i, j)
            const int64_t rs = M > 1 ? blk_addr(c, N, 0) - c.off : 0, cs = N > 1 ? blk_addr(c, 1, 0) - c.off : 0;
            for (int64_t i = 0; i < M; ++i)
                for (int64_t j = 0; j < N; ++j)
                    if (blk_addr(c, i * N + j, 0) != c.off + i * rs + j * cs)
                        ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: a stage-2 output block is not one strided M x N view");
            f.outs.push_back({c.off, rs, cs});
            if (!(M > 1 && N > 1 && std::llabs(rs) < std::llabs(cs))) trans = false;
            f.alg_bytes += M * N * esz;
        }
        std::vector<int32_t> blk_k2;    // stage-2 contracted key of each stage-1 block (its weight row)
        auto ar = a2_rows.find(m2);
        if (ar != a2_rows.end()) {
            std::vector<size_t> a2s = ar->second;
            std::sort(a2s.begin(), a2s.end(), [&](size_t x, size_t y) { return s2.A[x].c < s2.A[y].c; });
            for (size_t ai : a2s) {
                const Blk &a2 = s2.A[ai];
                auto hit = c1_at.find(a2.off);
                if (hit == c1_at.end())
                    ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: a stage-2 A block is not a stage-1 C block");
                const Blk &c1 = s1.C[hit->second];
                const int64_t R1 = s1.dm[(size_t)c1.r], N1 = s1.dn[(size_t)c1.c];
                if (R1 != M || N1 != N || s2.dk[(size_t)a2.c] != 1)
                    ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: a stage-2 A block does not fuse its stage-1 block's rows "
                                               "and columns (outer, inner)");
                // every element must coincide: stage-2 (i N + j, 0) == stage-1 (i, j)
                for (int64_t i = 0; i < M; ++i)
                    for (int64_t j = 0; j < N; ++j)
                        if (blk_addr(a2, i * N + j, 0) != blk_addr(c1, i, j))
                            ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: a stage-2 A block views its stage-1 block "
                                                       "in another element order");
                const auto &pl = prods[hit->second];
                if (pl.empty()) continue;   // a stage-1 block with no product stays zero: no term
                if (blk_k2.size() >= (size_t)INT16_MAX)
                    ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: a stage-2 row fuses too many stage-1 blocks");
                for (size_t pi = 0; pi < pl.size(); ++pi)
                    push_chan(f, s1, s1.A[pl[pi].first], s1.B[pl[pi].second], M, N, (int32_t)blk_k2.size(),
                              pi + 1 == pl.size(), "bsc_fused_plan: stage 1");
                blk_k2.push_back(a2.c);
            }
        }
        g.nchan = (int32_t)f.chans.size() - g.chan0;
        g.nblk = (int32_t)blk_k2.size();
        g.wbase = (int32_t)f.widx.size();
        for (size_t r = 0; r < blk_k2.size(); ++r)
            for (size_t oi : outs) {
                auto w = w_at.find({blk_k2[r], s2.C[oi].c});
                const int64_t wi = w == w_at.end() ? -1 : w->second;
                if (wi > INT32_MAX) ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: stage 2's B buffer beyond 2^31 elements");
                f.widx.push_back((int32_t)wi);
                if (wi >= 0) f.terms++;
                if (wi >= 0) f.useful_flops += 2 * M * N;
            }
        if (f.widx.size() > (size_t)INT32_MAX) ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: weight table too large");
        if (trans) g.flags |= G_FTRANS;
        f.groups.push_back(g);
    }
    f.alg_bytes += (int64_t)s2.B.size() * (s1.dtype == BSC_F64 ? 8 : 4);   // W read once
    finish_fused(f, s1, max_parts, tile_cols);
}

// The part both plans share: kernel instance, wave tile, tasks, splits, the
// parts of every workgroup and the device image.
void finish_fused(FusedPlan &f, const Plan &s1, int32_t max_parts, int32_t tile_cols) {
    const int64_t esz = s1.dtype == BSC_F64 ? 8 : 4;
    // outputs per task: the smallest kernel instance that holds every group's
    // outputs (larger groups are split over tasks, each recomputing the tile),
    // as long as every group's weights (blocks x outputs per task) fit the
    // wave's lane-held table
    int32_t most = 1, most_blk = 0;
    for (const FGroup &g : f.groups) {
        most = std::max(most, g.nout);
        most_blk = std::max(most_blk, g.nblk);
    }
    f.outs_per_task = most <= 1 ? 1 : most <= 4 ? 4 : most <= 8 ? 8 : FUSED_MAX_OUT;
    while (f.outs_per_task > 4 && (int64_t)most_blk * f.outs_per_task > FUSED_WCAP) f.outs_per_task /= 2;
    if ((int64_t)most_blk * f.outs_per_task > FUSED_WCAP)
        ffail(BSC_ERR_UNSUPPORTED, "bsc_fused_plan: a stage-2 row fuses more than " +
                                       std::to_string(FUSED_WCAP / 4) + " stage-1 blocks");
    // the wave tile: 32 x 32 (two by two matrix-core blocks) for fp32 plans of
    // at most 4 outputs per task (fp64 accumulators, or more outputs, would
    // not fit the registers), when 32 x 32 tiles cover at most a quarter more
    // padding than 16 x 16 ones and still make at least FUSED_WIDE_TASKS tasks
    // (fewer, larger tasks leave the chip idle: on a 768-bond chain they were
    // slower, on a 2048-bond chain 11 % faster); 16 x 16 otherwise.
    // tile_cols 16 or 32 fixes the choice (32 only where it fits).
    {
        int64_t cover16 = 0, cover32 = 0, tasks32 = 0;
        for (const FGroup &g : f.groups) {
            const int64_t tiles32 = (int64_t)((g.M + 31) / 32) * ((g.N + 31) / 32);
            cover16 += (int64_t)((g.M + 15) / 16) * ((g.N + 15) / 16) * 256;
            cover32 += tiles32 * 1024;
            tasks32 += tiles32 * ((g.nout + f.outs_per_task - 1) / f.outs_per_task);
        }
        const bool fits = f.dtype == BSC_F32 && f.outs_per_task <= 4;
        const bool pays = cover16 > 0 && cover32 * 4 <= cover16 * 5 && tasks32 >= FUSED_WIDE_TASKS;
        f.tile_blocks = fits && (tile_cols == 32 || (tile_cols == 0 && pays)) ? 2 : 1;
    }
    const int32_t TILE = FUSED_TILE * f.tile_blocks;
    std::vector<int64_t> work(f.groups.size(), 0);   // register chunks of one part
    for (size_t gi = 0; gi < f.groups.size(); ++gi) {
        const FGroup &g = f.groups[gi];
        const int32_t nchunks = std::max(1, (g.nout + f.outs_per_task - 1) / f.outs_per_task);
        for (int32_t oc = 0; oc < nchunks; ++oc)
            for (int32_t i0 = 0; i0 < g.M; i0 += TILE)
                for (int32_t j0 = 0; j0 < g.N; j0 += TILE) f.tasks.push_back({(int32_t)gi, i0, j0, oc});
    }
    f.useful_flops += f.stage1_flops;
    // algorithmic bytes: stage-1 operand blocks read once (W and the outputs are counted above)
    for (const Blk &b : s1.A) f.alg_bytes += s1.dm[(size_t)b.r] * s1.dk[(size_t)b.c] * esz;
    for (const Blk &b : s1.B) f.alg_bytes += s1.dk[(size_t)b.r] * s1.dn[(size_t)b.c] * esz;
    // splits: a task's register chunks over S parts (S <= min(4, nblk)) when it
    // holds more than a wave's share of the whole launch; each (group, S) gets
    // its parts' product lists once
    std::vector<int64_t> gchunks(f.groups.size(), 0);
    int64_t total_chunks = 0;
    std::vector<int64_t> ntile(f.groups.size(), 0);
    for (const FTask &t : f.tasks) ntile[(size_t)t.group]++;
    for (size_t gi = 0; gi < f.groups.size(); ++gi) {
        const FGroup &g = f.groups[gi];
        for (int32_t c = 0; c < g.nchan; ++c) gchunks[gi] += (f.chans[(size_t)(g.chan0 + c)].K + FUSED_KC - 1) / FUSED_KC;
        total_chunks += gchunks[gi] * ntile[gi];
    }
    (void)total_chunks;
    auto split_of = [&](size_t gi, int64_t share) {
        return (int32_t)std::max<int64_t>(
            1, std::min<int64_t>({(int64_t)max_parts, (int64_t)f.groups[gi].nblk, (gchunks[gi] + share - 1) / share}));
    };
    // workgroups the first-fit packing makes for a share (tasks keep their order)
    auto wgs_for = [&](int64_t share) {
        int64_t wgs = 0;
        int32_t used = 4;
        for (const FTask &t : f.tasks) {
            const int32_t S = split_of((size_t)t.group, share);
            if (used + S > 4) {
                ++wgs;
                used = 0;
            }
            used += S;
        }
        return wgs;
    };
    // Split only a plan whose unsplit workgroups leave CUs idle, and then up
    // to a quarter over what fits at once (the longest parts go first and
    // finish last).  Measured on MI355X: U(1)xU(1) (1289 unsplit workgroups,
    // 1280 resident) 33.2 us unsplit, 36.3 us split to 1489; the U(1) update
    // (329 unsplit, 512 resident) 30.5 -> 21.2 us split to 549.
    const int64_t resident = (int64_t)FUSED_CUS * fused_wgs_per_cu(f.dtype, f.outs_per_task, f.tile_blocks);
    const int64_t cap = resident * 5 / 4;
    int64_t share = INT64_MAX;
    const bool idle = ((int64_t)f.tasks.size() + 3) / 4 < resident;   // unsplit: four tasks per workgroup
    for (int64_t cand : {4, 5, 6, 8, 10, 12, 16, 24, 32, 48, 64}) {
        if (max_parts <= 1 || !idle) break;
        if (cand < FUSED_MIN_PART) continue;
        if (wgs_for(cand) <= cap) {
            share = cand;
            break;
        }
    }
    std::vector<int32_t> split(f.groups.size(), 1);
    std::vector<std::vector<std::pair<int32_t, int32_t>>> plist(f.groups.size());   // per part: (pchans start, count)
    for (size_t gi = 0; gi < f.groups.size(); ++gi) {
        const FGroup &g = f.groups[gi];
        const int64_t chunks = gchunks[gi];
        const int32_t S = share == INT64_MAX ? 1 : split_of(gi, share);
        split[gi] = S;
        // block starts of the group's products
        std::vector<int32_t> bst;
        for (int32_t c = 0; c < g.nchan; ++c)
            if (c == 0 || f.chans[(size_t)(g.chan0 + c - 1)].last) bst.push_back(c);
        bst.push_back(g.nchan);
        for (int32_t p = 0; p < S; ++p) {
            const int32_t start = (int32_t)f.pchans.size();
            for (int32_t r = p; r < g.nblk; r += S)
                for (int32_t c = bst[(size_t)r]; c < bst[(size_t)r + 1]; ++c) f.pchans.push_back(f.chans[(size_t)(g.chan0 + c)]);
            plist[gi].push_back({start, (int32_t)f.pchans.size() - start});
        }
        work[gi] = (chunks + S - 1) / S;
        f.longest_chunks = std::max(f.longest_chunks, work[gi]);
    }
    // longest parts first (tiles of one group stay together)
    std::stable_sort(f.tasks.begin(), f.tasks.end(),
                     [&](const FTask &x, const FTask &y) { return work[(size_t)x.group] > work[(size_t)y.group]; });
    // workgroups of four slots: the parts of a task in consecutive slots, first fit in task order
    std::vector<FPart> wg;
    auto close_wg = [&]() {
        if (wg.empty()) return;
        int32_t npass = 0, reduce = 0;
        for (const FPart &pr : wg) {
            npass = std::max(npass, (pr.no + 3) / 4);
            if (pr.nparts > 1) reduce = 1;
        }
        while (wg.size() < 4) wg.push_back(FPart{});
        for (FPart &pr : wg) {
            pr.npass = npass;
            pr.reduce = reduce;
            f.parts.push_back(pr);
        }
        wg.clear();
    };
    for (const FTask &t : f.tasks) {
        const FGroup &g = f.groups[(size_t)t.group];
        const int32_t S = split[(size_t)t.group], o0 = t.oc * f.outs_per_task;
        if (wg.size() + (size_t)S > 4) close_wg();
        for (int32_t p = 0; p < S; ++p) {
            FPart pr{};
            pr.i0 = t.i0;
            pr.j0 = t.j0;
            pr.ml = std::min(TILE, g.M - t.i0);
            pr.nl = std::min(TILE, g.N - t.j0);
            pr.M = g.M;
            pr.N = g.N;
            pr.chan0 = plist[(size_t)t.group][(size_t)p].first;
            pr.nchan = plist[(size_t)t.group][(size_t)p].second;
            pr.no = std::min(f.outs_per_task, g.nout - o0);
            pr.out0 = g.out0 + o0;
            pr.wbase = g.wbase + o0;
            pr.wstride = g.nout;
            pr.nblk = g.nblk;
            pr.flags = g.flags;
            pr.part = p;
            pr.nparts = S;
            if (pr.nchan > 0) pr.first = f.pchans[(size_t)pr.chan0];
            wg.push_back(pr);
        }
    }
    close_wg();
    // device image
    auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
    size_t off = 0;
    f.off_groups = off; off = align(off + f.groups.size() * sizeof(FGroup));
    f.off_chans = off;  off = align(off + f.chans.size() * sizeof(FChan));
    f.off_outs = off;   off = align(off + f.outs.size() * sizeof(FOut));
    f.off_widx = off;   off = align(off + f.widx.size() * sizeof(int32_t));
    f.off_tasks = off;  off = align(off + f.tasks.size() * sizeof(FTask));
    f.off_parts = off;  off = align(off + f.parts.size() * sizeof(FPart));
    f.off_pchans = off; off = align(off + f.pchans.size() * sizeof(FChan));
    f.off_ones = off;   off = align(off + sizeof(double));   // a stream plan's weight 1 in the plan's type
    f.image.assign(std::max<size_t>(off, 256), 0);
    auto put = [&](size_t o, const void *src, size_t nbytes) { if (nbytes) std::memcpy(f.image.data() + o, src, nbytes); };
    put(f.off_groups, f.groups.data(), f.groups.size() * sizeof(FGroup));
    put(f.off_chans, f.chans.data(), f.chans.size() * sizeof(FChan));
    put(f.off_outs, f.outs.data(), f.outs.size() * sizeof(FOut));
    put(f.off_widx, f.widx.data(), f.widx.size() * sizeof(int32_t));
    put(f.off_tasks, f.tasks.data(), f.tasks.size() * sizeof(FTask));
    put(f.off_parts, f.parts.data(), f.parts.size() * sizeof(FPart));
    put(f.off_pchans, f.pchans.data(), f.pchans.size() * sizeof(FChan));
    if (f.dtype == BSC_F64) {
        const double one = 1.0;
        put(f.off_ones, &one, sizeof(one));
    } else {
        const float one = 1.0f;
        put(f.off_ones, &one, sizeof(one));
    }
}

}  // namespace

}  // namespace bsc

using namespace bsc;

extern "C" bsc_status bsc_fused_plan(const bsc_index *m1, const bsc_index *k1, const bsc_index *n1,
                                     const bsc_operand *A1, const bsc_operand *B1, const bsc_operand *C1,
                                     const bsc_index *m2, const bsc_index *k2, const bsc_index *n2,
                                     const bsc_operand *A2, const bsc_operand *B2, const bsc_operand *C2,
                                     bsc_dtype dtype, const bsc_options *opt, bsc_fused_t *out) {
    set_error("");
    if (!out) {
        set_error("bsc_fused_plan: out is NULL");
        return BSC_ERR_ARG;
    }
    *out = nullptr;
    if (dtype != BSC_F64 && dtype != BSC_F32) {
        set_error("bsc_fused_plan: f64 and f32 only (stage 2 reads stage 1's output in the operands' type)");
        return BSC_ERR_UNSUPPORTED;
    }
    bsc_options o;
    if (opt) o = *opt;
    else bsc_options_default(&o);
    const bool accumulate = o.accumulate != 0;
    // split_k: the most parts a task is split into (0: automatic, up to 4; 1: never)
    if (o.split_k < 0) {
        set_error("bsc_fused_plan: split_k must be >= 0");
        return BSC_ERR_ARG;
    }
    const int32_t max_parts = o.split_k == 0 ? 4 : std::min(4, o.split_k);
    // tile_cols: the wave tile's edge (0: automatic, 16, or 32 where it fits)
    if (o.tile_cols != 0 && o.tile_cols != 16 && o.tile_cols != 32) {
        set_error("bsc_fused_plan: tile_cols must be 0, 16 or 32");
        return BSC_ERR_ARG;
    }
    const int32_t tile_cols = o.tile_cols;
    o.tile_cols = 0;
    o.accumulate = 0;
    o.split_k = 0;
    o.launch_mode = BSC_LAUNCH_GROUPED;
    PlanGuard g1, g2;
    bsc_status st = bsc_plan(m1, k1, n1, A1, B1, C1, dtype, BSC_AXIS_AUTO, &o, &g1.p);
    if (st != BSC_OK) {
        set_error(std::string("bsc_fused_plan: stage 1: ") + bsc_last_error());
        return st;
    }
    st = bsc_plan(m2, k2, n2, A2, B2, C2, dtype, BSC_AXIS_AUTO, &o, &g2.p);
    if (st != BSC_OK) {
        set_error(std::string("bsc_fused_plan: stage 2: ") + bsc_last_error());
        return st;
    }
    FusedPlan *f = new (std::nothrow) FusedPlan();
    if (!f) {
        set_error("bsc_fused_plan: out of host memory");
        return BSC_ERR_UNSUPPORTED;
    }
    f->dtype = dtype;
    try {
        build_fused(*f, *reinterpret_cast<Plan *>(g1.p), *reinterpret_cast<Plan *>(g2.p), m2, accumulate, max_parts, tile_cols);
    } catch (const FFail &e) {
        delete f;
        return e.st;
    } catch (const std::bad_alloc &) {
        delete f;
        set_error("bsc_fused_plan: out of host memory");
        return BSC_ERR_UNSUPPORTED;
    } catch (const std::out_of_range &) {
        delete f;
        set_error("bsc_fused_plan: inconsistent stage-1 sector join");
        return BSC_ERR_ARG;
    }
    *out = reinterpret_cast<bsc_fused_t>(f);
    return BSC_OK;
}

extern "C" bsc_status bsc_stream_plan(const bsc_index *m, const bsc_index *k, const bsc_index *n,
                                      const bsc_operand *A, const bsc_operand *B, const bsc_operand *C,
                                      bsc_dtype dtype, const bsc_options *opt, bsc_fused_t *out) {
    set_error("");
    if (!out) {
        set_error("bsc_stream_plan: out is NULL");
        return BSC_ERR_ARG;
    }
    *out = nullptr;
    if (dtype != BSC_F64 && dtype != BSC_F32) {
        set_error("bsc_stream_plan: f64 and f32 only");
        return BSC_ERR_UNSUPPORTED;
    }
    bsc_options o;
    if (opt) o = *opt;
    else bsc_options_default(&o);
    const bool accumulate = o.accumulate != 0;
    if (o.tile_cols != 0 && o.tile_cols != 16 && o.tile_cols != 32) {
        set_error("bsc_stream_plan: tile_cols must be 0, 16 or 32");
        return BSC_ERR_ARG;
    }
    const int32_t tile_cols = o.tile_cols;
    o.tile_cols = 0;
    o.accumulate = 0;
    o.split_k = 0;
    o.launch_mode = BSC_LAUNCH_GROUPED;
    PlanGuard g1;
    bsc_status st = bsc_plan(m, k, n, A, B, C, dtype, BSC_AXIS_AUTO, &o, &g1.p);
    if (st != BSC_OK) {
        set_error(std::string("bsc_stream_plan: ") + bsc_last_error());
        return st;
    }
    FusedPlan *f = new (std::nothrow) FusedPlan();
    if (!f) {
        set_error("bsc_stream_plan: out of host memory");
        return BSC_ERR_UNSUPPORTED;
    }
    f->dtype = dtype;
    try {
        build_stream(*f, *reinterpret_cast<Plan *>(g1.p), accumulate, tile_cols);
    } catch (const FFail &e) {
        delete f;
        return e.st;
    } catch (const std::bad_alloc &) {
        delete f;
        set_error("bsc_stream_plan: out of host memory");
        return BSC_ERR_UNSUPPORTED;
    } catch (const std::out_of_range &) {
        delete f;
        set_error("bsc_stream_plan: inconsistent sector join");
        return BSC_ERR_ARG;
    }
    *out = reinterpret_cast<bsc_fused_t>(f);
    return BSC_OK;
}

extern "C" bsc_status bsc_fused_device_bytes(bsc_fused_t plan, size_t *bytes) {
    if (!plan || !bytes) {
        set_error("bsc_fused_device_bytes: NULL argument");
        return BSC_ERR_ARG;
    }
    *bytes = reinterpret_cast<FusedPlan *>(plan)->image.size();
    return BSC_OK;
}

extern "C" bsc_status bsc_fused_stats(bsc_fused_t plan, bsc_fused_summary *out) {
    if (!plan || !out) {
        set_error("bsc_fused_stats: NULL argument");
        return BSC_ERR_ARG;
    }
    const FusedPlan *f = reinterpret_cast<FusedPlan *>(plan);
    std::memset(out, 0, sizeof(*out));
    out->groups = (int64_t)f->groups.size();
    out->channels = (int64_t)f->chans.size();
    out->outputs = (int64_t)f->outs.size();
    out->terms = f->terms;
    out->items = (int64_t)f->tasks.size();
    out->launches_per_contract = f->tasks.empty() ? 0 : 1;
    out->useful_flops = f->useful_flops;
    out->stage1_flops = f->stage1_flops;
    out->alg_bytes = f->alg_bytes;
    out->device_bytes = (int64_t)f->image.size();
    out->launches_issued = f->launches_issued;
    out->off_groups = (int64_t)f->off_groups;
    out->off_chans = (int64_t)f->off_chans;
    out->off_outs = (int64_t)f->off_outs;
    out->off_widx = (int64_t)f->off_widx;
    out->off_tasks = (int64_t)f->off_tasks;
    out->outs_per_task = f->outs_per_task;
    out->tile_blocks = f->tile_blocks;
    out->off_parts = (int64_t)f->off_parts;
    out->n_parts = (int64_t)f->parts.size();
    out->off_pchans = (int64_t)f->off_pchans;
    out->n_pchans = (int64_t)f->pchans.size();
    out->stream = f->stream ? 1 : 0;
    out->off_ones = (int64_t)f->off_ones;
    out->longest_chunks = f->longest_chunks;
    out->stream_preferred = f->stream && f->longest_chunks <= STREAM_MAX_CHUNKS ? 1 : 0;
    return BSC_OK;
}

extern "C" bsc_status bsc_fused_worklist(bsc_fused_t plan, void *buf, size_t bytes) {
    if (!plan || !buf) {
        set_error("bsc_fused_worklist: NULL argument");
        return BSC_ERR_ARG;
    }
    const FusedPlan *f = reinterpret_cast<FusedPlan *>(plan);
    if (bytes < f->image.size()) {
        set_error("bsc_fused_worklist: buffer smaller than bsc_fused_device_bytes");
        return BSC_ERR_ARG;
    }
    std::memcpy(buf, f->image.data(), f->image.size());
    return BSC_OK;
}

extern "C" void bsc_fused_destroy(bsc_fused_t plan) { delete reinterpret_cast<FusedPlan *>(plan); }
