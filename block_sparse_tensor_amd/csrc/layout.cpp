// Layout planning: block layouts chosen for the contraction that will read (or
// write) the operand, so that its coalescing groups find their members already
// interleaved along the coalesced axis and address them as one strided view
// (uni20 "block coalescing": "Interleaved vs contiguous — the real tradeoff is
// a copy" — the zero-copy interleaved arrangement needs the producer to have
// laid the axis out that way; "Open questions": mixing the coalescing axis per
// contraction stage).  A chain of contractions asks this for each
// intermediate, with the consumer's index tables and block lists, and lets the
// producer write the intermediate through the returned views: no gather
// launch and no per-member walk in the consumer.
//
// Grouping depends only on the block keys, never on the layout, so the
// operand is first given a provisional layout (each block row-major on its
// own), the contraction is planned, and the groups are read back.  The blocks
// then go into panels, one per key of the axis the groups do not coalesce:
//
//   free-m grouping   A: one panel per k, blocks stacked down the rows (m)
//                     C: one panel per n, blocks stacked down the rows (m)
//   free-n grouping   B: one panel per k, blocks side by side (n)
//                     C: one panel per m, blocks side by side (n)
//   contraction-axis  A: one panel per m, blocks side by side (k)
//                     B: one panel per n, blocks stacked down the rows (k)
//
// (the remaining operand of each grouping is read one block per segment and
// keeps one row-major block per panel).  Inside a panel the members of a
// group are placed consecutively in ascending key order, the group with the
// most useful flops first; a block that an earlier group already placed
// stays where it is, and that later group then walks its members one by one.
// Panels and leading dimensions are rounded up to `align` elements.
#include <algorithm>
#include <cstring>
#include <new>
#include <numeric>
#include <vector>

#include "bsc_internal.h"

namespace bsc {
namespace {

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Panels from the groups of plan p (see the top of this file).
bsc_status place(const Plan &p, const bsc_operand &Xr, const bsc_index &rir, const bsc_index &cir, int32_t which,
                 int64_t align, int64_t *offset, int64_t *row_stride, int64_t *col_stride, int64_t *buffer_elems) {
    const bsc_operand *X = &Xr;
    const bsc_index *ri = &rir, *ci = &cir;
    const int64_t nb = X->nblocks;
    auto rdim = [&](int64_t b) { return ri->dim[X->row_key[b]]; };
    auto cdim = [&](int64_t b) { return ci->dim[X->col_key[b]]; };
    auto rin = [&](int64_t b) { return ri->inner ? ri->inner[X->row_key[b]] : int64_t(1); };
    auto cin = [&](int64_t b) { return ci->inner ? ci->inner[X->col_key[b]] : int64_t(1); };
    int64_t top = 0;
    // which key of a block names its panel, and whether blocks stack down the rows
    enum { PLAIN, BY_COL_STACK_ROWS, BY_ROW_SIDE_BY_SIDE } kind = PLAIN;
    if (p.axis == BSC_AXIS_FREE_M) kind = which == 0 || which == 2 ? BY_COL_STACK_ROWS : PLAIN;
    else if (p.axis == BSC_AXIS_FREE_N) kind = which == 1 || which == 2 ? BY_ROW_SIDE_BY_SIDE : PLAIN;
    else if (p.axis == BSC_AXIS_CONTRACT) kind = which == 0 ? BY_ROW_SIDE_BY_SIDE : (which == 1 ? BY_COL_STACK_ROWS : PLAIN);

    // block index of each (row key, col key) of X
    std::vector<std::pair<uint64_t, int64_t>> keyed(nb);
    for (int64_t b = 0; b < nb; ++b)
        keyed[b] = {(static_cast<uint64_t>(static_cast<uint32_t>(X->row_key[b])) << 32) |
                        static_cast<uint32_t>(X->col_key[b]), b};
    std::sort(keyed.begin(), keyed.end());
    auto find_blk = [&](int32_t r, int32_t c) -> int64_t {
        const uint64_t key = (static_cast<uint64_t>(static_cast<uint32_t>(r)) << 32) | static_cast<uint32_t>(c);
        auto it = std::lower_bound(keyed.begin(), keyed.end(), std::make_pair(key, int64_t(-1)));
        return (it != keyed.end() && it->first == key) ? it->second : -1;
    };
    auto panel_key = [&](int64_t b) { return kind == BY_COL_STACK_ROWS ? X->col_key[b] : X->row_key[b]; };
    auto along_key = [&](int64_t b) { return kind == BY_COL_STACK_ROWS ? X->row_key[b] : X->col_key[b]; };

    std::vector<std::vector<int64_t>> panel_order;   // by panel key: block indices in placement order
    std::vector<char> placed(nb, 0);
    if (kind != PLAIN) {
        const int32_t npanels = kind == BY_COL_STACK_ROWS ? ci->nkeys : ri->nkeys;
        panel_order.assign(npanels, {});
        // members of each group: the X blocks of each panel the group reads or writes
        int32_t ng = 0;
        for (int32_t g : p.group_of_triple) ng = std::max(ng, g + 1);
        std::vector<std::vector<std::array<int32_t, 3>>> gt(ng);
        for (size_t t = 0; t < p.triples.size(); ++t) {
            const int32_t g = p.group_of_triple[t];
            if (g >= 0 && g < ng) gt[g].push_back(p.triples[t]);
        }
        std::vector<double> gflops(ng, 0.0);
        for (int32_t g = 0; g < ng; ++g)
            for (auto &t : gt[g]) gflops[g] += 2.0 * p.dm[t[0]] * p.dk[t[1]] * p.dn[t[2]];
        std::vector<int32_t> gorder(ng);
        std::iota(gorder.begin(), gorder.end(), 0);
        std::stable_sort(gorder.begin(), gorder.end(), [&](int32_t x, int32_t y) { return gflops[x] > gflops[y]; });
        for (int32_t g : gorder) {
            // (panel key, along key) of X's blocks in this group, per panel
            std::vector<std::pair<int32_t, int32_t>> pa;
            for (auto &t : gt[g]) {
                const int32_t r = which == 0 ? t[0] : (which == 1 ? t[1] : t[0]);
                const int32_t c = which == 0 ? t[1] : (which == 1 ? t[2] : t[2]);
                const int32_t pk = kind == BY_COL_STACK_ROWS ? c : r;
                const int32_t ak = kind == BY_COL_STACK_ROWS ? r : c;
                pa.push_back({pk, ak});
            }
            std::sort(pa.begin(), pa.end());
            pa.erase(std::unique(pa.begin(), pa.end()), pa.end());
            for (size_t i = 0; i < pa.size();) {
                size_t j = i;
                std::vector<int64_t> run;
                bool free = true;
                while (j < pa.size() && pa[j].first == pa[i].first) {
                    const int64_t b = kind == BY_COL_STACK_ROWS ? find_blk(pa[j].second, pa[j].first)
                                                                : find_blk(pa[j].first, pa[j].second);
                    if (b >= 0) {
                        run.push_back(b);
                        free = free && !placed[b];
                    }
                    ++j;
                }
                if (free)
                    for (int64_t b : run) {
                        placed[b] = 1;
                        panel_order[pa[i].first].push_back(b);
                    }
                i = j;
            }
        }
        // blocks no group placed: at the end of their panel, in key order
        std::vector<int64_t> rest;
        for (int64_t b = 0; b < nb; ++b)
            if (!placed[b]) rest.push_back(b);
        std::stable_sort(rest.begin(), rest.end(), [&](int64_t x, int64_t y) { return along_key(x) < along_key(y); });
        for (int64_t b : rest) panel_order[panel_key(b)].push_back(b);
    }
    // place the panels
    auto put = [&](int64_t b, int64_t o, int64_t ld) {
        offset[b] = o;
        row_stride[2 * b] = rin(b) * ld;
        row_stride[2 * b + 1] = ld;
        col_stride[2 * b] = cin(b);
        col_stride[2 * b + 1] = 1;
    };
    if (kind == PLAIN) {
        std::vector<int64_t> order(nb);
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(), [&](int64_t x, int64_t y) {
            return X->row_key[x] != X->row_key[y] ? X->row_key[x] < X->row_key[y] : X->col_key[x] < X->col_key[y];
        });
        for (int64_t b : order) {
            const int64_t ld = round_up(cdim(b), align);
            top = round_up(top, align);
            put(b, top, ld);
            top += rdim(b) * ld;
        }
    } else {
        for (auto &pl : panel_order) {
            if (pl.empty()) continue;
            top = round_up(top, align);
            if (kind == BY_COL_STACK_ROWS) {
                const int64_t ld = round_up(cdim(pl[0]), align);   // one column key: one width
                int64_t r0 = 0;
                for (int64_t b : pl) {
                    put(b, top + r0 * ld, ld);
                    r0 += rdim(b);
                }
                top += r0 * ld;
            } else {
                int64_t w = 0;
                for (int64_t b : pl) w += cdim(b);
                const int64_t ld = round_up(w, align);
                int64_t c0 = 0;
                for (int64_t b : pl) {
                    put(b, top + c0, ld);
                    c0 += cdim(b);
                }
                top += rdim(pl[0]) * ld;   // one row key: one height
            }
        }
    }
    *buffer_elems = round_up(top, align);
    return BSC_OK;
}

}  // namespace
}  // namespace bsc

using namespace bsc;

static bsc_status plan_layout(const bsc_index *m, const bsc_index *k, const bsc_index *n, const bsc_operand *A,
                              const bsc_operand *B, const bsc_operand *C, bsc_dtype dtype, bsc_axis axis,
                              const bsc_options *opt, int32_t which, int64_t align, int64_t *offset,
                              int64_t *row_stride, int64_t *col_stride, int64_t *buffer_elems) {
    set_error("");
    if (which < 0 || which > 2 || align < 1 || !buffer_elems || !m || !k || !n || !A || !B || !C) {
        set_error("bsc_plan_layout: bad operand selector, alignment or NULL argument");
        return BSC_ERR_ARG;
    }
    const bsc_operand *X = which == 0 ? A : (which == 1 ? B : C);
    const bsc_index *ri = which == 0 ? m : (which == 1 ? k : m);   // row index of X
    const bsc_index *ci = which == 0 ? k : (which == 1 ? n : n);   // column index of X
    const int64_t nb = X->nblocks;
    if (nb < 0 || (nb > 0 && (!X->row_key || !X->col_key || !offset || !row_stride || !col_stride))) {
        set_error("bsc_plan_layout: bad block list or NULL output array");
        return BSC_ERR_ARG;
    }
    if ((ri->nkeys > 0 && !ri->dim) || (ci->nkeys > 0 && !ci->dim)) {
        set_error("bsc_plan_layout: index without dimensions");
        return BSC_ERR_ARG;
    }
    for (int64_t b = 0; b < nb; ++b)
        if (X->row_key[b] < 0 || X->row_key[b] >= ri->nkeys || X->col_key[b] < 0 || X->col_key[b] >= ci->nkeys) {
            set_error("bsc_plan_layout: block key out of range");
            return BSC_ERR_SHAPE;
        }
    auto rdim = [&](int64_t b) { return ri->dim[X->row_key[b]]; };
    auto cdim = [&](int64_t b) { return ci->dim[X->col_key[b]]; };
    auto rin = [&](int64_t b) { return ri->inner ? ri->inner[X->row_key[b]] : int64_t(1); };
    auto cin = [&](int64_t b) { return ci->inner ? ci->inner[X->col_key[b]] : int64_t(1); };
    for (int64_t b = 0; b < nb; ++b)
        if (rdim(b) < 1 || cdim(b) < 1 || rin(b) < 1 || cin(b) < 1) {
            set_error("bsc_plan_layout: dimensions and inner extents must be >= 1");
            return BSC_ERR_SHAPE;
        }

    // provisional layout: blocks row-major, one after another
    std::vector<int64_t> off(nb), rs(2 * nb), cs(2 * nb);
    int64_t top = 0;
    for (int64_t b = 0; b < nb; ++b) {
        off[b] = top;
        rs[2 * b] = rin(b) * cdim(b);
        rs[2 * b + 1] = cdim(b);
        cs[2 * b] = cin(b);
        cs[2 * b + 1] = 1;
        top += rdim(b) * cdim(b);
    }
    bsc_operand prov = *X;
    prov.offset = off.data();
    prov.row_stride = rs.data();
    prov.col_stride = cs.data();
    prov.buffer_elems = top;
    bsc_plan_t h = nullptr;
    bsc_status st = bsc_plan(m, k, n, which == 0 ? &prov : A, which == 1 ? &prov : B, which == 2 ? &prov : C,
                                   dtype, axis, opt, &h);
    if (st != BSC_OK) return st;
    try {
        st = place(*reinterpret_cast<Plan *>(h), *X, *ri, *ci, which, align, offset, row_stride, col_stride,
                   buffer_elems);
    } catch (const std::bad_alloc &) {
        set_error("bsc_plan_layout: out of host memory");
        st = BSC_ERR_UNSUPPORTED;
    }
    bsc_plan_destroy(h);
    return st;
}


extern "C" bsc_status bsc_plan_layout(const bsc_index *m, const bsc_index *k, const bsc_index *n, const bsc_operand *A,
                                      const bsc_operand *B, const bsc_operand *C, bsc_dtype dtype, bsc_axis axis,
                                      const bsc_options *opt, int32_t which, int64_t align, int64_t *offset,
                                      int64_t *row_stride, int64_t *col_stride, int64_t *buffer_elems) {
    try {
        return plan_layout(m, k, n, A, B, C, dtype, axis, opt, which, align, offset, row_stride, col_stride,
                           buffer_elems);
    } catch (const std::bad_alloc &) {   // the provisional layout's arrays
        set_error("bsc_plan_layout: out of host memory");
        return BSC_ERR_UNSUPPORTED;
    }
}
