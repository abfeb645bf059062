// Host planner: descriptors -> validated sectors -> sector join -> single-axis
// groups -> strided pieces and runs -> work list.  Host-only C++17 (no HIP), so
// it also builds with g++ for sanitizer runs.
//
// Follows the uni20 design note "block coalescing":
//   * sections "Summary" and "Why single-axis coalescing is hole-free": one GEMM
//     per sector combination (m, k, n), grouped along one axis only;
//   * section "Expressed as strided views over shared storage": each block
//     keeps its own (offset, strides) view and the coalesced operand is a wider
//     view when the members line up;
//   * section "Interleaved vs contiguous": members that do not line up stay
//     separate pieces that the kernel walks (no copy);
//   * section "Coalescing is a plan-time transform": all of this happens here,
//     once, never inside the kernel.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <numeric>
#include <stdexcept>
#include <unordered_map>
#include <utility>

#include "bsc_internal.h"

namespace bsc {

namespace {

struct Fail {
    bsc_status st;
};

[[noreturn]] void fail(bsc_status st, const std::string &msg) {
    set_error(msg);
    throw Fail{st};
}

struct Idx {
    int32_t nkeys = 0;
    std::vector<int32_t> q;      // nkeys * nq
    std::vector<int64_t> dim, inner;
};

Idx copy_index(const bsc_index *x, const char *name, int32_t nq) {
    if (!x) fail(BSC_ERR_ARG, std::string("index ") + name + " is NULL");
    if (x->nkeys < 0) fail(BSC_ERR_ARG, std::string("index ") + name + ": negative key count");
    if (x->nq != nq) fail(BSC_ERR_ARG, std::string("index ") + name + ": charge arity differs from index m");
    Idx r;
    r.nkeys = x->nkeys;
    if (r.nkeys > 0 && (!x->charge || !x->dim)) fail(BSC_ERR_ARG, std::string("index ") + name + ": NULL array");
    r.q.assign(x->charge, x->charge + (size_t)r.nkeys * nq);
    r.dim.assign(x->dim, x->dim + r.nkeys);
    r.inner.assign(r.nkeys, 1);
    if (x->inner) r.inner.assign(x->inner, x->inner + r.nkeys);
    for (int32_t i = 0; i < r.nkeys; ++i) {
        if (r.dim[i] < 1 || r.dim[i] > (int64_t(1) << 31) - 1)
            fail(BSC_ERR_SHAPE, std::string("index ") + name + ": key " + std::to_string(i) + " has dim outside 1..2^31-1");
        if (r.inner[i] < 1 || r.dim[i] % r.inner[i] != 0)
            fail(BSC_ERR_SHAPE, std::string("index ") + name + ": key " + std::to_string(i) + " inner extent does not divide dim");
    }
    return r;
}

// Canonical form of one axis of a view: a single leg (inner 1, stride s0, s1 = 0)
// whenever the two legs collapse, stride 0 for an axis of extent 1.
void canon_axis(int64_t ext, int64_t inner, int64_t &s0, int64_t &s1, int32_t &in) {
    int64_t outer = ext / inner;
    if (ext == 1) { s0 = 0; s1 = 0; in = 1; return; }
    if (inner == 1) { s1 = 0; in = 1; return; }
    if (outer == 1) { s0 = s1; s1 = 0; in = 1; return; }
    if (s0 == inner * s1) { s0 = s1; s1 = 0; in = 1; return; }
    in = (int32_t)inner;
}

using u128 = unsigned __int128;

u128 max_addr(int64_t off, int64_t ext_r, int64_t in_r, int64_t rs0, int64_t rs1,
              int64_t ext_c, int64_t in_c, int64_t cs0, int64_t cs1) {
    return (u128)off + (u128)(ext_r / in_r - 1) * (u128)rs0 + (u128)(in_r - 1) * (u128)rs1 +
           (u128)(ext_c / in_c - 1) * (u128)cs0 + (u128)(in_c - 1) * (u128)cs1;
}

std::vector<Blk> copy_operand(const bsc_operand *X, const char *name, const Idx &R, const Idx &Cc, int32_t nq,
                              int64_t &elems, std::vector<int32_t> &flux) {
    if (!X) fail(BSC_ERR_ARG, std::string("operand ") + name + " is NULL");
    if (X->nblocks < 0) fail(BSC_ERR_ARG, std::string("operand ") + name + ": negative block count");
    if (X->buffer_elems < 0) fail(BSC_ERR_ARG, std::string("operand ") + name + ": negative buffer size");
    if (!X->flux) fail(BSC_ERR_ARG, std::string("operand ") + name + ": NULL flux");
    if (X->nblocks > 0 && (!X->row_key || !X->col_key || !X->offset || !X->row_stride || !X->col_stride))
        fail(BSC_ERR_ARG, std::string("operand ") + name + ": NULL block array");
    flux.assign(X->flux, X->flux + nq);
    elems = X->buffer_elems;
    std::vector<Blk> out((size_t)X->nblocks);
    std::unordered_map<uint64_t, int64_t> seen;
    seen.reserve((size_t)X->nblocks * 2 + 1);
    for (int64_t b = 0; b < X->nblocks; ++b) {
        Blk k;
        k.r = X->row_key[b];
        k.c = X->col_key[b];
        std::string where = std::string("operand ") + name + " block " + std::to_string(b);
        if (k.r < 0 || k.r >= R.nkeys || k.c < 0 || k.c >= Cc.nkeys) fail(BSC_ERR_SHAPE, where + ": key out of range");
        uint64_t key = ((uint64_t)(uint32_t)k.r << 32) | (uint32_t)k.c;
        if (!seen.emplace(key, b).second) fail(BSC_ERR_SHAPE, where + ": duplicate (row, col) key pair");
        for (int32_t j = 0; j < nq; ++j)
            if ((int64_t)R.q[(size_t)k.r * nq + j] - Cc.q[(size_t)k.c * nq + j] != flux[j])
                fail(BSC_ERR_CHARGE, where + ": charge rule q_row - q_col == flux broken");
        k.off = X->offset[b];
        k.rs0 = X->row_stride[2 * b];
        k.rs1 = X->row_stride[2 * b + 1];
        k.cs0 = X->col_stride[2 * b];
        k.cs1 = X->col_stride[2 * b + 1];
        int64_t er = R.dim[k.r], ir = R.inner[k.r], ec = Cc.dim[k.c], ic = Cc.inner[k.c];
        const int64_t legs[4][2] = {{er / ir, k.rs0}, {ir, k.rs1}, {ec / ic, k.cs0}, {ic, k.cs1}};
        for (auto &lg : legs)
            if (lg[1] < 0 || (lg[0] > 1 && lg[1] < 1)) fail(BSC_ERR_SHAPE, where + ": a leg of extent > 1 needs a stride >= 1");
        if (k.off < 0) fail(BSC_ERR_BOUNDS, where + ": negative offset");
        if (max_addr(k.off, er, ir, k.rs0, k.rs1, ec, ic, k.cs0, k.cs1) >= (u128)elems)
            fail(BSC_ERR_BOUNDS, where + ": view reaches past the buffer");
        canon_axis(er, ir, k.rs0, k.rs1, k.ri);
        canon_axis(ec, ic, k.cs0, k.cs1, k.ci);
        out[(size_t)b] = k;
    }
    return out;
}

// Element addresses of a canonical block, in row-major element order.
template <class F>
void for_each_addr(const Blk &b, int64_t R, int64_t C, F &&f) {
    for (int64_t r = 0; r < R; ++r) {
        int64_t rp = b.off + (r / b.ri) * b.rs0 + (r % b.ri) * b.rs1;
        for (int64_t c = 0; c < C; ++c) f(rp + (c / b.ci) * b.cs0 + (c % b.ci) * b.cs1);
    }
}

// C views must be pairwise disjoint and must not alias themselves.  Blocks whose
// address ranges do not intersect are disjoint; only clusters of intersecting
// ranges (interleaved views) are checked element by element with a bitmap.
void check_c_disjoint(const std::vector<Blk> &C, const std::vector<int64_t> &dm, const std::vector<int64_t> &dn) {
    struct Iv {
        int64_t lo, hi;
        size_t i;
    };
    std::vector<Iv> iv;
    iv.reserve(C.size());
    for (size_t i = 0; i < C.size(); ++i) {
        const Blk &b = C[i];
        int64_t R = dm[b.r], Cn = dn[b.c];
        int64_t hi = (int64_t)max_addr(b.off, R, b.ri, b.rs0, b.rs1, Cn, b.ci, b.cs0, b.cs1);
        iv.push_back({b.off, hi, i});
    }
    std::sort(iv.begin(), iv.end(), [](const Iv &a, const Iv &b) { return a.lo < b.lo || (a.lo == b.lo && a.i < b.i); });
    auto self_safe = [&](const Blk &b) {
        int64_t R = dm[b.r], Cn = dn[b.c];
        std::vector<std::pair<int64_t, int64_t>> legs;  // (stride, extent)
        int64_t ext[4] = {R / b.ri, b.ri, Cn / b.ci, b.ci};
        int64_t st[4] = {b.rs0, b.rs1, b.cs0, b.cs1};
        for (int j = 0; j < 4; ++j)
            if (ext[j] > 1) legs.push_back({st[j], ext[j]});
        std::sort(legs.begin(), legs.end());
        for (size_t j = 1; j < legs.size(); ++j)
            if ((u128)legs[j].first < (u128)legs[j - 1].first * (u128)legs[j - 1].second) return false;
        return true;
    };
    size_t a = 0;
    while (a < iv.size()) {
        size_t e = a + 1;
        int64_t hi = iv[a].hi;
        while (e < iv.size() && iv[e].lo <= hi) {
            hi = std::max(hi, iv[e].hi);
            ++e;
        }
        bool exact = (e - a) > 1 || !self_safe(C[iv[a].i]);
        if (exact) {
            int64_t lo = iv[a].lo;
            std::vector<uint64_t> bits((size_t)((hi - lo) / 64 + 1), 0);
            for (size_t j = a; j < e; ++j) {
                const Blk &b = C[iv[j].i];
                for_each_addr(b, dm[b.r], dn[b.c], [&](int64_t ad) {
                    uint64_t x = (uint64_t)(ad - lo);
                    uint64_t &w = bits[x >> 6];
                    uint64_t m = uint64_t(1) << (x & 63);
                    if (w & m) fail(BSC_ERR_OVERLAP, "operand C: two C elements share buffer element " + std::to_string(ad));
                    w |= m;
                });
            }
        }
        a = e;
    }
}

// ---------------------------------------------------------------------------
// strided pieces
// ---------------------------------------------------------------------------

// Piece of a canonical block.  along_rows: axis a = block rows, b = block cols.
DView piece_of(const Blk &b, bool along_rows, int32_t begin, int32_t len) {
    DView v;
    v.off = b.off;
    if (along_rows) {
        v.sa0 = b.rs0; v.sa1 = b.rs1; v.ia = b.ri;
        v.sb0 = b.cs0; v.sb1 = b.cs1; v.ib = b.ci;
    } else {
        v.sa0 = b.cs0; v.sa1 = b.cs1; v.ia = b.ci;
        v.sb0 = b.rs0; v.sb1 = b.rs1; v.ib = b.ri;
    }
    v.begin = begin;
    v.len = len;
    return v;
}

// Try to extend view `m` (extent m.len along a) by `w` placed right after it
// along axis a.  Succeeds iff the union is again one strided view.
bool merge_along_a(DView &m, const DView &w) {
    if (m.sb0 != w.sb0 || m.sb1 != w.sb1 || m.ib != w.ib) return false;
    if (m.ia != w.ia) return false;
    int64_t ia = m.ia;
    if (ia > 1 && m.sa1 != w.sa1) return false;
    int64_t mouter = m.len / ia, wouter = w.len / ia;
    int64_t d = w.off - m.off;
    if (d <= 0 || d % mouter != 0) return false;
    int64_t t = d / mouter;                 // outer stride of the union
    if (mouter > 1 && m.sa0 != t) return false;
    if (wouter > 1 && w.sa0 != t) return false;
    m.sa0 = t;
    m.len += w.len;
    return true;
}

// Same along axis b (the contracted axis for A and B pieces): `w` continues `m`
// along b; both cover the same range along a with identical a-structure.
bool merge_along_b(DView &m, int64_t m_blen, const DView &w, int64_t w_blen) {
    if (m.begin != w.begin || m.len != w.len || m.ia != w.ia || m.sa1 != w.sa1) return false;
    if (m.len > 1 || m.ia > 1) {
        if (m.sa0 != w.sa0) return false;
    }
    if (m.ib != w.ib) return false;
    int64_t ib = m.ib;
    if (ib > 1 && m.sb1 != w.sb1) return false;
    int64_t mouter = m_blen / ib, wouter = w_blen / ib;
    int64_t d = w.off - m.off;
    if (d <= 0 || d % mouter != 0) return false;
    int64_t t = d / mouter;
    if (mouter > 1 && m.sb0 != t) return false;
    if (wouter > 1 && w.sb0 != t) return false;
    m.sb0 = t;
    return true;
}

// Stack member views along a: one piece if they interleave into one view.
std::vector<DView> stack(const std::vector<DView> &mem) {
    std::vector<DView> out;
    if (mem.empty()) return out;
    DView cur = mem[0];
    bool ok = true;
    for (size_t i = 1; i < mem.size() && ok; ++i) ok = merge_along_a(cur, mem[i]);
    if (ok) {
        out.push_back(cur);
        return out;
    }
    return mem;
}

// 16-byte vector eligibility of a run's operand pieces (bf16: 8 elements).
bool vec_kcontig(const std::vector<DView> &v, int64_t K) {
    for (auto &p : v) {
        if (p.ib != 1 || !(p.sb0 == 1 || K == 1) || p.ia != 1) return false;
        if (p.off % 8 != 0 || (p.len > 1 && p.sa0 % 8 != 0)) return false;
    }
    return true;
}

bool vec_ncontig(const std::vector<DView> &v, int64_t K, int64_t buffer_elems) {
    if (v.size() != 1) return false;
    const DView &p = v[0];
    if (p.ia != 1 || !(p.sa0 == 1 || p.len == 1) || p.ib != 1) return false;
    if (p.off % 8 != 0 || (K > 1 && p.sb0 % 8 != 0)) return false;
    const int64_t padded = (p.len + 7) / 8 * 8;   // the edge granule reads up to a multiple of 8 columns
    return p.off + (K - 1) * p.sb0 + padded <= buffer_elems;
}

int32_t run_flags(const std::vector<DView> &ap, const std::vector<DView> &bp, int64_t K, int64_t b_elems) {
    auto unit_b = [](const std::vector<DView> &v) {
        for (auto &p : v)
            if (p.ib != 1 || (p.sb0 != 1 && p.sb0 != 0)) return false;
        return true;
    };
    auto unit_a = [](const std::vector<DView> &v) {
        for (auto &p : v)
            if (p.ia != 1 || (p.sa0 != 1 && p.len > 1)) return false;
        return true;
    };
    int32_t f = 0;
    if (unit_b(ap)) f |= R_A_KUNIT;
    if (unit_a(ap)) f |= R_A_FUNIT;
    if (unit_b(bp)) f |= R_B_KUNIT;
    if (unit_a(bp)) f |= R_B_FUNIT;
    if (vec_kcontig(ap, K)) f |= R_A_VEC;
    if (vec_kcontig(bp, K)) f |= R_B_VECK;
    if (vec_ncontig(bp, K, b_elems)) f |= R_B_VECN;
    return f;
}

struct Trip {
    int32_t m, k, n;
    int32_t ai, bi, ci;
};

struct GroupSpec {
    std::vector<int32_t> rows, cols;      // member m keys / n keys
    std::vector<int32_t> ks;              // contracted keys (ascending)
    std::vector<int32_t> cblk;            // C block per (row, col) member pair, row-major
    bool accumulate = false;
};

}  // namespace

bsc_status build_plan(Plan &p, const bsc_index *m, const bsc_index *k, const bsc_index *n,
                      const bsc_operand *A, const bsc_operand *B, const bsc_operand *C) {
    try {
        if (!m) fail(BSC_ERR_ARG, "index m is NULL");
        if (m->nq < 1) fail(BSC_ERR_ARG, "index m: charge arity must be >= 1");
        const int32_t nq = m->nq;
        p.nq = nq;
        Idx im = copy_index(m, "m", nq), ik = copy_index(k, "k", nq), in = copy_index(n, "n", nq);
        p.dm = im.dim;
        p.dk = ik.dim;
        p.dn = in.dim;
        std::vector<int32_t> fa, fb, fc;
        p.A = copy_operand(A, "A", im, ik, nq, p.a_elems, fa);
        p.B = copy_operand(B, "B", ik, in, nq, p.b_elems, fb);
        p.C = copy_operand(C, "C", im, in, nq, p.c_elems, fc);
        for (int32_t j = 0; j < nq; ++j)
            if ((int64_t)fa[j] + fb[j] != fc[j]) fail(BSC_ERR_CHARGE, "flux_C != flux_A + flux_B");
        check_c_disjoint(p.C, p.dm, p.dn);

        const bool per_sector = p.opt.launch_mode == BSC_LAUNCH_PER_SECTOR;
        if (!per_sector && p.axis == BSC_AXIS_NONE)
            fail(BSC_ERR_ARG, "axis NONE needs the per-sector launch mode");

        // ---- sector join on k --------------------------------------------------
        std::vector<std::vector<int32_t>> b_by_k((size_t)ik.nkeys);
        for (size_t i = 0; i < p.B.size(); ++i) b_by_k[(size_t)p.B[i].r].push_back((int32_t)i);
        std::unordered_map<uint64_t, int32_t> cmap;
        cmap.reserve(p.C.size() * 2 + 1);
        for (size_t i = 0; i < p.C.size(); ++i)
            cmap[((uint64_t)(uint32_t)p.C[i].r << 32) | (uint32_t)p.C[i].c] = (int32_t)i;
        std::vector<Trip> trips;
        for (size_t ai = 0; ai < p.A.size(); ++ai) {
            const Blk &a = p.A[ai];
            for (int32_t bi : b_by_k[(size_t)a.c]) {
                int32_t nn = p.B[(size_t)bi].c;
                auto it = cmap.find(((uint64_t)(uint32_t)a.r << 32) | (uint32_t)nn);
                if (it == cmap.end())
                    fail(BSC_ERR_MISSING_OUTPUT, "product sector (m=" + std::to_string(a.r) + ", n=" + std::to_string(nn) +
                                                     ") has no C block");
                trips.push_back({a.r, a.c, nn, (int32_t)ai, bi, it->second});
            }
        }
        std::sort(trips.begin(), trips.end(), [](const Trip &x, const Trip &y) {
            if (x.m != y.m) return x.m < y.m;
            if (x.n != y.n) return x.n < y.n;
            return x.k < y.k;
        });
        p.triples.resize(trips.size());
        int64_t flops = 0, tail = 0;
        for (size_t i = 0; i < trips.size(); ++i) {
            p.triples[i] = {trips[i].m, trips[i].k, trips[i].n};
            int64_t f = 2 * p.dm[trips[i].m] * p.dk[trips[i].k] * p.dn[trips[i].n];
            flops += f;
            if (f <= 1024) ++tail;
        }

        // C blocks with their k-lists: contiguous stretches of the sorted triples
        struct CL {
            int32_t m, n, ci;
            size_t t0, t1;
        };
        std::vector<CL> cls;
        for (size_t i = 0; i < trips.size();) {
            size_t j = i;
            while (j < trips.size() && trips[j].m == trips[i].m && trips[j].n == trips[i].n) ++j;
            cls.push_back({trips[i].m, trips[i].n, trips[i].ci, i, j});
            i = j;
        }
        std::vector<char> c_has_work(p.C.size(), 0);
        for (auto &c : cls) c_has_work[(size_t)c.ci] = 1;

        // ---- single-axis grouping ------------------------------------------------
        int32_t axis = p.axis;
        auto klist = [&](const CL &c) {
            std::vector<int32_t> v;
            for (size_t t = c.t0; t < c.t1; ++t) v.push_back(trips[t].k);
            return v;
        };
        if (per_sector) {
            axis = BSC_AXIS_NONE;
        } else if (axis == BSC_AXIS_AUTO) {
            size_t multi = 0;
            for (auto &c : cls) multi += (c.t1 - c.t0) > 1;
            if (!cls.empty() && 4 * multi > cls.size()) {
                axis = BSC_AXIS_CONTRACT;
            } else {
                std::map<std::pair<int32_t, std::vector<int32_t>>, int> gm, gn;
                for (auto &c : cls) {
                    auto kl = klist(c);
                    gm[{c.n, kl}] = 1;
                    gn[{c.m, kl}] = 1;
                }
                axis = gm.size() <= gn.size() ? BSC_AXIS_FREE_M : BSC_AXIS_FREE_N;
            }
        }
        p.axis = axis;

        std::vector<GroupSpec> specs;
        std::vector<int32_t> gid_of_cl(cls.size(), -1);
        if (axis == BSC_AXIS_NONE) {
            for (size_t c = 0; c < cls.size(); ++c)
                for (size_t t = cls[c].t0; t < cls[c].t1; ++t) {
                    GroupSpec g;
                    g.rows = {trips[t].m};
                    g.cols = {trips[t].n};
                    g.ks = {trips[t].k};
                    g.cblk = {trips[t].ci};
                    g.accumulate = p.opt.accumulate != 0 || t > cls[c].t0;
                    specs.push_back(std::move(g));
                }
        } else if (axis == BSC_AXIS_CONTRACT) {
            for (size_t c = 0; c < cls.size(); ++c) {
                GroupSpec g;
                g.rows = {cls[c].m};
                g.cols = {cls[c].n};
                g.ks = klist(cls[c]);
                g.cblk = {cls[c].ci};
                g.accumulate = p.opt.accumulate != 0;
                gid_of_cl[c] = (int32_t)specs.size();
                specs.push_back(std::move(g));
            }
        } else if (axis == BSC_AXIS_FREE_M || axis == BSC_AXIS_FREE_N) {
            const bool fm = axis == BSC_AXIS_FREE_M;
            std::map<std::pair<int32_t, std::vector<int32_t>>, std::vector<size_t>> bucket;
            for (size_t c = 0; c < cls.size(); ++c) bucket[{fm ? cls[c].n : cls[c].m, klist(cls[c])}].push_back(c);
            struct Tmp {
                int32_t key, first;
                std::vector<size_t> members;
                std::vector<int32_t> ks;
            };
            std::vector<Tmp> tmp;
            for (auto &kv : bucket) {
                std::vector<size_t> mem = kv.second;
                std::sort(mem.begin(), mem.end(), [&](size_t x, size_t y) {
                    return fm ? cls[x].m < cls[y].m : cls[x].n < cls[y].n;
                });
                int32_t first = fm ? cls[mem[0]].m : cls[mem[0]].n;
                tmp.push_back({kv.first.first, first, mem, kv.first.second});
            }
            std::sort(tmp.begin(), tmp.end(), [](const Tmp &x, const Tmp &y) {
                return x.key != y.key ? x.key < y.key : x.first < y.first;
            });
            for (auto &t : tmp) {
                GroupSpec g;
                g.ks = t.ks;
                for (size_t c : t.members) {
                    if (fm) g.rows.push_back(cls[c].m);
                    else g.cols.push_back(cls[c].n);
                    g.cblk.push_back(cls[c].ci);
                    gid_of_cl[c] = (int32_t)specs.size();
                }
                if (fm) g.cols = {t.key};
                else g.rows = {t.key};
                g.accumulate = p.opt.accumulate != 0;
                specs.push_back(std::move(g));
            }
        } else {
            fail(BSC_ERR_ARG, "unknown axis");
        }

        // triple -> group
        p.group_of_triple.assign(trips.size(), -1);
        if (axis == BSC_AXIS_NONE) {
            for (size_t t = 0; t < trips.size(); ++t) p.group_of_triple[t] = (int32_t)t;
        } else {
            for (size_t c = 0; c < cls.size(); ++c)
                for (size_t t = cls[c].t0; t < cls[c].t1; ++t) p.group_of_triple[t] = gid_of_cl[c];
        }

        // zero-fill groups (overwrite mode): listed C blocks nothing contributes to
        int64_t zero_blocks = 0;
        std::vector<int32_t> zero_c;
        for (size_t i = 0; i < p.C.size(); ++i)
            if (!c_has_work[i]) {
                ++zero_blocks;
                if (!p.opt.accumulate) zero_c.push_back((int32_t)i);
            }

        // ---- pieces, runs and groups ---------------------------------------------
        std::unordered_map<uint64_t, int32_t> amap, bmap;
        amap.reserve(p.A.size() * 2 + 1);
        bmap.reserve(p.B.size() * 2 + 1);
        for (size_t i = 0; i < p.A.size(); ++i) amap[((uint64_t)(uint32_t)p.A[i].r << 32) | (uint32_t)p.A[i].c] = (int32_t)i;
        for (size_t i = 0; i < p.B.size(); ++i) bmap[((uint64_t)(uint32_t)p.B[i].r << 32) | (uint32_t)p.B[i].c] = (int32_t)i;
        auto akey = [](int32_t r, int32_t c) { return ((uint64_t)(uint32_t)r << 32) | (uint32_t)c; };

        p.groups.clear();
        p.runs.clear();
        p.apieces.clear();
        p.bpieces.clear();
        p.cpieces.clear();
        p.group_mode.clear();
        const int64_t LIM = (int64_t(1) << 31) - 1;
        p.packs.clear();
        p.pack_tasks.clear();
        p.ws_elems = 0;

        // Whether an operand of a group, as per-k-segment piece lists, is one
        // strided view over the group's whole free x contracted extent (the
        // view in v when it is).
        auto merged_view = [&](const std::vector<std::vector<DView>> &seg, const std::vector<int64_t> &segK,
                               DView &v) {
            v = DView{};
            int64_t kk = 0;
            for (size_t s = 0; s < seg.size(); ++s) {
                if (seg[s].size() != 1) return false;
                if (s == 0) v = seg[s][0];
                else if (!merge_along_b(v, kk, seg[s][0], segK[s])) return false;
                kk += segK[s];
            }
            return !seg.empty();
        };
        auto one_view = [&](const std::vector<std::vector<DView>> &seg, const std::vector<int64_t> &segK) {
            DView v;
            return merged_view(seg, segK, v);
        };
        // Pack-cost-versus-savings model (uni20 "block coalescing", section
        // "Interleaved vs contiguous — the real tradeoff is a copy", and the
        // launch-cost crossover of its open questions).  All times are whole-GPU
        // microseconds.  Gathering operand X of a group costs its traffic,
        // 2 * bytes / pack_gbps (read once, written once).  It saves, on each of
        // the group's output tiles, the set-up of every piece beyond one per
        // k-segment (t_seg_us each; tiles run CONCURRENT_TILES at a time), and
        // the matrix-core K-step padding of the k-segments it fuses
        // (pad flops / tile_gflops).  The one extra launch a plan with gathers
        // needs is charged afterwards, against the sum over all packed operands.
        const double concurrent = CONCURRENT_TILES;
        const int64_t esz = p.dtype == BSC_F64 ? 8 : (p.dtype == BSC_F32 ? 4 : 2);
        const int64_t kq = p.dtype == BSC_BF16_F32 ? 16 : 4;     // matrix-core K step
        double pack_net_us = 0;                                   // sum of savings - gather costs
        auto decide_pack = [&](const DGroup &dg, const std::vector<std::vector<DView>> &seg,
                               const std::vector<int64_t> &segK, bool is_a) -> bool {
            if (p.opt.layout_policy == BSC_LAYOUT_NEVER_PACK) return false;
            if (one_view(seg, segK)) return false;   // already zero-copy and single-view
            const int64_t free = is_a ? dg.M : dg.N;
            const int64_t other = is_a ? dg.N : dg.M;
            const int64_t T = p.dtype == BSC_BF16_F32 ? TILE_MFMA : TILE_MFMA_F;
            const int64_t tiles = ((dg.M + T - 1) / T) * ((dg.N + T - 1) / T);
            int64_t pieces = 0, pad = 0;
            for (size_t s = 0; s < seg.size(); ++s) {
                pieces += (int64_t)seg[s].size();
                pad += (segK[s] + kq - 1) / kq * kq - segK[s];
            }
            const int64_t pad_after = ((int64_t)dg.K + kq - 1) / kq * kq - dg.K;
            const double extra = (double)(pieces - 1);
            const double gain_seg = (double)tiles * extra * p.opt.t_seg_us / concurrent;
            const double gain_pad = 2.0 * (double)free * (double)other *
                                    (double)std::max<int64_t>(0, pad - pad_after) / (p.opt.tile_gflops * 1e3);
            const double cost = 2.0 * (double)(free * dg.K * esz) / (p.opt.pack_gbps * 1e3);
            if (p.opt.layout_policy != BSC_LAYOUT_FORCE_PACK && gain_seg + gain_pad <= cost) return false;
            pack_net_us += gain_seg + gain_pad - cost;
            p.gain_seg_us += gain_seg;
            p.gain_pad_us += gain_pad;
            p.pack_cost_us += cost;
            return true;
        };
        // Alignment gathers (bf16).  The direct-to-LDS tile copies 16-byte
        // granules, so it takes a group only when A is one view with K-contiguous
        // rows and B one view with N- or K-contiguous lines, every line starting
        // on a 16-byte boundary.  A group that is single views but misaligned
        // (blocks stored back to back with odd extents, as nothing pads them)
        // runs on the register-staged general tile (128 x 128) instead, whose
        // K chunks each hold a tile slot ALIGN_CHUNK_US longer than the direct
        // tile needs for the same work.  Gathering the misaligned operands into
        // 16-byte rows costs their traffic and saves that time on every chunk
        // of every general tile of the group (tiles run CONCURRENT_TILES at a
        // time).  Decides both operands of the group.
        auto decide_align = [&](const DGroup &dg, const GroupSpec &g, const std::vector<std::vector<DView>> &sa,
                                const std::vector<std::vector<DView>> &sb, const std::vector<int64_t> &segK,
                                bool &pa, bool &pb) {
            pa = pb = false;
            if (per_sector || p.dtype != BSC_BF16_F32 || p.opt.layout_policy == BSC_LAYOUT_NEVER_PACK) return;
            if (std::min(dg.M, dg.N) <= TILE_SKINNY_SHORT || (int64_t)dg.M * dg.N * dg.K < 32 * 32 * 16) return;
            if (g.rows.size() != 1 || g.cols.size() != 1) return;
            const Blk &cb = p.C[(size_t)g.cblk[0]];
            if (cb.ri != 1 || cb.ci != 1) return;   // the dense tile writes a single-leg C view
            DView va, vb;
            if (!merged_view(sa, segK, va) || !merged_view(sb, segK, vb) || va.ia != 1 || vb.ia != 1) return;
            const bool a_ok = vec_kcontig({va}, dg.K);
            const bool b_ok = vec_ncontig({vb}, dg.K, p.b_elems) || vec_kcontig({vb}, dg.K);
            if (a_ok && b_ok) return;
            const double tiles = (double)((dg.M + TILE_MFMA - 1) / TILE_MFMA) * ((dg.N + TILE_MFMA - 1) / TILE_MFMA);
            const double gain = tiles * (double)((dg.K + ALIGN_CHUNK_K - 1) / ALIGN_CHUNK_K) * ALIGN_CHUNK_US / concurrent;
            const double cost = 2.0 * (double)((a_ok ? 0 : (int64_t)dg.M * dg.K) + (b_ok ? 0 : (int64_t)dg.N * dg.K)) *
                                esz / (p.opt.pack_gbps * 1e3);
            if (p.opt.layout_policy != BSC_LAYOUT_FORCE_PACK && gain <= cost) return;
            pa = !a_ok;
            pb = !b_ok;
            pack_net_us += gain - cost;
            p.gain_align_us += gain;
            p.pack_cost_us += cost;
        };
        // Gather an operand into a fresh workspace region with a constant
        // leading dimension (rounded up to 8 elements: 16-byte rows for every
        // dtype).  The destination keeps the unit-stride axis most source bytes
        // have, so the copy stays coalesced on both sides: k-major
        // [free][ld >= K] or free-major [K][ld >= free].  bf16 A is always
        // k-major, the layout of the direct-to-LDS matrix-core tile.  Returns the
        // new per-segment pieces (one workspace piece per k-segment).
        auto pack_operand = [&](const std::vector<std::vector<DView>> &seg, const std::vector<int64_t> &segK,
                                int64_t free, int64_t K, int32_t src) {
            int64_t kbytes = 0, fbytes = 0;
            for (size_t s = 0; s < seg.size(); ++s)
                for (const DView &v : seg[s]) {
                    if (v.ib == 1 && v.sb0 == 1 && segK[s] > 1) kbytes += (int64_t)v.len * segK[s];
                    if (v.ia == 1 && v.sa0 == 1 && v.len > 1) fbytes += (int64_t)v.len * segK[s];
                }
            const bool kmajor = (p.dtype == BSC_BF16_F32 && src == 0) || kbytes >= fbytes;
            const int64_t ld = kmajor ? (K + 7) / 8 * 8 : (free + 7) / 8 * 8;
            if (ld > LIM) fail(BSC_ERR_UNSUPPORTED, "a packed operand's leading dimension exceeds 2^31-1");
            const int64_t base = (p.ws_elems + 63) / 64 * 64;
            p.ws_elems = base + (kmajor ? free : K) * ld;
            std::vector<std::vector<DView>> out(seg.size());
            int64_t kb = 0;
            for (size_t s = 0; s < seg.size(); ++s) {
                for (const DView &v : seg[s]) {
                    DPack d{};
                    d.off = v.off;
                    d.sa0 = v.sa0; d.sa1 = v.sa1; d.ia = v.ia;
                    d.sb0 = v.sb0; d.sb1 = v.sb1; d.ib = v.ib;
                    d.rows = v.len;
                    d.cols = (int32_t)segK[s];
                    d.dst = kmajor ? base + (int64_t)v.begin * ld + kb : base + kb * ld + v.begin;
                    d.ld = (int32_t)ld;
                    d.src = src;
                    d.dmode = kmajor ? 0 : 1;
                    const int32_t gi = (int32_t)p.packs.size();
                    p.packs.push_back(d);
                    int32_t tr = 0, tc = 0;
                    const int32_t mode = pack_mode(d);
                    pack_tile(d.rows, d.cols, mode, pack_big(p.dtype == BSC_BF16_F32 ? 2 : 4, mode), tr, tc);
                    for (int32_t x0 = 0; x0 < d.rows; x0 += tr)
                        for (int32_t y0 = 0; y0 < d.cols; y0 += tc) p.pack_tasks.push_back({0, gi, x0, y0});
                }
                DView w{};
                w.ia = w.ib = 1;
                w.begin = 0;
                w.len = (int32_t)free;
                if (kmajor) {
                    w.off = base + kb;
                    w.sa0 = free > 1 ? ld : 0;
                    w.sb0 = segK[s] > 1 ? 1 : 0;
                } else {
                    w.off = base + kb * ld;
                    w.sa0 = free > 1 ? 1 : 0;
                    w.sb0 = segK[s] > 1 ? ld : 0;
                }
                out[s].push_back(w);
                kb += segK[s];
            }
            return out;
        };

        for (auto &g : specs) {
            DGroup dg{};
            int64_t M = 0, N = 0, K = 0;
            std::vector<int32_t> rbeg, cbeg;
            for (int32_t r : g.rows) { rbeg.push_back((int32_t)M); M += p.dm[r]; }
            for (int32_t c : g.cols) { cbeg.push_back((int32_t)N); N += p.dn[c]; }
            for (int32_t kk : g.ks) K += p.dk[kk];
            if (M > LIM || N > LIM || K > LIM) fail(BSC_ERR_UNSUPPORTED, "a coalesced GEMM extent exceeds 2^31-1");
            dg.M = (int32_t)M;
            dg.N = (int32_t)N;
            dg.K = (int32_t)K;
            dg.flags = g.accumulate ? G_ACCUMULATE : 0;
            // per-segment pieces
            std::vector<std::vector<DView>> segA, segB;
            std::vector<int64_t> segK;
            for (int32_t kk : g.ks) {
                std::vector<DView> am, bm;
                for (size_t i = 0; i < g.rows.size(); ++i) {
                    const Blk &b = p.A[(size_t)amap.at(akey(g.rows[i], kk))];
                    am.push_back(piece_of(b, true, rbeg[i], (int32_t)p.dm[g.rows[i]]));
                }
                for (size_t j = 0; j < g.cols.size(); ++j) {
                    const Blk &b = p.B[(size_t)bmap.at(akey(kk, g.cols[j]))];
                    bm.push_back(piece_of(b, false, cbeg[j], (int32_t)p.dn[g.cols[j]]));
                }
                segA.push_back(stack(am));
                segB.push_back(stack(bm));
                segK.push_back(p.dk[kk]);
            }
            // operand arrangement: the zero-copy pieces, or one gather into the workspace
            bool align_a = false, align_b = false;
            decide_align(dg, g, segA, segB, segK, align_a, align_b);
            const bool pack_a = align_a || (!per_sector && decide_pack(dg, segA, segK, true));
            const bool pack_b = align_b || (!per_sector && decide_pack(dg, segB, segK, false));
            if (pack_a) segA = pack_operand(segA, segK, dg.M, dg.K, 0);
            if (pack_b) segB = pack_operand(segB, segK, dg.N, dg.K, 1);
            // merge consecutive segments into runs while both operands continue as one view
            dg.run0 = (int32_t)p.runs.size();
            bool a_view = true, b_view = true;
            int64_t kbase = 0;
            for (size_t s = 0; s < segA.size();) {
                std::vector<DView> ra = segA[s], rb = segB[s];
                int64_t rk = segK[s];
                size_t e = s + 1;
                while (e < segA.size()) {
                    if (segA[e].size() != ra.size() || segB[e].size() != rb.size()) break;
                    std::vector<DView> ta = ra, tb = rb;
                    bool ok = true;
                    for (size_t i = 0; i < ta.size() && ok; ++i) ok = merge_along_b(ta[i], rk, segA[e][i], segK[e]);
                    for (size_t j = 0; j < tb.size() && ok; ++j) ok = merge_along_b(tb[j], rk, segB[e][j], segK[e]);
                    if (!ok) break;
                    ra.swap(ta);
                    rb.swap(tb);
                    rk += segK[e];
                    ++e;
                }
                DRun r{};
                r.K = (int32_t)rk;
                r.kbase = (int32_t)kbase;
                r.nap = (int32_t)ra.size();
                r.ap0 = (int32_t)p.apieces.size();
                r.nbp = (int32_t)rb.size();
                r.bp0 = (int32_t)p.bpieces.size();
                r.flags = run_flags(ra, rb, rk, pack_b ? p.ws_elems : p.b_elems);
                if (pack_a) r.flags |= R_A_WS;
                if (pack_b) r.flags |= R_B_WS;
                a_view = a_view && ra.size() == 1;
                b_view = b_view && rb.size() == 1;
                p.apieces.insert(p.apieces.end(), ra.begin(), ra.end());
                p.bpieces.insert(p.bpieces.end(), rb.begin(), rb.end());
                p.runs.push_back(r);
                kbase += rk;
                s = e;
            }
            dg.nrun = (int32_t)p.runs.size() - dg.run0;
            // C pieces
            std::vector<DView> cm;
            const bool along_n = g.cols.size() > 1;
            for (size_t i = 0; i < g.rows.size(); ++i)
                for (size_t j = 0; j < g.cols.size(); ++j) {
                    const Blk &b = p.C[(size_t)g.cblk[i * g.cols.size() + j]];
                    if (along_n) cm.push_back(piece_of(b, false, cbeg[j], (int32_t)p.dn[g.cols[j]]));
                    else cm.push_back(piece_of(b, true, rbeg[i], (int32_t)p.dm[g.rows[i]]));
                }
            std::vector<DView> cp = stack(cm);
            dg.ncp = (int32_t)cp.size();
            dg.cp0 = (int32_t)p.cpieces.size();
            if (along_n) dg.flags |= G_C_ALONG_N;
            p.cpieces.insert(p.cpieces.end(), cp.begin(), cp.end());
            p.groups.push_back(dg);
            p.group_mode.push_back({pack_a ? BSC_MODE_PACK : a_view ? BSC_MODE_VIEW : BSC_MODE_SEGMENTS,
                                    pack_b ? BSC_MODE_PACK : b_view ? BSC_MODE_VIEW : BSC_MODE_SEGMENTS,
                                    cp.size() == 1 ? BSC_MODE_VIEW : BSC_MODE_SEGMENTS});
        }
        p.n_work_groups = (int32_t)p.groups.size();
        for (int32_t ci : zero_c) {
            const Blk &b = p.C[(size_t)ci];
            DGroup dg{};
            dg.M = (int32_t)p.dm[b.r];
            dg.N = (int32_t)p.dn[b.c];
            dg.K = 0;
            dg.nrun = 0;
            dg.run0 = (int32_t)p.runs.size();
            dg.ncp = 1;
            dg.cp0 = (int32_t)p.cpieces.size();
            p.cpieces.push_back(piece_of(b, true, 0, dg.M));
            p.groups.push_back(dg);
        }

        // ---- tasks ------------------------------------------------------------------
        p.tasks.clear();
        p.fast.clear();
        p.tail.clear();
        p.launches.clear();
        p.n_counters = 0;
        p.part_elems = 0;
        p.split_tiles = 0;
        // Direct-to-LDS bf16 tiles of this plan: the 256 x 128 tile, two workgroups
        // per CU, or the wide tile, one workgroup per CU with the whole LDS
        // (tile_cols option; 0 = the engine's choice).
        const bool wide = !per_sector && p.dtype == BSC_BF16_F32 && p.opt.tile_cols == TILE_WIDE;
        // tile class per group: matrix-core tiles where the group is more than a
        // single instruction's worth of work, vector-ALU tiles for the tiny tail
        auto class_of = [&](const DGroup &g) -> int32_t {
            if (g.nrun == 0) return T_ZERO;
            // at most 16 output rows or columns: a bandwidth-bound stream over the long operand
            // (the long operand's pieces must have a single contracted leg)
            if (std::min(g.M, g.N) <= TILE_SKINNY_SHORT) {
                const bool long_m = g.M >= g.N;
                bool single_k = true;
                for (int32_t r = 0; r < g.nrun && single_k; ++r) {
                    const DRun &run = p.runs[(size_t)(g.run0 + r)];
                    const std::vector<DView> &pcs = long_m ? p.apieces : p.bpieces;
                    const int32_t first = long_m ? run.ap0 : run.bp0, cnt = long_m ? run.nap : run.nbp;
                    for (int32_t i = 0; i < cnt && single_k; ++i) single_k = pcs[(size_t)(first + i)].ib == 1;
                }
                if (single_k) return long_m ? T_SKINNY_M : T_SKINNY_N;
            }
            if (p.dtype != BSC_BF16_F32) {
                // fp32 / fp64: 16 x 16 x 4 matrix-core steps once both free extents reach half a step
                return ((int64_t)g.M * g.N * g.K >= 16 * 16 * 16 && g.M >= 8 && g.N >= 8) ? T_MFMA : T_GENERIC;
            }
            if ((int64_t)g.M * g.N * g.K >= 32 * 32 * 16 && g.M >= 8 && g.N >= 8) {
                // dense tile: one run, one piece per operand, single-leg views, 16-byte vectors
                if (g.nrun == 1 && g.ncp == 1) {
                    const DRun &r = p.runs[(size_t)g.run0];
                    const DView &c = p.cpieces[(size_t)g.cp0];
                    const bool single = r.nap == 1 && r.nbp == 1 && c.ia == 1 && c.ib == 1 &&
                                        p.apieces[(size_t)r.ap0].ia == 1 && p.bpieces[(size_t)r.bp0].ia == 1;
                    if (single && (r.flags & R_A_VEC) && (r.flags & R_B_VECN)) return wide ? T_MFMA_WIDE_N : T_MFMA_FAST_N;
                    if (single && (r.flags & R_A_VEC) && (r.flags & R_B_VECK)) return wide ? T_MFMA_WIDE_K : T_MFMA_FAST_K;
                }
                return T_MFMA;
            }
            return T_GENERIC;
        };
        // The record of a tile whose A rows, B columns and C block each lie in one
        // single-leg view of a one-run group (false otherwise).
        auto dense_record = [&](const DGroup &g, int32_t gi, int32_t m0, int32_t ml, int32_t n0, int32_t nl,
                                DFast &f) -> bool {
            if (g.nrun != 1) return false;
            const DRun &r = p.runs[(size_t)g.run0];
            auto piece_at = [](const std::vector<DView> &pc, int32_t first, int32_t n, int32_t x0, int32_t len,
                               const DView *&out) {
                for (int32_t i = 0; i < n; ++i) {
                    const DView &v = pc[(size_t)(first + i)];
                    if (v.begin <= x0 && x0 + len <= v.begin + v.len) {
                        if (v.ia != 1 || v.ib != 1) return false;
                        out = &v;
                        return true;
                    }
                }
                return false;
            };
            const bool cn = (g.flags & G_C_ALONG_N) != 0;
            const DView *a = nullptr, *b = nullptr, *c = nullptr;
            if (!piece_at(p.apieces, r.ap0, r.nap, m0, ml, a)) return false;
            if (!piece_at(p.bpieces, r.bp0, r.nbp, n0, nl, b)) return false;
            if (!piece_at(p.cpieces, g.cp0, g.ncp, cn ? n0 : m0, cn ? nl : ml, c)) return false;
            f.a_base = a->off + (int64_t)(m0 - a->begin) * a->sa0;
            f.a_rs = a->sa0;
            f.a_ks = a->sb0;
            f.b_base = b->off + (int64_t)(n0 - b->begin) * b->sa0;
            f.b_ns = b->sa0;
            f.b_ks = b->sb0;
            // C piece axis a is rows (or columns when cut along N)
            f.c_rs = cn ? c->sb0 : c->sa0;
            f.c_cs = cn ? c->sa0 : c->sb0;
            f.c_base = c->off + (int64_t)(m0 - (cn ? 0 : c->begin)) * f.c_rs + (int64_t)(n0 - (cn ? c->begin : 0)) * f.c_cs;
            f.mlen = ml;
            f.nlen = nl;
            f.K = r.K;
            f.group = gi;
            f.flags = (g.flags & G_ACCUMULATE) | ((r.flags & R_A_WS) ? F_A_WS : 0) | ((r.flags & R_B_WS) ? F_B_WS : 0);
            f.nsplit = 1;
            return true;
        };
        // Skinny groups of one run whose views are all single-leg become items
        // addressed through records: the long axis is cut at every piece boundary
        // of the long operand and of C (and every skinny_long lines), so each item
        // lies in one view of each operand.  Returns false (nothing emitted) when
        // the group does not qualify.
        auto skinny_records = [&](const DGroup &g, int32_t gi, bool long_m, std::vector<DTask> &out,
                                  std::vector<double> *cost) -> bool {
            if (g.nrun != 1) return false;
            const DRun &r = p.runs[(size_t)g.run0];
            const bool cn = (g.flags & G_C_ALONG_N) != 0;
            const bool c_long = long_m ? !cn : cn;
            const int32_t lfirst = long_m ? r.ap0 : r.bp0, lcnt = long_m ? r.nap : r.nbp;
            const int32_t sfirst = long_m ? r.bp0 : r.ap0, scnt = long_m ? r.nbp : r.nap;
            const std::vector<DView> &lp = long_m ? p.apieces : p.bpieces;
            const std::vector<DView> &sp = long_m ? p.bpieces : p.apieces;
            auto single = [](const DView &v) { return v.ia == 1 && v.ib == 1; };
            if (scnt != 1 || !single(sp[(size_t)sfirst])) return false;
            if (!c_long && g.ncp != 1) return false;
            std::vector<int32_t> cuts;
            for (int32_t i = 0; i < lcnt; ++i) {
                if (!single(lp[(size_t)(lfirst + i)])) return false;
                cuts.push_back(lp[(size_t)(lfirst + i)].begin);
            }
            for (int32_t i = 0; i < g.ncp; ++i) {
                const DView &c = p.cpieces[(size_t)(g.cp0 + i)];
                if (!single(c)) return false;
                if (c_long) cuts.push_back(c.begin);
            }
            const int32_t X = long_m ? g.M : g.N, Y = long_m ? g.N : g.M;
            cuts.push_back(X);
            std::sort(cuts.begin(), cuts.end());
            cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
            const int32_t ext = skinny_long(p.dtype, Y);
            const DView &s = sp[(size_t)sfirst];
            int32_t li = 0, ci = 0;
            for (size_t q = 0; q + 1 < cuts.size(); ++q) {
                for (int32_t x0 = cuts[q]; x0 < cuts[q + 1]; x0 += ext) {
                    const int32_t xl = std::min(ext, cuts[q + 1] - x0);
                    while (li + 1 < lcnt && lp[(size_t)(lfirst + li + 1)].begin <= x0) ++li;
                    const DView &l = lp[(size_t)(lfirst + li)];
                    const DView *c = &p.cpieces[(size_t)g.cp0];
                    if (c_long) {
                        while (ci + 1 < g.ncp && p.cpieces[(size_t)(g.cp0 + ci + 1)].begin <= x0) ++ci;
                        c = &p.cpieces[(size_t)(g.cp0 + ci)];
                    }
                    DFast f{};
                    const int64_t lbase = l.off + (int64_t)(x0 - l.begin) * l.sa0;
                    // (tile-local i, j as in every record: i along M, j along N)
                    if (long_m) {
                        f.a_base = lbase; f.a_rs = l.sa0; f.a_ks = l.sb0;
                        f.b_base = s.off; f.b_ns = s.sa0; f.b_ks = s.sb0;
                        f.mlen = xl; f.nlen = Y;
                    } else {
                        f.b_base = lbase; f.b_ns = l.sa0; f.b_ks = l.sb0;
                        f.a_base = s.off; f.a_rs = s.sa0; f.a_ks = s.sb0;
                        f.mlen = Y; f.nlen = xl;
                    }
                    const int32_t cm0 = long_m ? x0 : 0, cn0 = long_m ? 0 : x0;
                    f.c_rs = cn ? c->sb0 : c->sa0;
                    f.c_cs = cn ? c->sa0 : c->sb0;
                    f.c_base = c->off + (int64_t)(cm0 - (cn ? 0 : c->begin)) * f.c_rs + (int64_t)(cn0 - (cn ? c->begin : 0)) * f.c_cs;
                    f.K = r.K;
                    f.group = gi;
                    f.flags = (g.flags & G_ACCUMULATE) | ((r.flags & R_A_WS) ? F_A_WS : 0) | ((r.flags & R_B_WS) ? F_B_WS : 0);
                    out.push_back({long_m ? T_SKINNY_DENSE_M : T_SKINNY_DENSE_N, (int32_t)p.fast.size(), cm0, cn0});
                    p.fast.push_back(f);
                    if (cost) cost->push_back(4.0 * (double)xl * (double)(r.K + Y) + 2.0e4);
                }
            }
            return true;
        };
        // The direct-to-LDS tile addresses each operand of a tile through a buffer
        // descriptor with 32-bit byte offsets: its range must stay below 2 GiB
        // (else the tile runs on the general matrix-core tile).
        auto fast_in_range = [&](int32_t cls, const DFast &f) -> bool {
            if (!is_direct(cls)) return true;
            const double lim = 2147483647.0;
            const double bn = is_wide(cls) ? TILE_WIDE : TILE_MFMA;   // B row extent an N-contiguous copy reads
            const double a = 2.0 * ((double)(f.mlen - 1) * (double)f.a_rs + f.K) + 16;
            const double b = (cls == T_MFMA_FAST_N || cls == T_MFMA_WIDE_N)
                                 ? 2.0 * ((double)(f.K - 1) * (double)f.b_ks + bn) + 16
                                 : 2.0 * ((double)(f.nlen - 1) * (double)f.b_ns + f.K) + 16;
            return f.a_rs >= 0 && f.b_ks >= 0 && f.b_ns >= 0 && a < lim && b < lim;
        };
        // relative throughput of a tile class (used only to order work longest-first)
        auto rate_of = [&](int32_t cls) {
            if (is_direct(cls)) return 48.0;
            if (cls == T_MFMA || cls == T_MFMA_DENSE) return p.dtype == BSC_BF16_F32 ? 16.0 : 4.0;
            return 1.0;
        };
        // K split of the bf16 direct-to-LDS tiles (grouped launches only): a tile
        // whose K chain is much longer than one slot's share of the plan's work
        // would alone set the launch's duration, so it is cut into K-slices of
        // about that share.  Every slice moves a 128 KB partial tile through
        // device-coherent memory and the last one reads them all back, which on
        // MI355X costs more than the shorter chain saves unless the slices stay
        // long: automatic slices are at least SPLIT_MIN_CHUNKS chunks of 32
        // (K >= 2048), so only very long K chains are cut.
        constexpr int32_t SPLIT_CHUNK = 32, SPLIT_MIN_CHUNKS = 64, SPLIT_MAX = 32;
        // one slot's share of the plan's direct-to-LDS work, in 256 x 128 x 32
        // chunks, and the number of such 256 x 128 tiles
        double fast_share = 0, fast_tiles = 0;
        if (!per_sector && p.dtype == BSC_BF16_F32) {
            double total = 0;
            for (int32_t gi = 0; gi < p.n_work_groups; ++gi) {
                const DGroup &g = p.groups[(size_t)gi];
                const int32_t cls = class_of(g);
                if (!is_direct(cls)) continue;
                int32_t TM = 0, TN = 0;
                tile_extents(p.dtype, cls, g.M, g.N, TM, TN);
                const double tiles = (double)((g.M + TM - 1) / TM) * (double)((g.N + TN - 1) / TN);
                fast_tiles += tiles;
                total += tiles * (double)((g.K + SPLIT_CHUNK - 1) / SPLIT_CHUNK);
            }
            // tiles in flight at once: two per CU, or one per CU for the wide tile
            fast_share = total / (wide ? CONCURRENT_TILES / 2 : CONCURRENT_TILES);
        }
        int64_t split_target = 0;   // most chunks per slice; 0: no split
        if (!per_sector && p.dtype == BSC_BF16_F32 && p.opt.split_k >= 0)
            split_target = p.opt.split_k > 0 ? p.opt.split_k
                                             : std::max<int64_t>(SPLIT_MIN_CHUNKS, (int64_t)std::ceil(fast_share));
        // 128-row tiles: when the plan's 256 x 128 tiles would leave CUs with at
        // most one tile each, a group whose K chain is long (at least 16
        // chunks) and above one slot's share is cut into 128-row tiles: twice
        // the tiles (two per CU), each computed by four 64 x 64 waves with four
        // chunks of copies in flight.  Measured on MI355X: one 1024^3 block
        // 23.7 -> 16.7 us, eight 32.6 -> 29.2 us; with more tiles than CUs the
        // extra tiles only add load (bench workload 31.5 -> 40.3 us), so they
        // stay 256 rows.
        auto half_rows = [&](const DGroup &g) {
            if (p.opt.tile_rows != 0) return p.opt.tile_rows == TILE_MFMA_DENSE_M / 2;
            const int64_t chunks = (g.K + SPLIT_CHUNK - 1) / SPLIT_CHUNK;
            return fast_share > 0 && fast_tiles <= BSC_XCDS * BSC_CUS_PER_XCD && chunks >= 16 &&
                   (double)chunks > 1.5 * fast_share;
        };
        // Wide tiles of at most 128 rows (128 x 256 on eight 64 x 64 waves):
        // the groups whose K chain is far above one CU's share of the launch
        // (the chains that would end last), or every group with tile_rows = 128.
        auto wide_half_rows = [&](const DGroup &g) {
            if (p.opt.tile_rows != 0) return p.opt.tile_rows == TILE_MFMA_DENSE_M / 2;
            const int64_t chunks = (g.K + SPLIT_CHUNK - 1) / SPLIT_CHUNK;
            return fast_share > 0 && chunks >= 16 && (double)chunks > WIDE_HALF_SHARE * fast_share;
        };
        // slices of a tile with K contracted indices (1: no split)
        auto slices_of = [&](int32_t K) -> int32_t {
            if (split_target <= 0) return 1;
            const int64_t chunks = (K + SPLIT_CHUNK - 1) / SPLIT_CHUNK;
            if (p.opt.split_k == 0 && chunks <= 2 * split_target) return 1;   // automatic: only clear wins
            int64_t S = std::min<int64_t>(SPLIT_MAX, (chunks + split_target - 1) / split_target);
            if (S <= 1) return 1;
            const int64_t per = (chunks + S - 1) / S;   // chunks per slice; the last slice takes the rest
            return (int32_t)((chunks + per - 1) / per);
        };
        // Tail groups: near-zero-flop groups (2 M N K <= TAIL_MAX_FLOPS) that are
        // one run of single views, so a single wave computes the whole group from
        // its record (bases and strides) as part of a tail bundle.  Measured on
        // MI355X: tail bundles for every group of at most 256 outputs (records or
        // piece walks) made the U(1) update's W stage slower than its skinny
        // streams (28.0 -> 36.8 us); for near-zero groups the skinny stream's
        // 256-thread workgroup is mostly idle.
        std::vector<std::pair<int32_t, DFast>> tail_groups;
        auto tail_of = [&](const DGroup &g, int32_t gi, DFast &f) -> bool {
            if (per_sector || g.nrun != 1 || 2 * (int64_t)g.M * g.N * g.K > TAIL_MAX_FLOPS) return false;
            if ((int64_t)g.M * g.N > TAIL_MAX_OUT || g.K > TAIL_MAX_K || g.M + g.N > TAIL_STAGE) return false;
            const int32_t mn = g.M * g.N, lanes = tail_lanes_host(mn);
            const int32_t outs = (mn + 64 / lanes - 1) / (64 / lanes);   // outputs per lane
            if ((int64_t)outs * ((g.K + lanes - 1) / lanes) > TAIL_LANE_WORK) return false;
            return dense_record(g, gi, 0, g.M, 0, g.N, f);
        };
        auto tiles_of = [&](int32_t gi, std::vector<DTask> &out, std::vector<double> *cost) {
            const DGroup &g = p.groups[(size_t)gi];
            const int32_t cls = class_of(g);
            {
                DFast f{};
                if (cls != T_ZERO && tail_of(g, gi, f)) {
                    tail_groups.push_back({gi, f});
                    return;
                }
            }
            int32_t TM = 0, TN = 0;
            tile_extents(p.dtype, cls, g.M, g.N, TM, TN);
            if ((cls == T_MFMA_FAST_N || cls == T_MFMA_FAST_K) && half_rows(g)) TM = TILE_MFMA_DENSE_M / 2;
            if (is_wide(cls) && wide_half_rows(g)) TM = TILE_WIDE / 2;
            if ((cls == T_SKINNY_M || cls == T_SKINNY_N) && skinny_records(g, gi, cls == T_SKINNY_M, out, cost)) return;
            for (int32_t m0 = 0; m0 < g.M; m0 += TM)
                for (int32_t n0 = 0; n0 < g.N; n0 += TN) {
                    const int32_t ml = std::min(TM, g.M - m0), nl = std::min(TN, g.N - n0);
                    DFast f{};
                    if ((is_direct(cls) || cls == T_MFMA) &&
                        dense_record(g, gi, m0, ml, n0, nl, f) && fast_in_range(cls, f)) {
                        // bf16 direct-to-LDS tiles always qualify; fp32 / fp64 tiles that do
                        // become record-addressed dense tiles
                        const int32_t c2 = cls == T_MFMA ? (p.dtype == BSC_BF16_F32 ? T_MFMA : T_MFMA_DENSE) : cls;
                        const int32_t S = is_direct(c2) ? slices_of(f.K) : 1;
                        if (S > 1) {
                            // K-slices of SPLIT_CHUNK multiples (only the last may end in a partial chunk)
                            const int32_t chunks = (f.K + SPLIT_CHUNK - 1) / SPLIT_CHUNK;
                            const int32_t per = (chunks + S - 1) / S;
                            const int32_t counter = p.n_counters++;
                            const int64_t part = p.part_elems;
                            // partial tiles of the class's full tile size (the kernel's slice stride)
                            int32_t PTM = 0, PTN = 0;
                            tile_extents(p.dtype, c2, g.M, g.N, PTM, PTN);
                            p.part_elems += (int64_t)S * PTM * PTN;
                            p.split_tiles++;
                            for (int32_t sl = 0; sl < S; ++sl) {
                                DFast fs = f;
                                const int32_t k0 = sl * per * SPLIT_CHUNK;
                                fs.K = std::min(f.K, k0 + per * SPLIT_CHUNK) - k0;
                                fs.a_base += (int64_t)k0 * f.a_ks;
                                fs.b_base += (int64_t)k0 * f.b_ks;
                                fs.split = sl;
                                fs.nsplit = S;
                                fs.counter = counter;
                                fs.part = part;
                                out.push_back({c2, (int32_t)p.fast.size(), m0, n0});
                                p.fast.push_back(fs);
                                if (cost) {
                                    const double mlf = ml, nlf = nl;
                                    // the slice's flops, its partial tile out, and the last slice's reads
                                    cost->push_back((2.0 * mlf * nlf * fs.K) / rate_of(cls) + 8.0 * mlf * nlf + 2.0e4);
                                }
                            }
                            continue;
                        }
                        if (c2 != T_MFMA) {
                            out.push_back({c2, (int32_t)p.fast.size(), m0, n0});
                            p.fast.push_back(f);
                        } else {
                            out.push_back({cls, gi, m0, n0});
                        }
                    } else {
                        // a direct-to-LDS tile without a record or beyond the descriptor range runs on the general tile
                        out.push_back({is_direct(cls) ? T_MFMA : cls, gi, m0, n0});
                    }
                    if (cost) {
                        double ml = std::min(TM, g.M - m0), nl = std::min(TN, g.N - n0);
                        cost->push_back((2.0 * ml * nl * g.K) / rate_of(cls) + 4.0 * ml * nl + 2.0e4 * g.nrun);
                    }
                }
        };
        if (per_sector) {
            for (int32_t gi = 0; gi < p.n_work_groups; ++gi) {
                int32_t t0 = (int32_t)p.tasks.size();
                tiles_of(gi, p.tasks, nullptr);
                p.launches.push_back({t0, (int32_t)p.tasks.size()});
            }
            if ((int32_t)p.groups.size() > p.n_work_groups) {
                int32_t t0 = (int32_t)p.tasks.size();
                for (int32_t gi = p.n_work_groups; gi < (int32_t)p.groups.size(); ++gi) tiles_of(gi, p.tasks, nullptr);
                p.launches.push_back({t0, (int32_t)p.tasks.size()});
            }
        } else {
            // XCD-aware order: each chiplet gets a queue of tiles balanced by cost;
            // a group's tiles stay together (small groups whole, large ones in
            // contiguous row-major slices) so its operand panels are fetched into
            // few L2s.  Each queue runs longest first; queues are interleaved so
            // task t lands on XCD t % BSC_XCDS, padded with no-op tasks.
            std::vector<DTask> tk;
            std::vector<double> cost;
            std::vector<std::pair<size_t, size_t>> span;   // per group: [first, last) task
            for (int32_t gi = 0; gi < (int32_t)p.groups.size(); ++gi) {
                size_t a = tk.size();
                tiles_of(gi, tk, &cost);
                if (tk.size() > a) span.push_back({a, tk.size()});
            }
            // Tail bundles: tiny groups sorted by work, TAIL_BUNDLE consecutive ones
            // per workgroup (one per wave), so the waves of a bundle finish together.
            {
                auto work = [&](int32_t gi) {
                    const DGroup &g = p.groups[(size_t)gi];
                    return 2.0 * g.M * g.N * g.K + 4.0 * g.M * g.N + 2.0e4 * g.nrun;
                };
                std::stable_sort(tail_groups.begin(), tail_groups.end(),
                                 [&](const std::pair<int32_t, DFast> &x, const std::pair<int32_t, DFast> &y) {
                                     return work(x.first) > work(y.first);
                                 });
                for (size_t b = 0; b < tail_groups.size(); b += TAIL_BUNDLE) {
                    const size_t e = std::min(tail_groups.size(), b + TAIL_BUNDLE);
                    const size_t a = tk.size();
                    tk.push_back({T_TAIL, (int32_t)p.tail.size(), (int32_t)(e - b), 0});
                    cost.push_back(work(tail_groups[b].first));
                    for (size_t i = b; i < e; ++i) p.tail.push_back(tail_groups[i].second);
                    span.push_back({a, tk.size()});
                }
            }
            double total = 0;
            for (double c : cost) total += c;
            const double target = total / BSC_XCDS;
            std::vector<double> gcost(span.size(), 0.0);
            for (size_t g = 0; g < span.size(); ++g)
                for (size_t i = span[g].first; i < span[g].second; ++i) gcost[g] += cost[i];
            std::vector<size_t> gord(span.size());
            std::iota(gord.begin(), gord.end(), 0);
            std::stable_sort(gord.begin(), gord.end(), [&](size_t x, size_t y) { return gcost[x] > gcost[y]; });
            std::vector<std::vector<size_t>> q(BSC_XCDS);
            std::vector<double> load(BSC_XCDS, 0.0);
            auto least = [&]() { return (size_t)(std::min_element(load.begin(), load.end()) - load.begin()); };
            // A group of at most one tile per CU of a chiplet stays on one chiplet
            // up to twice a chiplet's share: its tiles then run without partners
            // and share their panels in one L2, and the other chiplets take the
            // rest (bf16 block-diagonal workload: the 32 tiles of its 1024^3 sector
            // on one chiplet, 32.8-33.6 -> 31.7-32.0 us).  Larger groups are cut
            // into contiguous slices of at most half a share.
            for (size_t g : gord) {
                const size_t a = span[g].first, b = span[g].second;
                const size_t ntile = b - a;
                size_t parts = 1;
                const bool whole = ntile <= (size_t)BSC_CUS_PER_XCD && gcost[g] <= 2.0 * target;
                if (!whole && gcost[g] > 0.5 * target)
                    parts = std::min<size_t>({(size_t)BSC_XCDS, ntile, (size_t)std::ceil(gcost[g] / (0.5 * target))});
                for (size_t part = 0; part < parts; ++part) {
                    const size_t lo = a + ntile * part / parts, hi = a + ntile * (part + 1) / parts;
                    const size_t x = least();
                    for (size_t i = lo; i < hi; ++i) {
                        q[x].push_back(i);
                        load[x] += cost[i];
                    }
                }
            }
            // Each queue runs longest first.  Its first BSC_CUS_PER_XCD tiles take a
            // CU each; the next ones become the second residents of those CUs:
            // two tiles on one CU each run slower than one alone, so the longest
            // tiles get no partner (a no-op in that slot) and the remaining
            // partners go to the shortest first residents, longest partner first.
            const size_t CUX = BSC_CUS_PER_XCD;
            constexpr size_t NONE = ~size_t(0);
            std::vector<std::vector<size_t>> slots(BSC_XCDS);
            size_t depth = 0;
            for (int x = 0; x < BSC_XCDS; ++x) {
                std::vector<size_t> &v = q[(size_t)x];
                std::stable_sort(v.begin(), v.end(), [&](size_t a, size_t b) { return cost[a] > cost[b]; });
                std::vector<size_t> &s = slots[(size_t)x];
                if (v.size() <= CUX || wide) {   // wide tiles: one workgroup per CU, plain longest-first
                    s = v;
                } else {
                    s.assign(v.begin(), v.begin() + CUX);
                    s.resize(2 * CUX, NONE);
                    const size_t m = std::min(CUX, v.size() - CUX);   // partners
                    for (size_t i = 0; i < m; ++i) s[CUX + (CUX - 1 - i)] = v[CUX + i];
                    s.insert(s.end(), v.begin() + CUX + m, v.end());
                }
                depth = std::max(depth, s.size());
            }
            for (size_t d = 0; d < depth; ++d)
                for (int x = 0; x < BSC_XCDS; ++x) {
                    const std::vector<size_t> &s = slots[(size_t)x];
                    p.tasks.push_back(d < s.size() && s[d] != NONE ? tk[s[d]] : DTask{T_NOP, 0, 0, 0});
                }
            // trailing no-ops of the last row carry no mapping information
            while (!p.tasks.empty() && p.tasks.back().cls == T_NOP) p.tasks.pop_back();
            if (!p.tasks.empty()) p.launches.push_back({0, (int32_t)p.tasks.size()});
        }
        // Records in task order (record t belongs to task t), so a workgroup
        // reads its task and its record at once instead of one after the other;
        // tasks without a record leave their slot empty.
        {
            std::vector<DFast> by_task(p.tasks.size(), DFast{});
            for (size_t t = 0; t < p.tasks.size(); ++t) {
                DTask &tk = p.tasks[t];
                if (has_record(tk.cls)) {
                    by_task[t] = p.fast[(size_t)tk.group];
                    tk.group = (int32_t)t;
                }
            }
            p.fast.swap(by_task);
        }
        if (p.tasks.size() > (size_t)LIM || p.pack_tasks.size() > (size_t)LIM)
            fail(BSC_ERR_UNSUPPORTED, "too many work items");
        // a plan with gathers needs one more launch: keep them only if they pay for it
        if (!p.packs.empty() && p.opt.layout_policy == BSC_LAYOUT_AUTO && pack_net_us <= p.opt.t_launch_us) {
            p.opt.layout_policy = BSC_LAYOUT_NEVER_PACK;
            p.gain_seg_us = p.gain_pad_us = p.gain_align_us = p.pack_cost_us = 0;
            return build_plan(p, m, k, n, A, B, C);
        }

        // ---- device image --------------------------------------------------------------
        auto align = [](size_t x) { return (x + 255) & ~size_t(255); };
        size_t off = 0;
        p.off_groups = off; off = align(off + p.groups.size() * sizeof(DGroup));
        p.off_runs = off;   off = align(off + p.runs.size() * sizeof(DRun));
        p.off_ap = off;     off = align(off + p.apieces.size() * sizeof(DView));
        p.off_bp = off;     off = align(off + p.bpieces.size() * sizeof(DView));
        p.off_cp = off;     off = align(off + p.cpieces.size() * sizeof(DView));
        p.off_tasks = off;  off = align(off + p.tasks.size() * sizeof(DTask));
        p.off_fast = off;   off = align(off + p.fast.size() * sizeof(DFast));
        p.off_tail = off;   off = align(off + p.tail.size() * sizeof(DFast));
        p.off_packs = off;  off = align(off + p.packs.size() * sizeof(DPack));
        p.off_ptasks = off; off = align(off + p.pack_tasks.size() * sizeof(DTask));
        p.off_cnt = off;    off = align(off + (size_t)p.n_counters * sizeof(int32_t));   // zero in the image
        p.image.assign(std::max<size_t>(off, 256), 0);
        p.off_ws = p.image.size();
        p.off_part = align(p.off_ws + (size_t)(p.ws_elems * esz));
        p.dev_bytes = p.off_part + (size_t)p.part_elems * sizeof(float);
        auto put = [&](size_t o, const void *src, size_t nbytes) { if (nbytes) std::memcpy(p.image.data() + o, src, nbytes); };
        put(p.off_groups, p.groups.data(), p.groups.size() * sizeof(DGroup));
        put(p.off_runs, p.runs.data(), p.runs.size() * sizeof(DRun));
        put(p.off_ap, p.apieces.data(), p.apieces.size() * sizeof(DView));
        put(p.off_bp, p.bpieces.data(), p.bpieces.size() * sizeof(DView));
        put(p.off_cp, p.cpieces.data(), p.cpieces.size() * sizeof(DView));
        put(p.off_tasks, p.tasks.data(), p.tasks.size() * sizeof(DTask));
        put(p.off_fast, p.fast.data(), p.fast.size() * sizeof(DFast));
        put(p.off_tail, p.tail.data(), p.tail.size() * sizeof(DFast));
        put(p.off_packs, p.packs.data(), p.packs.size() * sizeof(DPack));
        put(p.off_ptasks, p.pack_tasks.data(), p.pack_tasks.size() * sizeof(DTask));

        // ---- statistics ---------------------------------------------------------------
        bsc_stats &s = p.stats;
        std::memset(&s, 0, sizeof(s));
        s.triples = (int64_t)trips.size();
        s.c_blocks = (int64_t)p.C.size();
        s.zero_blocks = zero_blocks;
        s.groups = p.n_work_groups;
        s.zero_groups = (int64_t)p.groups.size() - p.n_work_groups;
        s.axis = axis;
        s.dtype = p.dtype;
        for (auto &gm : p.group_mode)
            for (int o = 0; o < 3; ++o) s.mode_count[o][gm[(size_t)o]]++;
        s.runs = (int64_t)p.runs.size();
        s.items = 0;
        for (auto &t : p.tasks) s.items += t.cls != T_NOP;
        p.features = 0;
        p.only_wide = false;
        bool other = false;
        for (auto &t : p.tasks) {
            if (is_wide(t.cls)) p.only_wide = true;
            else if (t.cls != T_TAIL && t.cls != T_NOP) other = true;
        }
        if (other) p.only_wide = false;
        for (auto &t : p.tasks) {
            if (t.cls == T_NOP) continue;
            const int32_t slot = (t.cls == T_MFMA_FAST_K || is_wide(t.cls)) ? T_MFMA_FAST_N
                                 : (t.cls == T_SKINNY_M || t.cls == T_SKINNY_N || t.cls == T_SKINNY_DENSE_M ||
                                    t.cls == T_SKINNY_DENSE_N) ? 5
                                 : t.cls == T_MFMA_DENSE ? T_MFMA : t.cls;
            s.items_by_class[slot]++;
            if (t.cls == T_MFMA || t.cls == T_MFMA_DENSE) p.features |= FEAT_MFMA;
            if (t.cls == T_MFMA_FAST_N) p.features |= FEAT_FAST_N;
            if (t.cls == T_MFMA_FAST_K) p.features |= FEAT_FAST_K;
            if (is_wide(t.cls)) p.features |= FEAT_WIDE;
        }
        s.launches_per_contract = (int64_t)p.launches.size() + (p.packs.empty() ? 0 : 1);
        s.launches_per_sector = s.triples + (zero_c.empty() ? 0 : 1);
        s.useful_flops = flops;
        const int64_t ab = p.dtype == BSC_F64 ? 8 : (p.dtype == BSC_F32 ? 4 : 2);
        const int64_t cb = p.dtype == BSC_F64 ? 8 : 4;
        int64_t ea = 0, eb = 0, ec = 0;
        for (auto &b : p.A) ea += p.dm[b.r] * p.dk[b.c];
        for (auto &b : p.B) eb += p.dk[b.r] * p.dn[b.c];
        for (auto &b : p.C) ec += p.dm[b.r] * p.dn[b.c];
        s.alg_bytes = ab * (ea + eb) + cb * ec;
        s.pack_bytes = 0;
        for (auto &d : p.packs) s.pack_bytes += (int64_t)d.rows * d.cols * ab;
        s.device_bytes = (int64_t)p.dev_bytes;
        s.tail_triples = tail;
        s.split_tiles = p.split_tiles;
        s.pack_gain_seg_us = p.gain_seg_us;
        s.pack_gain_pad_us = p.gain_pad_us;
        s.pack_cost_us = p.pack_cost_us;
        s.pack_gain_align_us = p.gain_align_us;
        s.wide_only = p.only_wide ? 1 : 0;
        const double rate_gflops = p.dtype == BSC_BF16_F32 ? 2.5e6 : (p.dtype == BSC_F32 ? 157.3e3 : 78.6e3);
        s.predicted_us = s.launches_per_contract * p.opt.t_launch_us +
                         std::max((double)flops / (rate_gflops * 1e3), (double)s.alg_bytes / 8.0e6) +
                         2.0 * (double)s.pack_bytes / (p.opt.pack_gbps * 1e3);
        return BSC_OK;
    } catch (const Fail &f) {
        return f.st;
    } catch (const std::bad_alloc &) {
        set_error("out of host memory while planning");
        return BSC_ERR_UNSUPPORTED;
    } catch (const std::exception &e) {
        set_error(std::string("planner: ") + e.what());
        return BSC_ERR_ARG;
    }
}

}  // namespace bsc
