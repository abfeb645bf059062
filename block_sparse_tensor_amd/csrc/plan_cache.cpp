// Plan cache: reuse of coalescing plans across repeated contractions with the
// same block structure (uni20 "block coalescing", "Open questions": caching the
// coalescing groups across DMRG sweeps once the block structure of a site is
// stable).  Planning costs milliseconds of host time (validation, the sector
// join, grouping, the cost model and the work list) while a contraction of an
// environment update runs in tens of microseconds, so a sweep that revisits a
// site should plan it once.
//
// The key is the complete input of bsc_plan, serialized field by field: every
// index table, every operand descriptor (keys, offsets, strides, flux, buffer
// length), the dtype, the axis and every option.  Equal keys give equal plans
// (planning is deterministic), so a hit hands out a copy of the stored plan.
// Keys are compared in full, not by hash alone.
#include <cstring>
#include <list>
#include <mutex>
#include <new>
#include <string>
#include <unordered_map>

#include "bsc_internal.h"

namespace bsc {

namespace {

struct KeyWriter {
    std::string s;
    template <typename T>
    void put(const T &v) {
        s.append(reinterpret_cast<const char *>(&v), sizeof(T));
    }
    template <typename T>
    void arr(const T *p, int64_t n) {
        put(n);
        if (n > 0) s.append(reinterpret_cast<const char *>(p), static_cast<size_t>(n) * sizeof(T));
    }
};

// false when the arguments are malformed (NULL tables, negative counts,
// mismatched nq); bsc_plan then reports the error itself
bool write_index(KeyWriter &w, const bsc_index *x, int32_t nq) {
    if (!x || x->nkeys < 0 || x->nq != nq) return false;
    if (x->nkeys > 0 && (!x->charge || !x->dim)) return false;
    w.put(x->nkeys);
    w.put(x->nq);
    w.arr(x->charge, static_cast<int64_t>(x->nkeys) * nq);
    w.arr(x->dim, static_cast<int64_t>(x->nkeys));
    const int8_t has_inner = x->inner ? 1 : 0;
    w.put(has_inner);
    if (x->inner) w.arr(x->inner, static_cast<int64_t>(x->nkeys));
    return true;
}

bool write_operand(KeyWriter &w, const bsc_operand *o, int32_t nq) {
    if (!o || o->nblocks < 0 || !o->flux) return false;
    if (o->nblocks > 0 && (!o->row_key || !o->col_key || !o->offset || !o->row_stride || !o->col_stride)) return false;
    w.put(o->nblocks);
    w.arr(o->row_key, o->nblocks);
    w.arr(o->col_key, o->nblocks);
    w.arr(o->offset, o->nblocks);
    w.arr(o->row_stride, 2 * o->nblocks);
    w.arr(o->col_stride, 2 * o->nblocks);
    w.arr(o->flux, static_cast<int64_t>(nq));
    w.put(o->buffer_elems);
    return true;
}

void write_options(KeyWriter &w, const bsc_options &o) {
    // field by field: the struct's padding bytes are not part of the key
    w.put(o.launch_mode);
    w.put(o.layout_policy);
    w.put(o.accumulate);
    w.put(o.grid_limit);
    w.put(o.t_launch_us);
    w.put(o.t_seg_us);
    w.put(o.pack_gbps);
    w.put(o.tile_gflops);
    w.put(o.split_k);
    w.put(o.tile_rows);
    w.put(o.tile_cols);
}

}  // namespace

struct PlanCache {
    std::mutex mu;
    int32_t capacity = 0;
    std::list<std::string> lru;   // most recently used first
    struct Entry {
        Plan plan;
        std::list<std::string>::iterator pos;
    };
    std::unordered_map<std::string, Entry> map;
    int64_t hits = 0, misses = 0;
};

}  // namespace bsc

using namespace bsc;

extern "C" {

bsc_status bsc_plan_cache_create(int32_t capacity, bsc_plan_cache_t *out) {
    set_error("");
    if (!out) {
        set_error("bsc_plan_cache_create: out is NULL");
        return BSC_ERR_ARG;
    }
    *out = nullptr;
    if (capacity < 1) {
        set_error("bsc_plan_cache_create: capacity must be >= 1");
        return BSC_ERR_ARG;
    }
    PlanCache *c = new (std::nothrow) PlanCache();
    if (!c) {
        set_error("bsc_plan_cache_create: out of host memory");
        return BSC_ERR_UNSUPPORTED;
    }
    c->capacity = capacity;
    *out = reinterpret_cast<bsc_plan_cache_t>(c);
    return BSC_OK;
}

static bsc_status plan_cached(bsc_plan_cache_t cache, const bsc_index *m, const bsc_index *k, const bsc_index *n,
                              const bsc_operand *A, const bsc_operand *B, const bsc_operand *C, bsc_dtype dtype,
                              bsc_axis axis, const bsc_options *opt, bsc_plan_t *out, int32_t *hit) {
    set_error("");
    if (!cache || !out) {
        set_error("bsc_plan_cached: cache or out is NULL");
        return BSC_ERR_ARG;
    }
    *out = nullptr;
    if (hit) *hit = 0;
    PlanCache &c = *reinterpret_cast<PlanCache *>(cache);

    bsc_options o;
    if (opt) o = *opt;
    else bsc_options_default(&o);
    KeyWriter w;
    const int32_t nq = m ? m->nq : 0;
    w.put(static_cast<int32_t>(dtype));
    w.put(static_cast<int32_t>(axis));
    write_options(w, o);
    const bool keyed = write_index(w, m, nq) && write_index(w, k, nq) && write_index(w, n, nq) &&
                       write_operand(w, A, nq) && write_operand(w, B, nq) && write_operand(w, C, nq);
    if (!keyed) return bsc_plan(m, k, n, A, B, C, dtype, axis, opt, out);   // reports the malformed argument

    {
        std::lock_guard<std::mutex> lock(c.mu);
        auto it = c.map.find(w.s);
        if (it != c.map.end()) {
            Plan *p = new (std::nothrow) Plan(it->second.plan);
            if (!p) {
                set_error("bsc_plan_cached: out of host memory");
                return BSC_ERR_UNSUPPORTED;
            }
            c.lru.splice(c.lru.begin(), c.lru, it->second.pos);
            ++c.hits;
            *out = reinterpret_cast<bsc_plan_t>(p);
            if (hit) *hit = 1;
            return BSC_OK;
        }
    }
    // plan outside the lock (planning takes milliseconds)
    bsc_plan_t fresh = nullptr;
    const bsc_status st = bsc_plan(m, k, n, A, B, C, dtype, axis, opt, &fresh);
    if (st != BSC_OK) return st;
    Plan *p = reinterpret_cast<Plan *>(fresh);
    std::lock_guard<std::mutex> lock(c.mu);
    ++c.misses;
    if (c.map.find(w.s) == c.map.end()) {   // another thread may have planned the same key meanwhile
        try {
            if (static_cast<int32_t>(c.map.size()) >= c.capacity) {
                c.map.erase(c.lru.back());
                c.lru.pop_back();
            }
            c.lru.push_front(w.s);
            auto ins = c.map.emplace(w.s, PlanCache::Entry{*p, c.lru.begin()});
            (void)ins;
        } catch (const std::bad_alloc &) {
            // the plan is still valid; it is only not cached
            if (!c.lru.empty() && c.map.find(c.lru.front()) == c.map.end()) c.lru.pop_front();
        }
    }
    *out = fresh;
    return BSC_OK;
}

bsc_status bsc_plan_cached(bsc_plan_cache_t cache, const bsc_index *m, const bsc_index *k, const bsc_index *n,
                           const bsc_operand *A, const bsc_operand *B, const bsc_operand *C, bsc_dtype dtype,
                           bsc_axis axis, const bsc_options *opt, bsc_plan_t *out, int32_t *hit) {
    try {
        return plan_cached(cache, m, k, n, A, B, C, dtype, axis, opt, out, hit);
    } catch (const std::bad_alloc &) {   // building the key; nothing was handed out
        if (out) *out = nullptr;
        set_error("bsc_plan_cached: out of host memory");
        return BSC_ERR_UNSUPPORTED;
    }
}

bsc_status bsc_plan_cache_stats(bsc_plan_cache_t cache, int64_t *hits, int64_t *misses, int64_t *entries) {
    if (!cache) {
        set_error("bsc_plan_cache_stats: NULL cache");
        return BSC_ERR_ARG;
    }
    PlanCache &c = *reinterpret_cast<PlanCache *>(cache);
    std::lock_guard<std::mutex> lock(c.mu);
    if (hits) *hits = c.hits;
    if (misses) *misses = c.misses;
    if (entries) *entries = static_cast<int64_t>(c.map.size());
    return BSC_OK;
}

void bsc_plan_cache_destroy(bsc_plan_cache_t cache) { delete reinterpret_cast<PlanCache *>(cache); }

}  // extern "C"
