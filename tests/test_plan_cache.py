"""Host-side tests of the plan cache (bsc_plan_cache_*): a cached plan is the
plan bsc_plan makes for the same inputs (same sector map, groups, operand
modes and byte-identical device work list), any change of an input misses,
the least recently used plan is dropped beyond the capacity, failures are not
cached, and a hit skips the planning work."""
import copy
import threading
import time

import numpy as np
import pytest

from workloads import configs as C

bst = pytest.importorskip("block_sparse_tensor_amd")
from block_sparse_tensor_amd import _capi  # noqa: E402


def _lib_or_skip():
    import os
    if not os.path.exists(_capi.LIB_PATH):
        pytest.skip("libbsc.so not built")


def _same_plan(p, q):
    for x, y in zip(p.export(), q.export()):
        assert np.array_equal(x, y)
    ip, bp = p.worklist()
    iq, bq = q.worklist()
    assert ip == iq
    assert bp == bq
    sp, sq = p.stats(), q.stats()
    for key in ("groups", "runs", "items", "grid", "useful_flops", "pack_bytes", "device_bytes", "split_tiles"):
        assert sp[key] == sq[key], key


@pytest.mark.parametrize("make", [lambda: C.tiny_u1("diag").con, lambda: C.ragged_batch().con,
                                  lambda: C.rabc_u1(layout="natural").stages[1].con,
                                  lambda: C.blockdiag_bf16(values=False, ld_align=8, align=8).con],
                         ids=["tiny", "ragged", "rabc_stage2", "blockdiag"])
def test_hit_equals_fresh_plan(make):
    _lib_or_skip()
    con = make()
    cache = bst.PlanCache(4)
    p1 = bst.Plan(con, cache=cache)
    p2 = bst.Plan(con, cache=cache)
    assert not p1.cache_hit and p2.cache_hit
    assert cache.stats() == {"hits": 1, "misses": 1, "entries": 1}
    fresh = bst.Plan(con)
    _same_plan(p2, fresh)
    _same_plan(p1, fresh)
    del p1   # copies are independent of each other
    _same_plan(p2, fresh)


def _variants(con):
    """Copies of `con` that differ from it in exactly one input."""
    out = []
    c = copy.deepcopy(con)
    c.A.offset = np.asarray(c.A.offset).copy()
    c.A.offset[0] += 0   # unchanged copy: must hit
    out.append(("same", c, {}, True))
    c = copy.deepcopy(con)
    c.C.buffer_elems = int(c.C.buffer_elems) + 1
    out.append(("c_buffer_elems", c, {}, False))
    c = copy.deepcopy(con)
    c.B.offset = np.asarray(c.B.offset).copy()
    c.B.buffer_elems = int(c.B.buffer_elems) + 16
    out.append(("b_buffer_elems", c, {}, False))
    c = copy.deepcopy(con)
    c.A.offset = np.asarray(c.A.offset).copy() + 0
    c.A.buffer_elems = int(c.A.buffer_elems) + 8
    c.A.offset[-1] += 8
    out.append(("a_offset", c, {}, False))
    out.append(("split_k", con, {"split_k": -1}, False))
    out.append(("accumulate", con, {"accumulate": True}, False))
    out.append(("axis", con, {"axis": "contract"}, False))
    out.append(("dtype", con, {"dtype": "f32"}, False))
    out.append(("layout", con, {"layout": "force_pack"}, False))
    return out


def test_any_changed_input_misses():
    _lib_or_skip()
    con = C.tiny_u1("diag").con
    cache = bst.PlanCache(64)
    bst.Plan(con, cache=cache)
    for name, c, kw, expect_hit in _variants(con):
        p = bst.Plan(c, cache=cache, **kw)
        assert p.cache_hit == expect_hit, name
        _same_plan(p, bst.Plan(c, **kw))


def test_dims_and_charges_are_part_of_the_key():
    _lib_or_skip()
    a = C.random_problem(3).con
    cache = bst.PlanCache(8)
    bst.Plan(a, cache=cache)
    b = C.random_problem(4).con
    assert not bst.Plan(b, cache=cache).cache_hit
    assert bst.Plan(copy.deepcopy(a), cache=cache).cache_hit
    assert cache.stats()["entries"] == 2


def test_lru_eviction():
    _lib_or_skip()
    cons = [C.random_problem(s).con for s in (11, 12, 13)]
    cache = bst.PlanCache(2)
    bst.Plan(cons[0], cache=cache)
    bst.Plan(cons[1], cache=cache)
    assert bst.Plan(cons[0], cache=cache).cache_hit      # 0 is now the most recent
    bst.Plan(cons[2], cache=cache)                         # evicts 1
    assert cache.stats()["entries"] == 2
    assert bst.Plan(cons[0], cache=cache).cache_hit
    assert bst.Plan(cons[2], cache=cache).cache_hit
    assert not bst.Plan(cons[1], cache=cache).cache_hit


def test_failed_plan_not_cached():
    _lib_or_skip()
    p = C.tiny_u1("diag")
    p.con.C.offset[1] = p.con.C.offset[0]
    cache = bst.PlanCache(4)
    for _ in range(2):
        with pytest.raises(bst.BscError) as e:
            bst.Plan(p.con, cache=cache)
        assert e.value.name == "BSC_ERR_OVERLAP"
    assert cache.stats() == {"hits": 0, "misses": 0, "entries": 0}


def test_bad_capacity():
    _lib_or_skip()
    with pytest.raises(bst.BscError) as e:
        bst.PlanCache(0)
    assert e.value.name == "BSC_ERR_ARG"


def test_hit_skips_planning():
    """A hit copies the stored plan: on the U(1)xU(1) update's stage 3 (1002
    groups) it takes a small fraction of a fresh plan's time."""
    _lib_or_skip()
    con = C.rabc_u1u1(layout="coop").stages[2].con
    cache = bst.PlanCache(4)
    bst.Plan(con, cache=cache)
    t_plan = min(_timed(lambda: bst.Plan(con)) for _ in range(3))
    t_hit = min(_timed(lambda: bst.Plan(con, cache=cache)) for _ in range(3))
    print(f"plan {t_plan * 1e3:.2f} ms, cached {t_hit * 1e3:.2f} ms")
    assert t_hit < 0.5 * t_plan


def _timed(f):
    t = time.perf_counter()
    f()
    return time.perf_counter() - t


def test_threads_share_one_cache():
    _lib_or_skip()
    cons = [C.random_problem(s).con for s in (21, 22)]
    cache = bst.PlanCache(8)
    ref = [bst.Plan(c) for c in cons]
    errors = []

    def work(i):
        try:
            for j in range(6):
                q = bst.Plan(cons[(i + j) % 2], cache=cache)
                _same_plan(q, ref[(i + j) % 2])
        except Exception as ex:  # reported below
            errors.append(ex)

    th = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in th:
        t.start()
    for t in th:
        t.join()
    assert not errors, errors
    s = cache.stats()
    assert s["entries"] == 2 and s["hits"] + s["misses"] == 24


def test_cache_plan_without_products():
    """A plan with no sector products (every C block zero-filled) is cached
    like any other."""
    _lib_or_skip()
    con = copy.deepcopy(C.tiny_u1("diag").con)
    op = con.A
    op.row_key, op.col_key = np.zeros(0, np.int32), np.zeros(0, np.int32)
    op.offset, op.row_stride, op.col_stride = np.zeros(0, np.int64), np.zeros((0, 2), np.int64), np.zeros((0, 2), np.int64)
    cache = bst.PlanCache(2)
    assert not bst.Plan(con, cache=cache).cache_hit
    p = bst.Plan(con, cache=cache)
    assert p.cache_hit and p.stats()["zero_blocks"] == con.C.nblocks
    _same_plan(p, bst.Plan(con))
