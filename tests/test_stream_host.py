"""Host checks of the stream plan (bsc_stream_plan): one block-sparse
contraction planned for the fused launch's register-stream kernel, every C
block its own group of one stage-1 block and one output with the plan's own
weight 1.

The device image is replayed on the host as the kernel evaluates it (the fused
plan's replay, tile by tile and product by product, with that weight) and must
equal the oracle's contraction bit for bit on integer values (every summation
order is exact).  C blocks no product reaches come out zero, or unchanged under
accumulation; a planner mistake (a product on the wrong block, a missed tile, a
transposed view) changes the result."""
import numpy as np
import pytest

import oracle

from gpuhelp import c_addresses
from stream_cases import CASES
from test_fused_host import decode, replay

bst = pytest.importorskip("block_sparse_tensor_amd")


def _lib_ok():
    try:
        bst._capi.lib()
        return True
    except Exception:
        return False


pytestmark = pytest.mark.skipif(not _lib_ok(), reason="libbsc.so not built")


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("accumulate", [False, True])
def test_stream_replay_equals_oracle(name, accumulate):
    make, tile = CASES[name]
    con, a, b = make()
    sp = bst.StreamPlan(con, accumulate=accumulate, tile_cols=tile)
    s = sp.stats()
    assert s["stream"] == 1 and s["tile_blocks"] == (2 if tile == 32 else 1)
    rng = np.random.default_rng(5)
    c0 = rng.integers(-3, 4, con.C.buffer_elems).astype(np.float64)
    want = oracle.contract(con, a, b, c0.copy(), accumulate=accumulate) if accumulate else \
        oracle.contract(con, a, b, np.where(c_addresses(con)[1], 0.0, c0))
    got = replay(sp, a, b, np.ones(1), c0.copy())
    _, mask = c_addresses(con)
    assert np.array_equal(got[mask], want[mask])
    assert np.array_equal(got[~mask], c0[~mask]), "a write outside the C views"


def test_stream_stats_and_zero_blocks():
    con, a, b = CASES["random-f64-sparse"][0]()
    s = bst.StreamPlan(con).stats()
    t = oracle.triples(con)
    reached = {(int(m), int(n)) for m, k, n in t}
    assert s["groups"] == s["outputs"] == con.C.nblocks
    assert s["terms"] == len(reached) < con.C.nblocks   # some C blocks no product reaches
    assert s["channels"] == len(t)
    assert s["useful_flops"] == s["stage1_flops"] == oracle.useful_flops(con)
    assert s["alg_bytes"] == oracle.algorithmic_bytes(con)
    assert s["launches_per_contract"] == 1 and s["launches_issued"] == 0
    # the plan's own weight 1 in its type
    st, img = bst.StreamPlan(con).worklist()
    assert np.frombuffer(img, np.float64, count=1, offset=st["off_ones"])[0] == 1.0
    groups = decode(bst.StreamPlan(con))[1]
    assert (groups["nout"] == 1).all() and set(np.unique(groups["nblk"])) <= {0, 1}


def test_stream_refuses_what_it_cannot_plan():
    con, a, b = CASES["small-coop-stage1"][0]()
    with pytest.raises(bst.BscError) as e:
        bst.StreamPlan(con, dtype="bf16")
    assert e.value.name == "BSC_ERR_UNSUPPORTED"
    with pytest.raises(bst.BscError) as e:
        bst.StreamPlan(con, tile_cols=8)
    assert e.value.name == "BSC_ERR_ARG"
    # the W stage writes C blocks whose columns fuse two legs
    from workloads import configs as C
    w = C.rabc_u1(layout="coop").stages[1].con
    with pytest.raises(bst.BscError) as e:
        bst.StreamPlan(w)
    assert e.value.name == "BSC_ERR_UNSUPPORTED"
    # planning errors of the contraction itself are reported as bsc_plan reports them
    bad = CASES["small-coop-stage1"][0]()[0]
    bad.A.offset[0] = -1
    with pytest.raises(bst.BscError) as e:
        bst.StreamPlan(bad)
    assert e.value.name == "BSC_ERR_BOUNDS"


def test_stream_device_entry_checks_arguments():
    from ctypes import c_void_p
    con, a, b = CASES["small-coop-stage1"][0]()
    sp = bst.StreamPlan(con)
    L = bst._capi.lib()
    # unbound: refused before anything is enqueued (B2 may be NULL for a stream plan)
    st = L.bsc_fused_contract(sp._h, c_void_p(1), c_void_p(1), None, c_void_p(1), None)
    assert st in (-8, -7)
    assert L.bsc_stream_plan(None, None, None, None, None, None, 0, None, None) == -1


def test_stream_preference_follows_the_longest_stream():
    """stream_preferred: the longest wave's product stream is at most 32
    register chunks.  A bond-2048 stage 3 (a few C blocks, K up to 1571) runs
    longer streams and keeps the grouped tiles; its stage 1 (one product per
    block, K up to 417) does not."""
    from workloads import configs as C
    ch = C.small_chain(seed=3, layout="coop", dtype="f32", total=2048, qmax=4, sigma=2.0, w=1)
    for si, want in ((0, True), (2, False)):
        con = ch.stages[si].con
        sp = bst.StreamPlan(con)
        s = sp.stats()
        longest = max(sum((int(con.k.dim[k]) + 31) // 32 for m2, k, n2 in oracle.triples(con) if (m2, n2) == mn)
                      for mn in {(m, n) for m, k, n in oracle.triples(con)})
        assert s["longest_chunks"] == longest
        assert bool(s["stream_preferred"]) == want == (longest <= 32)
        assert isinstance(bst.best_plan(con), bst.StreamPlan if want else bst.Plan)
    # bf16 has no stream kernel: always the grouped plan
    bf = C.blockdiag_bf16(values=False).con
    assert isinstance(bst.best_plan(bf), bst.Plan)


def test_stream_splits_many_product_blocks():
    """C blocks of at least 8 products make each product a block of its own,
    so a launch that would leave CUs idle shares them over up to four waves
    (the replay checks the parts' blocks and their order)."""
    con, a, b = CASES["neutral-f32-stage3-split"][0]()
    sp = bst.StreamPlan(con)
    s, groups, chans, outs, widx, tasks, parts, pchans = decode(sp)
    assert (groups["nblk"] >= 8).all() and parts["nparts"].max() > 1
    few = bst.StreamPlan(CASES["small-coop-stage3"][0]()[0])
    assert decode(few)[6]["nparts"].max() == 1


def test_stream_long_product_list_stays_one_block():
    """A C block of 300 products (more than a wave's 256 lane-held weights)
    stays one block and still replays to the oracle's result."""
    from workloads.model import Contraction, Index, Operand
    nk = 300
    m = Index(np.zeros((1, 1), np.int32), [20])
    n = Index(np.zeros((1, 1), np.int32), [18])
    k = Index(np.zeros((nk, 1), np.int32), np.full(nk, 3))
    rng = np.random.default_rng(1)
    A = Operand(np.zeros(nk), np.arange(nk), np.arange(nk) * 60, np.tile([3, 0], (nk, 1)), np.tile([1, 0], (nk, 1)),
                [0], nk * 60)
    B = Operand(np.arange(nk), np.zeros(nk), np.arange(nk) * 54, np.tile([18, 0], (nk, 1)), np.tile([1, 0], (nk, 1)),
                [0], nk * 54)
    Cb = Operand([0], [0], [0], [[18, 0]], [[1, 0]], [0], 360)
    con = Contraction(m, k, n, A, B, Cb, "f64")
    a = rng.integers(-2, 3, nk * 60).astype(float)
    b = rng.integers(-2, 3, nk * 54).astype(float)
    sp = bst.StreamPlan(con)
    groups = decode(sp)[1]
    assert groups["nblk"].tolist() == [1] and groups["nchan"].tolist() == [nk]
    assert np.array_equal(replay(sp, a, b, np.ones(1), np.zeros(360)), oracle.contract(con, a, b, np.zeros(360)))
