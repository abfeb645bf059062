"""GPU parity of the fused two-stage launch (bsc_fused_*): T2 = (E^T A) W of the
environment update computed in one kernel, compared with the oracle's two
stages.  Integer-valued chains compare bit for bit (every partial sum is an
exact integer in the operands' type); normal-valued chains compare per output
block against the forward error bound of the two nested sums,
||dT2_b|| / ||(|W| (|E|^T |A|))_b|| <= the dtype tolerance.  Elements of the
output buffer outside every T2 view hold a NaN canary that must survive."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import TOL, block_errors, c_addresses, have_gpu, int_chain_bound, to_dev, torch

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:
    bst = None


def _wide(total):
    return lambda v: C.small_chain(seed=3, layout="coop", dtype="f32", total=total, qmax=4, sigma=2.0, w=1, values=v)


def _cases():
    # name: chain for a value kind, split bound, wave tile edge (0 automatic)
    return {
        "small-coop-f64": (lambda v: C.small_chain(seed=3, layout="coop", values=v), 0, 0),
        "small-natural-f32": (lambda v: C.small_chain(seed=5, layout="natural", values=v, dtype="f32"), 0, 0),
        "rabc_u1": (lambda v: C.rabc_u1(layout="coop", values=v), 0, 0),
        "rabc_u1u1": (lambda v: C.rabc_u1u1(layout="natural", values=v), 0, 0),
        # all charges zero: several products per stage-1 block, 20 outputs per row
        # (three output chunks), K over two chunks; unsplit past 64 records per wave
        "neutral-natural-unsplit": (lambda v: C.neutral_chain(layout="natural", values=v), 1, 0),
        "neutral-coop-f32-split": (lambda v: C.neutral_chain(seed=4, layout="coop", dtype="f32", values=v), 0, 0),
        # 32 x 32 wave tiles: asked for on a 1024 bond, chosen on a 2048 bond
        "wide-coop-f32-tile32": (_wide(1024), 0, 32),
        "big-coop-f32-auto": (_wide(2048), 0, 0),
    }


def _two_stage(ch, bufs, c0=None, accumulate=False):
    s1, s2 = ch.stages[0], ch.stages[1]
    t1 = oracle.contract(s1.con, bufs[s1.a_buf], bufs[s1.b_buf], np.zeros(ch.sizes[s1.c_buf]))
    base = np.zeros(ch.sizes[s2.c_buf]) if c0 is None else np.asarray(c0, np.float64)
    return oracle.contract(s2.con, t1, bufs[s2.b_buf], base.copy(), accumulate=accumulate)


def _run_fused(ch, c_init, accumulate=False, repeats=1, split=0, tile=0):
    t = torch()
    s1, s2 = ch.stages[0], ch.stages[1]
    fp = bst.FusedPlan(s1.con, s2.con, accumulate=accumulate, split=split, tile_cols=tile).bind()
    A1 = to_dev(ch.buffers[s1.a_buf], ch.dtype)
    B1 = to_dev(ch.buffers[s1.b_buf], ch.dtype)
    W = to_dev(ch.buffers[s2.b_buf], ch.dtype)
    outs = []
    for _ in range(repeats):
        C2 = to_dev(c_init, ch.dtype)
        fp.contract(A1, B1, W, C2)
        t.cuda.synchronize()
        outs.append(C2.cpu().numpy())
    return fp, outs


@pytest.mark.parametrize("name", ["small-coop-f64", "small-natural-f32", "rabc_u1", "rabc_u1u1",
                                  "neutral-natural-unsplit", "neutral-coop-f32-split", "wide-coop-f32-tile32",
                                  "big-coop-f32-auto"])
@pytest.mark.parametrize("accumulate", [False, True])
def test_fused_int_bit_exact(name, accumulate):
    make, split, tile = _cases()[name]
    ch = make("int")
    if ch.dtype == "f32":
        assert int_chain_bound(ch) < 2 ** 24
    s2 = ch.stages[1]
    addr, mask = c_addresses(s2.con)
    rng = np.random.default_rng(21)
    c0 = np.full(ch.sizes[s2.c_buf], np.nan)
    c0[mask] = rng.integers(-3, 4, int(mask.sum())) if accumulate else 0.0
    bufs = {k: np.asarray(v, np.float64) for k, v in ch.buffers.items()}
    want = _two_stage(ch, bufs, np.nan_to_num(c0), accumulate)
    print(f"[fused] {name} int accumulate={accumulate}", flush=True)
    fp, (got, again) = _run_fused(ch, c0, accumulate, repeats=2, split=split, tile=tile)
    if name.endswith("tile32") or name.startswith("big"):
        assert fp.stats()["tile_blocks"] == 2
    assert np.all(np.isnan(got[~mask])), "a write landed outside the T2 views"
    assert np.array_equal(got[mask].astype(np.float64), want[mask]), name
    assert np.array_equal(got[mask], again[mask]), "repeats differ"
    assert fp.stats()["launches_issued"] == 2


@pytest.mark.parametrize("name", ["small-coop-f64", "rabc_u1", "rabc_u1u1", "neutral-coop-f32-split",
                                  "big-coop-f32-auto"])
def test_fused_normal_values_within_error_bound(name):
    make, split, tile = _cases()[name]
    ch = make("normal")
    s2 = ch.stages[1]
    addr, mask = c_addresses(s2.con)
    bufs = {k: np.asarray(v, np.float64) for k, v in ch.buffers.items()}
    want = _two_stage(ch, bufs)
    scale = _two_stage(ch, {k: np.abs(v) for k, v in bufs.items()})
    c0 = np.full(ch.sizes[s2.c_buf], np.nan)
    c0[mask] = 0.0
    print(f"[fused] {name} normal", flush=True)
    _, (got,) = _run_fused(ch, c0, split=split, tile=tile)
    assert np.all(np.isnan(got[~mask]))
    errs = block_errors(s2.con, got.astype(np.float64), want, scale)
    worst = int(np.argmax(errs)) if len(errs) else 0
    assert len(errs) == 0 or errs[worst] <= TOL[ch.dtype], (name, worst, float(errs[worst]))
    g, r = got[addr].astype(np.float64), want[addr]
    assert np.linalg.norm(g - r) <= TOL[ch.dtype] * np.linalg.norm(r)


def test_fused_then_stage_three_matches_chain():
    """The fused launch feeding the third stage (E' = T2 A) gives the chain's E'."""
    t = torch()
    ch = C.rabc_u1(layout="coop", values="int")
    s1, s2, s3 = ch.stages
    ref = oracle.run_chain(ch)
    fp = bst.FusedPlan(s1.con, s2.con).bind()
    p3 = bst.Plan(s3.con).bind()
    d = {k: to_dev(v, ch.dtype) for k, v in ch.buffers.items()}
    T2 = t.zeros(ch.sizes[s2.c_buf], dtype=t.float64, device="cuda")
    Ep = t.zeros(ch.sizes[s3.c_buf], dtype=t.float64, device="cuda")
    fp.contract(d[s1.a_buf], d[s1.b_buf], d[s2.b_buf], T2)
    p3.contract(T2, d[s3.b_buf], Ep)
    t.cuda.synchronize()
    _, mask = c_addresses(s3.con)
    assert np.array_equal(Ep.cpu().numpy()[mask], ref[s3.c_buf][mask])


def test_fused_contract_checks_tensors():
    t = torch()
    ch = C.small_chain(seed=3, layout="coop")
    s1, s2 = ch.stages[0], ch.stages[1]
    fp = bst.FusedPlan(s1.con, s2.con)
    A1 = to_dev(ch.buffers[s1.a_buf], "f64")
    B1 = to_dev(ch.buffers[s1.b_buf], "f64")
    W = to_dev(ch.buffers[s2.b_buf], "f64")
    C2 = t.zeros(ch.sizes[s2.c_buf], dtype=t.float64, device="cuda")
    with pytest.raises(bst.BscError):
        fp.contract(A1, B1, W, C2)                          # not bound
    fp.bind()
    with pytest.raises(TypeError):
        fp.contract(A1.float(), B1, W, C2)
    with pytest.raises(ValueError):
        fp.contract(A1, B1, W, C2[:-1])
