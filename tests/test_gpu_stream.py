"""GPU parity of the stream plan (bsc_stream_plan): one contraction through
the fused launch's register-stream kernel, every C block written by the waves
of its own tiles.  Integer-valued operands compare bit for bit with the oracle
(overwrite and accumulate, repeats identical, C blocks no product reaches
zero-filled); normal values compare per C block within the dtype's tolerance
of the forward error bound; a NaN canary outside the C views must survive.
The environment-update stages run at full size."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import TOL, block_errors, c_addresses, have_gpu, to_dev, torch
from stream_cases import CASES

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:
    bst = None


def _run(con, a, b, c_init, accumulate=False, tile=0, repeats=1):
    t = torch()
    sp = bst.StreamPlan(con, accumulate=accumulate, tile_cols=tile).bind()
    A, B = to_dev(a, con.dtype), to_dev(b, con.dtype)
    outs = []
    for _ in range(repeats):
        Cd = to_dev(c_init, con.dtype)
        sp.contract(A, B, Cd)
        t.cuda.synchronize()
        outs.append(Cd.cpu().numpy())
    return sp, outs


def _full_stage(ch, si, values):
    st = ch.stages[si]
    rng = np.random.default_rng(40 + si)
    def buf(name):
        if name in ch.buffers:
            return np.asarray(ch.buffers[name], np.float64)
        if values == "int":
            return rng.integers(-2, 3, ch.sizes[name]).astype(np.float64)
        return rng.standard_normal(ch.sizes[name])
    return st.con, buf(st.a_buf), buf(st.b_buf)


FULL = {
    "rabc_u1-stage1": lambda v: _full_stage(C.rabc_u1(values=v), 0, v),
    "rabc_u1-stage3": lambda v: _full_stage(C.rabc_u1(values=v), 2, v),
    "rabc_u1u1-stage1": lambda v: _full_stage(C.rabc_u1u1(values=v), 0, v),
    "rabc_u1u1-stage3": lambda v: _full_stage(C.rabc_u1u1(values=v), 2, v),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("accumulate", [False, True])
def test_stream_int_bit_exact(name, accumulate):
    make, tile = CASES[name]
    con, a, b = make()
    addr, mask = c_addresses(con)
    rng = np.random.default_rng(23)
    c0 = np.full(con.C.buffer_elems, np.nan)
    c0[mask] = rng.integers(-3, 4, int(mask.sum())) if accumulate else 0.0
    want = oracle.contract(con, a, b, np.nan_to_num(c0), accumulate=accumulate)
    print(f"[stream] {name} accumulate={accumulate}", flush=True)
    sp, (got, again) = _run(con, a, b, c0, accumulate, tile, repeats=2)
    assert np.all(np.isnan(got[~mask])), "a write landed outside the C views"
    assert np.array_equal(got[mask].astype(np.float64), want[mask]), name
    assert np.array_equal(got[mask], again[mask]), "repeats differ"
    assert sp.stats()["launches_issued"] == 2


@pytest.mark.parametrize("name", sorted(FULL))
def test_stream_full_size_int_bit_exact(name):
    con, a, b = FULL[name]("int")
    addr, mask = c_addresses(con)
    c0 = np.full(con.C.buffer_elems, np.nan)
    c0[mask] = 0.0
    want = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems))
    print(f"[stream] full {name} int", flush=True)
    _, (got,) = _run(con, a, b, c0)
    assert np.all(np.isnan(got[~mask]))
    assert np.array_equal(got[mask].astype(np.float64), want[mask]), name


@pytest.mark.parametrize("name", sorted(FULL))
def test_stream_full_size_normal_within_error_bound(name):
    con, a, b = FULL[name]("normal")
    addr, mask = c_addresses(con)
    want = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems))
    scale = oracle.contract(con, np.abs(a), np.abs(b), np.zeros(con.C.buffer_elems))
    c0 = np.full(con.C.buffer_elems, np.nan)
    c0[mask] = 0.0
    print(f"[stream] full {name} normal", flush=True)
    _, (got,) = _run(con, a, b, c0)
    assert np.all(np.isnan(got[~mask]))
    errs = block_errors(con, got.astype(np.float64), want, scale)
    worst = int(np.argmax(errs)) if len(errs) else 0
    assert len(errs) == 0 or errs[worst] <= TOL[con.dtype], (name, worst, float(errs[worst]))


def test_stream_matches_grouped_plan():
    """The stream plan and the grouped plan of the same contraction agree on
    integer values bit for bit (both exact), C blocks without products zero."""
    t = torch()
    con, a, b = CASES["random-f32-sparse"][0]()
    A, B = to_dev(a, con.dtype), to_dev(b, con.dtype)
    outs = []
    for plan in (bst.StreamPlan(con).bind(), bst.Plan(con).bind()):
        Cd = t.full((con.C.buffer_elems,), 7.0, dtype=t.float32, device="cuda")
        plan.contract(A, B, Cd)
        t.cuda.synchronize()
        outs.append(Cd.cpu().numpy())
    _, mask = c_addresses(con)
    assert np.array_equal(outs[0][mask], outs[1][mask])


def test_stream_contract_checks_tensors():
    t = torch()
    con, a, b = CASES["small-coop-stage1"][0]()
    sp = bst.StreamPlan(con)
    A, B = to_dev(a, "f64"), to_dev(b, "f64")
    Cd = t.zeros(con.C.buffer_elems, dtype=t.float64, device="cuda")
    with pytest.raises(bst.BscError):
        sp.contract(A, B, Cd)                               # not bound
    sp.bind()
    with pytest.raises(TypeError):
        sp.contract(A.float(), B, Cd)
    with pytest.raises(ValueError):
        sp.contract(A, B, Cd[:-1])
