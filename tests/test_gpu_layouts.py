"""GPU parity of chains laid out for their writers or readers (relayout_chain
over bsc_plan_layout): the oracle runs the chain in its source layout, the engine
runs the relaid chain (inputs moved block by block), and every block of every
stage's output is compared through its own view in each layout.  The oracle
never sees a layout the library produced."""
import numpy as np
import pytest

import oracle
from workloads import configs as C
from workloads.layout import view_addresses

from gpuhelp import have_gpu, to_dev, torch

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:
    bst = None


def _c_blocks(con, buf):
    """Values of every C block of `con` read from `buf`, one flat array per block."""
    out = []
    for j in range(con.C.nblocks):
        r, c = int(con.C.row_key[j]), int(con.C.col_key[j])
        ri = 1 if con.m.inner is None else int(con.m.inner[r])
        ci = 1 if con.n.inner is None else int(con.n.inner[c])
        a = view_addresses(con.C.offset[j], np.reshape(con.C.row_stride, (-1, 2))[j],
                           np.reshape(con.C.col_stride, (-1, 2))[j], int(con.m.dim[r]), int(con.n.dim[c]), ri, ci)
        out.append(buf[a].ravel())
    return out


def _c_values(con, buf):
    """Concatenated values of every C block of `con` read from `buf`."""
    out = _c_blocks(con, buf)
    return np.concatenate(out) if out else np.zeros(0)


def _check_blocks(old, new, got_buf, ref_buf, scale_buf, tol, label):
    """Per C block: ||got_b - ref_b|| / ||(|A||B|)_b|| <= tol (blocks in the same
    order in both layouts); a block with zero scale must match exactly."""
    for j, (g, r, s) in enumerate(zip(_c_blocks(new, got_buf), _c_blocks(old, ref_buf), _c_blocks(old, scale_buf))):
        ns = np.linalg.norm(s)
        if ns == 0:
            assert np.array_equal(g, r), (label, j)
        else:
            assert np.linalg.norm(g - r) / ns <= tol, (label, j, np.linalg.norm(g - r) / ns)


@pytest.mark.parametrize("make,tol", [(lambda: C.small_chain(seed=3, layout="natural"), 1e-12),
                                      (lambda: C.small_chain(seed=4, layout="natural", dtype="f32"), 1e-5),
                                      (lambda: C.rabc_u1(layout="natural"), 1e-12),
                                      (lambda: C.rabc_u1u1(layout="natural"), 1e-5),
                                      (lambda: C.rabc_u1u1(layout="natural", values="int"), 0.0)],
                         ids=["small_f64", "small_f32", "rabc_u1", "rabc_u1u1", "rabc_u1u1_int"])
@pytest.mark.parametrize("prefer", ["writer", "reader"])
def test_relaid_chain_matches_oracle(make, tol, prefer):
    t = torch()
    ch = make()
    ref = oracle.run_chain(ch)
    # magnitudes for the per-block check: the chain on absolute values
    absref = {k: np.abs(v) for k, v in ref.items() if k in ch.buffers}
    for s_ in ch.stages:
        absref[s_.c_buf] = oracle.contract(s_.con, absref[s_.a_buf], absref[s_.b_buf], np.zeros(ch.sizes[s_.c_buf]),
                                           check=False)
    st = [(s.con, s.a_buf, s.b_buf, s.c_buf) for s in ch.stages]
    new, sizes, _ = bst.layouts.relayout_chain(st, prefer=prefer)
    plans = [bst.Plan(c).bind() for c in new]
    print(f"[layouts] {ch.name}: launches {[p.stats()['launches_per_contract'] for p in plans]}", flush=True)
    cdt = {"f64": t.float64, "f32": t.float32}[ch.dtype]
    bufs = {}
    for buf, v in ch.buffers.items():
        i, which = next((i, w) for i, s in enumerate(st) for w, b in zip("AB", s[1:3]) if b == buf)
        bufs[buf] = to_dev(bst.layouts.move_blocks(np.asarray(v), st[i][0], which, new[i]), ch.dtype)
    for buf, n in sizes.items():
        if buf not in bufs:
            bufs[buf] = t.full((n,), float("nan"), dtype=cdt, device="cuda")
    for p, (c, a, b, cb) in zip(plans, st):
        p.contract(bufs[a], bufs[b], bufs[cb])
    t.cuda.synchronize()
    for (old, _, _, cb), nc in zip(st, new):
        gbuf = bufs[cb].cpu().numpy().astype(np.float64)
        got = _c_values(nc, gbuf)
        want = _c_values(old, ref[cb])
        assert np.isfinite(got).all()
        if tol == 0.0:   # integer values: bit for bit
            assert np.array_equal(got, want), cb
            continue
        err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
        assert err <= tol, (cb, err)
        _check_blocks(old, nc, gbuf, ref[cb], absref[cb], tol, cb)


def _move_operand(src, con, new, which):
    return bst.layouts.move_blocks(np.asarray(src), con, which, new)


@pytest.mark.parametrize("dtype,tol", [("f64", 1e-12), ("f32", 1e-5), ("bf16", 2e-2)])
@pytest.mark.parametrize("seed", [31, 32, 33])
def test_planned_layout_single_contraction(dtype, tol, seed):
    """Random sector structures (two-leg keys, scattered strided blocks) with
    every operand laid out by bsc_plan_layout at 8-element alignment (the
    16-byte rows the direct-to-LDS bf16 tiles need): the engine's C blocks
    equal the oracle's on the source layout."""
    import copy
    t = torch()
    p = C.random_problem(seed, nkeys=(8, 8, 8), maxdim=200, qrange=1, dtype=dtype, density=0.8)
    con = p.con
    assert len(oracle.triples(con)) > 0
    ref = oracle.contract(con, p.a, p.b, np.zeros(con.C.buffer_elems), check=False)
    scale = oracle.contract(con, np.abs(p.a), np.abs(p.b), np.zeros(con.C.buffer_elems), check=False)
    new = copy.deepcopy(con)
    for w in "ABC":
        off, rs, cs, tot = bst.plan_layout(con, w, align=8)
        op = getattr(new, w)
        op.offset, op.row_stride, op.col_stride, op.buffer_elems = off, rs, cs, tot
    a = _move_operand(p.a, con, new, "A")
    b = _move_operand(p.b, con, new, "B")
    plan = bst.Plan(new).bind()
    s = plan.stats()
    print(f"[layouts] random seed={seed} {dtype}: items {s['items_by_class']}", flush=True)
    A, B = to_dev(a, dtype), to_dev(b, dtype)
    cdt = t.float64 if dtype == "f64" else t.float32
    Cd = t.full((new.C.buffer_elems,), float("nan"), dtype=cdt, device="cuda")
    plan.contract(A, B, Cd)
    t.cuda.synchronize()
    gbuf = Cd.cpu().numpy().astype(np.float64)
    got = _c_values(new, gbuf)
    want = _c_values(con, ref)
    assert np.isfinite(got).all()
    err = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)
    assert err <= tol, err
    _check_blocks(con, new, gbuf, ref, scale, tol, f"seed {seed}")
