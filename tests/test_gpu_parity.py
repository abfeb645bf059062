"""GPU parity: the HIP engine (through the C-ABI) against the CPU oracle on the
same seeded inputs.  Tolerances (relative Frobenius over all C blocks):
1e-12 fp64, 1e-5 fp32, 2e-2 bf16 inputs with fp32 accumulation; integer-valued
inputs make every summation order exact, so those compare bit-for-bit."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import TOL, canary, check_canary, c_addresses, have_gpu, rel_frobenius, run_engine, to_dev, torch

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:  # collected on CPU but never run there
    bst = None

AXES = ["auto", "free_m", "free_n", "contract"]


def _parity(prob, axis="auto", launch_mode="grouped", layout="auto", tol=None, exact=False, accumulate=False):
    con = prob.con
    plan = bst.Plan(con, axis=axis, launch_mode=launch_mode, layout=layout, accumulate=accumulate).bind()
    print(f"[parity] {prob.name} dtype={con.dtype} axis={axis} mode={launch_mode} layout={layout}", flush=True)
    addr, mask = c_addresses(con)
    if accumulate:
        rng = np.random.default_rng(1)
        c0 = np.where(mask, rng.integers(-2, 3, con.C.buffer_elems), np.nan)
    else:
        c0 = canary(con, con.dtype)
    got = run_engine(plan, prob.a, prob.b, c0, con.dtype)
    ref = oracle.contract(con, prob.a, prob.b, np.asarray(c0, np.float64), accumulate=accumulate)
    check_canary(got, mask)
    if exact:
        assert np.array_equal(got[addr], ref[addr].astype(got.dtype)), "integer-valued parity must be bit-exact"
    else:
        err = rel_frobenius(got, ref, addr)
        assert err <= (tol or TOL[con.dtype]), err
    return plan, got


@pytest.mark.parametrize("variant", ["diag", "flux1", "flux1_3leg"])
@pytest.mark.parametrize("axis", AXES)
def test_tiny_u1(variant, axis):
    _parity(C.tiny_u1(variant), axis=axis)


@pytest.mark.parametrize("variant", ["diag", "flux1"])
def test_tiny_u1_per_sector(variant):
    _parity(C.tiny_u1(variant), launch_mode="per_sector")


@pytest.mark.parametrize("axis", AXES)
def test_ragged_batch(axis):
    plan, _ = _parity(C.ragged_batch(), axis=axis)
    if axis in ("auto", "free_m"):
        assert plan.stats()["launches_per_contract"] == 1


def test_ragged_batch_per_sector():
    plan, _ = _parity(C.ragged_batch(), launch_mode="per_sector")
    assert plan.stats()["launches_per_contract"] == 4000


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("seed", range(4))
def test_integer_values_bit_exact(dtype, seed):
    prob = C.random_problem(3000 + seed, nq=1 + seed % 2, nkeys=(6, 5, 6), maxdim=40, qrange=1, dtype=dtype,
                            flux=[(0, 0), (1, -1)][seed % 2], int_values=True, density=0.8)
    for axis in AXES:
        _parity(prob, axis=axis, exact=True)
    _parity(prob, launch_mode="per_sector", exact=True)


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("seed", range(6))
def test_random_strided(dtype, seed):
    prob = C.random_problem(4000 + seed, nq=1 + seed % 2, nkeys=(7, 6, 7), maxdim=24, qrange=1, dtype=dtype,
                            flux=[(0, 0), (1, -1), (1, 0)][seed % 3], density=0.8)
    for axis in AXES:
        _parity(prob, axis=axis)


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_accumulate(dtype):
    prob = C.random_problem(4100, nq=1, nkeys=(5, 5, 5), maxdim=20, qrange=1, dtype=dtype, int_values=True)
    _parity(prob, axis="auto", accumulate=True, exact=True)
    _parity(prob, launch_mode="per_sector", accumulate=True, exact=True)


def test_blockdiag_bf16_full_size():
    prob = C.blockdiag_bf16()
    plan, got = _parity(prob, axis="auto")
    s = plan.stats()
    assert s["launches_per_contract"] == 1 and s["launches_per_sector"] == 64


def test_blockdiag_bf16_full_size_aligned():
    """16-byte aligned, padded layout: the direct-to-LDS tile path."""
    prob = C.blockdiag_bf16(ld_align=8, align=8)
    plan, got = _parity(prob, axis="auto")
    s = plan.stats()
    assert s["items_by_class"]["mfma_fast"] > 0 and s["launches_per_contract"] == 1


def test_blockdiag_bf16_small_blocks_ragged():
    """A ragged bf16 block-diagonal case spanning several tiles with odd edges."""
    prob = C.random_problem(4200, nq=1, nkeys=(6, 6, 6), maxdim=150, qrange=2, dtype="bf16", two_leg=False,
                            dup_charges=False)
    _parity(prob)


def _chain_parity(ch, tol, axes=("auto", "auto", "auto")):
    t = torch()
    ref = oracle.run_chain(ch)
    dt = ch.dtype
    bufs = {k: to_dev(v, dt) for k, v in ch.buffers.items()}
    cdt = t.float64 if dt == "f64" else t.float32
    for name, n in ch.sizes.items():
        if name not in bufs:
            bufs[name] = t.zeros(n, dtype=cdt, device="cuda")
    for st, ax in zip(ch.stages, axes):
        print(f"[chain] {ch.name} stage {st.label} axis={ax}", flush=True)
        plan = bst.Plan(st.con, axis=ax).bind()
        plan.contract(bufs[st.a_buf], bufs[st.b_buf], bufs[st.c_buf])
    t.cuda.synchronize()
    for st in ch.stages:
        addr, _ = c_addresses(st.con)
        got = bufs[st.c_buf].cpu().numpy()
        err = rel_frobenius(got, ref[st.c_buf], addr)
        assert err <= tol, (st.label, err)


@pytest.mark.parametrize("layout", ["coop", "natural"])
def test_small_chain(layout):
    _chain_parity(C.small_chain(seed=3, layout=layout), 1e-12)


def test_rabc_u1_chain():
    _chain_parity(C.rabc_u1(), 1e-12)
    _chain_parity(C.rabc_u1(), 1e-12, axes=("contract", "free_n", "free_m"))


def test_rabc_u1u1_chain():
    _chain_parity(C.rabc_u1u1(), 1e-5)


def test_determinism():
    prob = C.ragged_batch()
    plan = bst.Plan(prob.con).bind()
    t = torch()
    A, B = to_dev(prob.a, "f32"), to_dev(prob.b, "f32")
    C0 = t.zeros(prob.con.C.buffer_elems, dtype=t.float32, device="cuda")
    outs = []
    for _ in range(10):
        plan.contract(A, B, C0)
        t.cuda.synchronize()
        outs.append(C0.cpu().numpy().copy())
    for o in outs[1:]:
        assert np.array_equal(o.view(np.uint32), outs[0].view(np.uint32))


def test_coalesced_equals_uncoalesced():
    prob = C.random_problem(4300, nq=1, nkeys=(6, 6, 6), maxdim=30, qrange=1, dtype="f64", density=0.9)
    results = []
    for kw in (dict(launch_mode="per_sector"), dict(axis="free_m"), dict(axis="free_n"), dict(axis="contract")):
        plan = bst.Plan(prob.con, **kw).bind()
        results.append(run_engine(plan, prob.a, prob.b, canary(prob.con, "f64"), "f64"))
    addr, _ = c_addresses(prob.con)
    for r in results[1:]:
        assert rel_frobenius(r, results[0], addr) <= 1e-13


def test_launch_counter():
    prob = C.ragged_batch()
    plan = bst.Plan(prob.con).bind()
    before = plan.stats()["launches_issued"]
    run_engine(plan, prob.a, prob.b, np.zeros(prob.con.C.buffer_elems, np.float32), "f32", repeats=3)
    assert plan.stats()["launches_issued"] - before == 3
