"""GPU parity: the HIP engine (through the C-ABI) against the CPU oracle on the
same seeded inputs.  Tolerances: 1e-12 fp64, 1e-5 fp32, 2e-2 bf16 inputs with
fp32 accumulation, applied to the relative Frobenius error over all C blocks
and to every C block on its own (gpuhelp); integer-valued inputs make every
summation order exact, so those compare bit-for-bit, at full size too.  Every
case asserts that it contracts something."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import (TOL, block_addresses, canary, check_blocks, check_canary, c_addresses, have_gpu,
                     int_chain_bound, rel_frobenius, run_engine, to_dev, torch)

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:  # collected on CPU but never run there
    bst = None

AXES = ["auto", "free_m", "free_n", "contract"]


def _parity(prob, axis="auto", launch_mode="grouped", layout="auto", tol=None, exact=False, accumulate=False,
            min_triples=1, **plan_kw):
    con = prob.con
    plan = bst.Plan(con, axis=axis, launch_mode=launch_mode, layout=layout, accumulate=accumulate, **plan_kw).bind()
    print(f"[parity] {prob.name} dtype={con.dtype} axis={axis} mode={launch_mode} layout={layout} {plan_kw}",
          flush=True)
    assert plan.stats()["triples"] >= min_triples, "the case must contract something"
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
        t = tol or TOL[con.dtype]
        err = rel_frobenius(got, ref, addr)
        assert err <= t, err
        check_blocks(con, got, ref, prob.a, prob.b, t, c0=c0, accumulate=accumulate, label=prob.name)
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


# (seed, charge components): seeds chosen so every case has at least 8 sector GEMMs
INT_CASES = [(3000, 1), (3073, 2), (3002, 1), (3709, 2)]


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("case", INT_CASES, ids=lambda c: f"s{c[0]}-q{c[1]}")
def test_integer_values_bit_exact(dtype, case):
    seed, nq = case
    prob = C.random_problem(seed, nq=nq, nkeys=(6, 5, 6), maxdim=40, qrange=1, dtype=dtype,
                            flux=[(0, 0), (1, -1)][nq - 1], int_values=True, density=0.8)
    for axis in AXES:
        _parity(prob, axis=axis, exact=True, min_triples=8)
    _parity(prob, launch_mode="per_sector", exact=True, min_triples=8)


# seeds chosen so every case has at least 6 sector GEMMs; case i has 1 + i % 2
# charge components and flux pair i % 3
STRIDED_SEEDS = [4000, 4049, 4008, 4003, 4004, 4029]


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("case", range(len(STRIDED_SEEDS)))
def test_random_strided(dtype, case):
    prob = C.random_problem(STRIDED_SEEDS[case], nq=1 + case % 2, nkeys=(7, 6, 7), maxdim=24, qrange=1, dtype=dtype,
                            flux=[(0, 0), (1, -1), (1, 0)][case % 3], density=0.8)
    for axis in AXES:
        _parity(prob, axis=axis, min_triples=6)


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_accumulate(dtype):
    prob = C.random_problem(4100, nq=1, nkeys=(5, 5, 5), maxdim=20, qrange=1, dtype=dtype, int_values=True)
    _parity(prob, axis="auto", accumulate=True, exact=True)
    _parity(prob, launch_mode="per_sector", accumulate=True, exact=True)


def test_blockdiag_bf16_full_size():
    """The as-generated layout (blocks back to back, rows off 16-byte
    boundaries): the large groups' operands are gathered into 16-byte rows
    (one gather launch) and run on the direct-to-LDS tile, the rest on the
    general tile."""
    prob = C.blockdiag_bf16()
    plan, got = _parity(prob, axis="auto")
    s = plan.stats()
    assert s["launches_per_contract"] == 2 and s["launches_per_sector"] == 64
    assert s["pack_bytes"] > 0 and s["pack_gain_align_us"] > 0
    assert s["items_by_class"]["mfma_fast"] > 0 and s["items_by_class"]["mfma"] > 0


def test_blockdiag_bf16_full_size_no_gathers():
    """The same layout without gathers: every tile on the general tile, whose
    16-byte loads and stores start at any element."""
    prob = C.blockdiag_bf16()
    plan, got = _parity(prob, axis="auto", layout="never_pack")
    s = plan.stats()
    assert s["launches_per_contract"] == 1 and s["items_by_class"]["mfma_fast"] == 0


def test_blockdiag_bf16_full_size_aligned():
    """16-byte aligned, padded layout: the direct-to-LDS tile path."""
    prob = C.blockdiag_bf16(ld_align=8, align=8)
    plan, got = _parity(prob, axis="auto")
    s = plan.stats()
    assert s["items_by_class"]["mfma_fast"] > 0 and s["launches_per_contract"] == 1


@pytest.mark.parametrize("ld_align,layout", [(8, "auto"), (1, "auto"), (1, "never_pack")])
def test_blockdiag_bf16_full_size_int_bit_exact(ld_align, layout):
    """The bench workload's structure and launch configuration (default plan
    options) on integer values in {-2..2}: every element of every C block,
    the 19 tail sectors of dims 1-4 included, equal to the oracle bit for
    bit (K <= 1024, so every partial sum is an exact fp32 integer).  Unpadded,
    automatically with alignment gathers and without any."""
    prob = C.blockdiag_bf16(ld_align=ld_align, align=ld_align, int_values=True)
    plan, got = _parity(prob, axis="auto", exact=True, min_triples=64, layout=layout)
    s = plan.stats()
    assert s["launches_per_contract"] == (2 if (ld_align, layout) == (1, "auto") else 1)
    if layout == "auto":
        assert s["items_by_class"]["mfma_fast"] > 0


def test_blockdiag_bf16_small_blocks_ragged():
    """A ragged bf16 case spanning several tiles with odd edges: sector GEMMs
    100 x 141 x 139 (two column tiles, a partial K chunk), 83 x 116 x 6,
    25 x 37 x 150 and 25 x 55 x 149 (two column tiles)."""
    prob = C.random_problem(4209, nq=1, nkeys=(6, 6, 6), maxdim=150, qrange=2, dtype="bf16", two_leg=False,
                            dup_charges=False)
    shapes = sorted((int(prob.con.m.dim[m]), int(prob.con.k.dim[k]), int(prob.con.n.dim[n]))
                    for m, k, n in oracle.triples(prob.con))
    assert max(max(mm, nn) for mm, _, nn in shapes) > 128 and max(kk for _, kk, _ in shapes) > 64, shapes
    for axis in AXES:
        _parity(prob, axis=axis, min_triples=4)


def _chain_parity(ch, tol, axes=("auto", "auto", "auto"), exact=False):
    t = torch()
    ref = oracle.run_chain(ch)
    if exact:
        assert int_chain_bound(ch) < 2 ** 24, "integer chain must stay exact in fp32"
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
        if exact:
            assert np.array_equal(got[addr].astype(np.float64), ref[st.c_buf][addr]), (st.label, "not bit-exact")
            continue
        err = rel_frobenius(got, ref[st.c_buf], addr)
        assert err <= tol, (st.label, err)
        # per block, against the magnitudes of the stage's inputs
        check_blocks(st.con, got, ref[st.c_buf], ref[st.a_buf], ref[st.b_buf], tol, label=st.label)


@pytest.mark.parametrize("layout", ["coop", "natural"])
def test_small_chain(layout):
    _chain_parity(C.small_chain(seed=3, layout=layout), 1e-12)


def test_rabc_u1_chain():
    _chain_parity(C.rabc_u1(), 1e-12)
    _chain_parity(C.rabc_u1(), 1e-12, axes=("contract", "free_n", "free_m"))


def test_rabc_u1u1_chain():
    _chain_parity(C.rabc_u1u1(), 1e-5)


def test_rabc_u1_chain_int_bit_exact():
    """Full-size U(1) update (fp64) on integer values: every element exact."""
    _chain_parity(C.rabc_u1(values="int"), 0.0, exact=True)
    _chain_parity(C.rabc_u1(values="int"), 0.0, axes=("contract", "free_n", "free_m"), exact=True)


def test_rabc_u1u1_chain_int_bit_exact():
    """Full-size U(1)xU(1) update (fp32, natural layout, gathers) on integer values."""
    _chain_parity(C.rabc_u1u1(values="int"), 0.0, exact=True)


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


def test_current_stream_handle():
    """The binding enqueues on torch's current stream, also inside a stream
    context (its raw-stream query against the Stream object's handle)."""
    from block_sparse_tensor_amd import engine
    t = torch()
    assert engine._current_stream_raw() == t.cuda.current_stream().cuda_stream
    s = t.cuda.Stream()
    with t.cuda.stream(s):
        assert engine._current_stream_raw() == s.cuda_stream
    assert engine._current_stream_raw() == t.cuda.current_stream().cuda_stream
