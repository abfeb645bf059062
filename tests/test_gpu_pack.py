"""GPU parity of the gather (pack) path: operands the planner copies into the
contiguous workspace before the grouped launch.  The oracle knows nothing of
packing, so every case compares with it directly; integer-valued inputs make
every summation order exact, so packed and zero-copy plans must then agree
bit-for-bit, and with the oracle too."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import TOL, c_addresses, canary, check_canary, check_float, have_gpu, run_engine, to_dev, torch

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:
    bst = None


def _run(prob, **kw):
    con = prob.con
    print(f"[pack] {prob.name} dtype={con.dtype} {kw}", flush=True)
    plan = bst.Plan(con, **kw).bind()
    addr, mask = c_addresses(con)
    got = run_engine(plan, prob.a, prob.b, canary(con, con.dtype), con.dtype)
    check_canary(got, mask)
    return plan, got, addr


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("axis", ["free_m", "free_n", "contract"])
@pytest.mark.parametrize("seed", range(3))
def test_force_pack_random(dtype, axis, seed):
    prob = C.random_problem(8100 + seed, nq=1, nkeys=(7, 7, 7), maxdim=90, qrange=1, dtype=dtype, density=0.9)
    plan, got, addr = _run(prob, axis=axis, layout="force_pack")
    s = plan.stats()
    assert s["mode_count"]["A"]["segments"] == 0 and s["mode_count"]["B"]["segments"] == 0
    ref = oracle.contract(prob.con, prob.a, prob.b, np.full(prob.con.C.buffer_elems, np.nan))
    check_float(prob.con, got, ref, prob.a, prob.b, TOL[dtype], label=prob.name)


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_pack_integer_bit_exact(dtype):
    """Integer values: packed == zero-copy == oracle, bit for bit."""
    prob = C.random_problem(8200, nq=1, nkeys=(7, 7, 7), maxdim=140, qrange=1, dtype=dtype, density=0.9,
                            int_values=True)
    ref = oracle.contract(prob.con, prob.a, prob.b, np.full(prob.con.C.buffer_elems, np.nan))
    outs = []
    for layout in ("force_pack", "never_pack"):
        plan, got, addr = _run(prob, axis="contract", layout=layout)
        assert np.array_equal(got[addr], ref[addr].astype(got.dtype))
        outs.append(got)
    assert np.array_equal(outs[0][addr], outs[1][addr])


@pytest.mark.parametrize("layout", ["force_pack", "auto"])
def test_pack_natural_chain(layout):
    ch = C.small_chain(seed=3, layout="natural")
    t = torch()
    ref = oracle.run_chain(ch)
    bufs = {k: to_dev(v, ch.dtype) for k, v in ch.buffers.items()}
    for name, n in ch.sizes.items():
        if name not in bufs:
            bufs[name] = t.zeros(n, dtype=t.float64, device="cuda")
    for st in ch.stages:
        print(f"[pack] small chain stage {st.label} layout={layout}", flush=True)
        plan = bst.Plan(st.con, layout=layout).bind()
        plan.contract(bufs[st.a_buf], bufs[st.b_buf], bufs[st.c_buf])
    t.cuda.synchronize()
    for st in ch.stages:
        check_float(st.con, bufs[st.c_buf].cpu().numpy(), ref[st.c_buf], ref[st.a_buf], ref[st.b_buf], 1e-12,
                    label=st.label)


@pytest.mark.parametrize("layout", ["force_pack", "auto"])
def test_pack_rabc_u1u1_full_size(layout):
    """The full U(1)xU(1) environment update in its natural layout, every
    gatherable operand gathered (force_pack) or as the calibrated pack-cost
    model decides (auto: on this workload it gathers nothing, measured
    faster)."""
    ch = C.rabc_u1u1()
    t = torch()
    ref = oracle.run_chain(ch)
    bufs = {k: to_dev(v, ch.dtype) for k, v in ch.buffers.items()}
    for name, n in ch.sizes.items():
        if name not in bufs:
            bufs[name] = t.zeros(n, dtype=t.float32, device="cuda")
    packed = 0
    for st in ch.stages:
        print(f"[pack] rabc_u1u1 stage {st.label} layout={layout}", flush=True)
        plan = bst.Plan(st.con, layout=layout).bind()
        packed += plan.stats()["pack_bytes"]
        plan.contract(bufs[st.a_buf], bufs[st.b_buf], bufs[st.c_buf])
    t.cuda.synchronize()
    assert packed > 0 if layout == "force_pack" else packed >= 0
    for st in ch.stages:
        check_float(st.con, bufs[st.c_buf].cpu().numpy(), ref[st.c_buf], ref[st.a_buf], ref[st.b_buf], 1e-5,
                    label=st.label)


def test_pack_repeat_and_accumulate():
    """The workspace is rewritten by every contraction; accumulate mode adds onto C."""
    prob = C.random_problem(8100, nq=1, nkeys=(7, 7, 7), maxdim=90, qrange=1, dtype="f64", density=0.9)
    con = prob.con
    plan = bst.Plan(con, axis="free_n", layout="force_pack", accumulate=True).bind()
    addr, mask = c_addresses(con)
    c0 = np.where(mask, 1.0, np.nan)
    got = run_engine(plan, prob.a, prob.b, c0, "f64", repeats=3)
    ref = np.asarray(c0, np.float64)
    for _ in range(3):
        ref = oracle.contract(con, prob.a, prob.b, ref, accumulate=True)
    check_float(con, got, ref, prob.a, prob.b, 1e-12, label="repeat+accumulate")


def test_unaligned_operand_base_bf16():
    """Operand pointers off a 16-byte boundary: the launch leaves the
    direct-to-LDS tile out and its dense tasks run on the general tile."""
    prob = C.blockdiag_bf16(ld_align=8, align=8)
    con = prob.con
    plan = bst.Plan(con).bind()
    assert plan.stats()["items_by_class"]["mfma_fast"] > 0
    t = torch()
    addr, mask = c_addresses(con)
    A = to_dev(np.concatenate([[0.0], prob.a]), "bf16")[1:]
    B = to_dev(np.concatenate([[0.0], prob.b]), "bf16")[1:]
    assert A.data_ptr() % 16 != 0 and B.data_ptr() % 16 != 0
    Cd = t.full((con.C.buffer_elems,), float("nan"), dtype=t.float32, device="cuda")
    print("[pack] blockdiag_bf16 unaligned operand bases", flush=True)
    plan.contract(A, B, Cd)
    t.cuda.synchronize()
    got = Cd.cpu().numpy()
    ref = oracle.contract(con, prob.a, prob.b, np.zeros(con.C.buffer_elems), check=False)
    check_canary(got, mask)
    check_float(con, got, ref, prob.a, prob.b, 2e-2, label="unaligned")
