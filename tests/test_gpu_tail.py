"""GPU parity of the tail bundles (whole near-zero-flop groups of one run of
single views, one per wave, up to four per workgroup): integer-valued inputs
compare bit for bit with the oracle in every dtype, over bundles whose groups
have different shapes (1 x 1 up to tens of outputs, a lane per output or
several lanes per output with a butterfly sum), strided and transposed block
layouts, under every grouping axis, in overwrite and accumulate mode, and the
ragged batch of 4000 GEMMs whose tiniest groups are all tail."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import c_addresses, canary, check_canary, check_float, have_gpu, run_engine

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:
    bst = None


def _tail_bundles(plan):
    return plan.stats()["items_by_class"]["tail"]


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("axis", ["auto", "free_m", "free_n", "contract"])
@pytest.mark.parametrize("seed", [85, 134, 124])
def test_tail_integer_bit_exact(dtype, axis, seed):
    prob = C.random_problem(seed, nq=1, nkeys=(10, 9, 10), maxdim=8, qrange=1, dtype=dtype, int_values=True,
                            density=0.9, two_leg=False)
    con = prob.con
    plan = bst.Plan(con, axis=axis).bind()
    print(f"[tail] seed={seed} {dtype} axis={axis} bundles={_tail_bundles(plan)} "
          f"triples={plan.stats()['triples']}", flush=True)
    assert _tail_bundles(plan) > 0 and plan.stats()["triples"] >= 8
    addr, mask = c_addresses(con)
    got = run_engine(plan, prob.a, prob.b, canary(con, dtype), dtype)
    check_canary(got, mask)
    ref = oracle.contract(con, prob.a, prob.b, np.zeros(con.C.buffer_elems), check=False)
    assert np.array_equal(got[addr], ref[addr].astype(got.dtype))


@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
def test_tail_accumulate_bit_exact(dtype):
    prob = C.random_problem(203, nq=1, nkeys=(9, 8, 9), maxdim=8, qrange=1, dtype=dtype, int_values=True,
                            two_leg=False)
    con = prob.con
    plan = bst.Plan(con, accumulate=True).bind()
    assert _tail_bundles(plan) > 0
    addr, mask = c_addresses(con)
    c0 = np.where(mask, 3.0, np.nan)
    print(f"[tail] accumulate {dtype}", flush=True)
    got = run_engine(plan, prob.a, prob.b, c0, dtype, repeats=2)
    ref = oracle.contract(con, prob.a, prob.b, np.asarray(c0, np.float64), accumulate=True, check=False)
    ref = oracle.contract(con, prob.a, prob.b, ref, accumulate=True, check=False)
    assert np.array_equal(got[addr], ref[addr].astype(got.dtype))


def test_tail_ragged_batch_float_and_int():
    prob = C.ragged_batch()
    con = prob.con
    plan = bst.Plan(con).bind()
    assert _tail_bundles(plan) >= 50 and plan.stats()["launches_per_contract"] == 1
    print("[tail] ragged batch", flush=True)
    got = run_engine(plan, prob.a, prob.b, canary(con, "f32"), "f32")
    _, mask = c_addresses(con)
    check_canary(got, mask)
    ref = oracle.contract(con, prob.a, prob.b, np.zeros(con.C.buffer_elems), check=False)
    check_float(con, got, ref, prob.a, prob.b, 1e-5, label="ragged batch")
    # integer values on the same structure: bit for bit
    rng = np.random.default_rng(5)
    ai = rng.integers(-2, 3, prob.a.size).astype(np.float32)
    bi = rng.integers(-2, 3, prob.b.size).astype(np.float32)
    got = run_engine(plan, ai, bi, canary(con, "f32"), "f32")
    ref = oracle.contract(con, ai, bi, np.zeros(con.C.buffer_elems), check=False)
    addr, _ = c_addresses(con)
    assert np.array_equal(got[addr], ref[addr].astype(np.float32))
