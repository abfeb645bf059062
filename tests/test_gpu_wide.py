"""GPU parity of the wide bf16 tile (one workgroup per CU: 256 x 256 output,
four waves of 128 x 128; 128 x 64 waves for tiles of at most 128 columns):
integer-valued inputs compare bit for bit with the oracle (every summation
order is exact), both B orientations, ragged edges, partial last K chunks,
K-slices, accumulation, and the bench workload's structure at full size."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import c_addresses, canary, check_canary, check_float, have_gpu, run_engine, to_dev, torch
from test_gpu_split import _single

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:
    bst = None

SHAPES = [(256, 1024, 256), (300, 600, 200), (100, 640, 152), (520, 1000, 260), (64, 1030, 70), (33, 40, 24),
          (257, 96, 257), (1024, 1024, 1024), (8, 33, 300)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("brow", [True, False])
@pytest.mark.parametrize("split_k", [-1, 3])
def test_wide_single_integer_bit_exact(shape, brow, split_k):
    M, K, N = shape
    con, a, b = _single(M, K, N, brow, seed=M + 3 * K + 7 * N, ints=True)
    plan = bst.Plan(con, tile_cols=256, split_k=split_k).bind()
    print(f"[wide] {M}x{K}x{N} brow={brow} split_k={split_k} items={plan.stats()['items']} "
          f"split_tiles={plan.stats()['split_tiles']}", flush=True)
    addr, mask = c_addresses(con)
    got = run_engine(plan, a, b, canary(con, "bf16"), "bf16")
    check_canary(got, mask)
    ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
    assert np.array_equal(got[addr], ref[addr].astype(np.float32))


@pytest.mark.parametrize("brow", [True, False])
def test_wide_float_and_repeat(brow):
    """bf16-rounded Gaussian values: within tolerance, and five launches in a
    row (K-split counters reset by the last slice) repeat bit for bit."""
    con, a, b = _single(520, 1000, 300, brow, seed=17)
    t = torch()
    A, B = to_dev(a, "bf16"), to_dev(b, "bf16")
    plan = bst.Plan(con, tile_cols=256, split_k=2).bind()
    Cd = t.zeros(con.C.buffer_elems, dtype=t.float32, device="cuda")
    outs = []
    for i in range(5):
        print(f"[wide] repeat {i} brow={brow}", flush=True)
        plan.contract(A, B, Cd)
        t.cuda.synchronize()
        outs.append(Cd.cpu().numpy().copy())
    addr, _ = c_addresses(con)
    for o in outs[1:]:
        assert np.array_equal(o[addr], outs[0][addr])
    ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
    check_float(con, outs[0], ref, a, b, 2e-2, label="wide float")


def test_wide_accumulate():
    con, a, b = _single(300, 700, 280, True, seed=23, ints=True)
    plan = bst.Plan(con, tile_cols=256, accumulate=True).bind()
    addr, mask = c_addresses(con)
    c0 = np.where(mask, 1.0, np.nan)
    print("[wide] accumulate x2", flush=True)
    got = run_engine(plan, a, b, c0, "bf16", repeats=2)
    ref = oracle.contract(con, a, b, np.asarray(c0, np.float64), accumulate=True, check=False)
    ref = oracle.contract(con, a, b, ref, accumulate=True, check=False)
    assert np.array_equal(got[addr], ref[addr].astype(np.float32))


@pytest.mark.parametrize("split_k", [0, 4])
def test_wide_blockdiag_full_size_int_bit_exact(split_k):
    """The bench workload's structure on the wide tile, integer values, every
    element of every C block (tail sectors included) bit for bit."""
    prob = C.blockdiag_bf16(ld_align=8, align=8, int_values=True)
    con = prob.con
    plan = bst.Plan(con, tile_cols=256, split_k=split_k).bind()
    s = plan.stats()
    print(f"[wide] blockdiag_bf16 int split_k={split_k} items={s['items']} split_tiles={s['split_tiles']}",
          flush=True)
    assert s["launches_per_contract"] == 1 and s["items_by_class"]["mfma_fast"] > 0
    addr, mask = c_addresses(con)
    got = run_engine(plan, prob.a, prob.b, canary(con, "bf16"), "bf16")
    check_canary(got, mask)
    ref = oracle.contract(con, prob.a, prob.b, np.zeros(con.C.buffer_elems), check=False)
    assert np.array_equal(got[addr], ref[addr].astype(np.float32))


def test_wide_blockdiag_full_size_float():
    prob = C.blockdiag_bf16(ld_align=8, align=8)
    con = prob.con
    plan = bst.Plan(con, tile_cols=256).bind()
    addr, mask = c_addresses(con)
    print("[wide] blockdiag_bf16 float", flush=True)
    got = run_engine(plan, prob.a, prob.b, canary(con, "bf16"), "bf16")
    check_canary(got, mask)
    ref = oracle.contract(con, prob.a, prob.b, np.zeros(con.C.buffer_elems), check=False)
    check_float(con, got, ref, prob.a, prob.b, 2e-2, label="wide blockdiag")
