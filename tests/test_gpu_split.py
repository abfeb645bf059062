"""GPU parity of K-split tiles: a 256 x 128 bf16 output tile cut into K-slices
that run as separate work items, the last to finish adding the partial tiles
in slice order.  The oracle knows nothing of splitting, so every case compares
with it directly; integer-valued inputs make every summation order exact, so
split and unsplit plans must agree bit-for-bit, and repeated launches (the
arrival counters reset themselves) must repeat bit-for-bit."""
import numpy as np
import pytest

import oracle
from workloads import configs as C
from workloads.layout import write_block
from workloads.model import Contraction, Index, Operand

from gpuhelp import c_addresses, canary, check_canary, check_float, have_gpu, run_engine, to_dev, torch

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:
    bst = None


def _single(M, K, N, brow, seed, ints=False, off=8):
    """One aligned bf16 GEMM block; values bf16-exact (small integers if ints)."""
    rng = np.random.default_rng(seed)
    if ints:
        A = rng.integers(-2, 3, (M, K)).astype(np.float32)
        B = rng.integers(-2, 3, (K, N)).astype(np.float32)
    else:
        A = C.bf16_round((rng.standard_normal((M, K)) * 0.05).astype(np.float32))
        B = C.bf16_round((rng.standard_normal((K, N)) * 0.05).astype(np.float32))
    lda, ldb, ldk = (K + 7) // 8 * 8, (N + 7) // 8 * 8, (K + 7) // 8 * 8
    brs, bcs = ((ldb, 0), (1, 0)) if brow else ((1, 0), (ldk, 0))
    abuf = np.zeros(off + M * lda + 8, np.float32)
    bbuf = np.zeros(off + max(K * ldb, N * ldk) + 8, np.float32)
    write_block(abuf, off, (lda, 0), (1, 0), A)
    write_block(bbuf, off, brs, bcs, B)
    idx = lambda d: Index([[0]], [d])
    con = Contraction(idx(M), idx(K), idx(N), Operand([0], [0], [off], [(lda, 0)], [(1, 0)], [0], abuf.size),
                      Operand([0], [0], [off], [brs], [bcs], [0], bbuf.size),
                      Operand([0], [0], [3], [(N + 1, 0)], [(1, 0)], [0], 3 + M * (N + 1)), "bf16")
    return con, abuf, bbuf


def _run(con, a, b, c0, **kw):
    plan = bst.Plan(con, **kw).bind()
    print(f"[split] {con.m.dim[0]}x{con.k.dim[0]}x{con.n.dim[0]} {kw} split_tiles={plan.stats()['split_tiles']}",
          flush=True)
    return plan, run_engine(plan, a, b, c0, "bf16")


def test_split_automatic_long_k():
    """A single tile with K = 20000: the automatic policy cuts it into slices."""
    con, a, b = _single(200, 20000, 100, True, seed=21)
    addr, mask = c_addresses(con)
    plan, got = _run(con, a, b, canary(con, "bf16"))
    assert plan.stats()["split_tiles"] >= 1
    check_canary(got, mask)
    ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
    check_float(con, got, ref, a, b, 2e-2, label="auto split")


@pytest.mark.parametrize("shape", [(300, 333, 150), (256, 1024, 128), (520, 1000, 260), (64, 700, 40)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("brow", [True, False])
@pytest.mark.parametrize("split_k", [1, 3, 0])
def test_split_parity(shape, brow, split_k):
    M, K, N = shape
    con, a, b = _single(M, K, N, brow, seed=M + K + N)
    addr, mask = c_addresses(con)
    plan, got = _run(con, a, b, canary(con, "bf16"), split_k=split_k)
    if split_k > 0:
        assert plan.stats()["split_tiles"] > 0
    check_canary(got, mask)
    ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
    check_float(con, got, ref, a, b, 2e-2)


@pytest.mark.parametrize("brow", [True, False])
@pytest.mark.parametrize("tile_rows", [128, 256])
def test_split_integer_bit_exact(brow, tile_rows):
    """Integer values: every slicing, at both tile heights, gives exactly the
    oracle's result."""
    con, a, b = _single(520, 1000, 260, brow, seed=5, ints=True)
    addr, _ = c_addresses(con)
    ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
    for split_k in (-1, 1, 2, 7):
        plan, got = _run(con, a, b, np.zeros(con.C.buffer_elems, np.float32), split_k=split_k, tile_rows=tile_rows)
        assert np.array_equal(got[addr], ref[addr].astype(np.float32)), split_k


def test_split_repeat_deterministic_and_accumulate():
    """Counters return to zero after every launch: five launches in a row give
    bit-identical results, and accumulate mode adds onto C once per launch."""
    con, a, b = _single(300, 900, 200, True, seed=9)
    addr, mask = c_addresses(con)
    t = torch()
    A, B = to_dev(a, "bf16"), to_dev(b, "bf16")
    plan = bst.Plan(con, split_k=2).bind()
    assert plan.stats()["split_tiles"] >= 4
    Cd = t.zeros(con.C.buffer_elems, dtype=t.float32, device="cuda")
    outs = []
    for i in range(5):
        print(f"[split] repeat {i}", flush=True)
        plan.contract(A, B, Cd)
        t.cuda.synchronize()
        outs.append(Cd.cpu().numpy().copy())
    for o in outs[1:]:
        assert np.array_equal(o[addr], outs[0][addr])
    ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
    check_float(con, outs[0], ref, a, b, 2e-2, label="repeat")
    pacc = bst.Plan(con, split_k=2, accumulate=True).bind()
    c0 = np.where(mask, 1.0, np.nan)
    got = run_engine(pacc, a, b, c0, "bf16", repeats=3)
    ref3 = oracle.contract(con, a, b, np.asarray(c0, np.float64), accumulate=True, check=False)
    ref3 = oracle.contract(con, a, b, ref3, accumulate=True, check=False)
    ref3 = oracle.contract(con, a, b, ref3, accumulate=True, check=False)
    check_float(con, got, ref3, a, b, 2e-2, label="accumulate x3")


@pytest.mark.parametrize("split_k", [15, 10, 6])
def test_split_normal_values_repeat_bit_identical(split_k):
    """Normal values, two to five slices: the partials are added in slice
    order whichever slice arrives last (the last slice adds the others around
    its own partial in that order), so launches repeat bit for bit."""
    con, a, b = _single(300, 900, 200, True, seed=10, ints=False)
    addr, mask = c_addresses(con)
    t = torch()
    A, B = to_dev(a, "bf16"), to_dev(b, "bf16")
    plan = bst.Plan(con, split_k=split_k).bind()
    assert plan.stats()["split_tiles"] >= 4
    Cd = t.zeros(con.C.buffer_elems, dtype=t.float32, device="cuda")
    outs = []
    for i in range(6):
        print(f"[split] normal repeat split_k={split_k} {i}", flush=True)
        plan.contract(A, B, Cd)
        t.cuda.synchronize()
        outs.append(Cd.cpu().numpy().copy())
    for o in outs[1:]:
        assert np.array_equal(o[addr], outs[0][addr])
    ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
    check_float(con, outs[0], ref, a, b, 2e-2, label=f"normal split_k={split_k}")


def test_split_unaligned_fallback():
    """Operand bases off a 16-byte boundary: split tiles run on the general
    matrix-core tile, the first slice computing the whole tile."""
    con, a, b = _single(300, 700, 200, False, seed=11, off=8)
    addr, mask = c_addresses(con)
    plan = bst.Plan(con, split_k=3).bind()
    assert plan.stats()["split_tiles"] > 0
    t = torch()
    A = to_dev(np.concatenate([[0.0], a]), "bf16")[1:]
    B = to_dev(np.concatenate([[0.0], b]), "bf16")[1:]
    assert A.data_ptr() % 16 != 0 and B.data_ptr() % 16 != 0
    Cd = t.full((con.C.buffer_elems,), float("nan"), dtype=t.float32, device="cuda")
    print("[split] unaligned operand bases", flush=True)
    plan.contract(A, B, Cd)
    t.cuda.synchronize()
    got = Cd.cpu().numpy()
    check_canary(got, mask)
    ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
    check_float(con, got, ref, a, b, 2e-2)


def test_split_blockdiag_full_size():
    """The block-diagonal bf16 workload at full size, every tile with K > 256 split."""
    prob = C.blockdiag_bf16(ld_align=8, align=8)
    con = prob.con
    plan = bst.Plan(con, split_k=8).bind()
    assert plan.stats()["split_tiles"] > 0
    addr, mask = c_addresses(con)
    print("[split] blockdiag_bf16 full size, slices of at most 256", flush=True)
    got = run_engine(plan, prob.a, prob.b, canary(con, "bf16"), "bf16", repeats=2)
    check_canary(got, mask)
    ref = oracle.contract(con, prob.a, prob.b, np.zeros(con.C.buffer_elems), check=False)
    check_float(con, got, ref, prob.a, prob.b, 2e-2, label="blockdiag split")
