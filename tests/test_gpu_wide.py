"""GPU parity of the wide bf16 tile (one workgroup per CU: 256 x 256 output).
A plan of wide tiles and tail bundles only runs eight waves of 128 x 64 per
workgroup (128 x 256 tiles of 64 x 64 waves for tiles of at most 128 rows,
the tail bundles on waves 0-3); a plan that also holds other tiles runs four
waves of 128 x 128 (128 x 64 for tiles of at most 128 columns).
Integer-valued inputs compare bit for bit with the oracle (every summation
order is exact), both B orientations, ragged edges, partial last K chunks,
K-slices, accumulation, several tiles per workgroup, unaligned operand bases,
and the bench workload's structure at full size (eight-wave form, its 1024^3
sector in 128-row tiles, tail bundles in the same launch)."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import c_addresses, canary, check_canary, check_float, have_gpu, run_engine, to_dev, torch
from test_gpu_split import _single
from workloads.layout import write_block
from workloads.model import Contraction, Index, Operand

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
          f"split_tiles={plan.stats()['split_tiles']} wide_only={plan.stats()['wide_only']}", flush=True)
    addr, mask = c_addresses(con)
    got = run_engine(plan, a, b, canary(con, "bf16"), "bf16")
    check_canary(got, mask)
    ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
    assert np.array_equal(got[addr], ref[addr].astype(np.float32))


def _blocks(dims, brow, seed):
    """Block-diagonal bf16 contraction: sector i is an M_i x K_i by K_i x N_i
    GEMM with 16-byte aligned rows, small integer values."""
    rng = np.random.default_rng(seed)
    nb = len(dims)
    lda = [(k + 7) // 8 * 8 for _, k, _ in dims]
    ldb = [(n + 7) // 8 * 8 for _, _, n in dims] if brow else [(k + 7) // 8 * 8 for _, k, _ in dims]
    aoff, boff, coff = [], [], []
    a_n = b_n = c_n = 0
    for (m, k, n), la, lb in zip(dims, lda, ldb):
        aoff.append(a_n); boff.append(b_n); coff.append(c_n)
        a_n += m * la
        b_n += k * lb if brow else n * lb
        c_n += m * n
    abuf, bbuf = np.zeros(a_n + 8, np.float32), np.zeros(b_n + 8, np.float32)
    brs = [((lb, 0), (1, 0)) if brow else ((1, 0), (lb, 0)) for lb in ldb]
    for i, (m, k, n) in enumerate(dims):
        write_block(abuf, aoff[i], (lda[i], 0), (1, 0), rng.integers(-2, 3, (m, k)).astype(np.float32))
        write_block(bbuf, boff[i], brs[i][0], brs[i][1], rng.integers(-2, 3, (k, n)).astype(np.float32))
    keys = [[i] for i in range(nb)]
    r = list(range(nb))
    con = Contraction(Index(keys, [d[0] for d in dims]), Index(keys, [d[1] for d in dims]),
                      Index(keys, [d[2] for d in dims]),
                      Operand(r, r, aoff, [(l, 0) for l in lda], [(1, 0)] * nb, [0], abuf.size),
                      Operand(r, r, boff, [b[0] for b in brs], [b[1] for b in brs], [0], bbuf.size),
                      Operand(r, r, coff, [(d[2], 0) for d in dims], [(1, 0)] * nb, [0], c_n), "bf16")
    return con, abuf, bbuf


@pytest.mark.parametrize("brow", [True, False])
@pytest.mark.parametrize("grid", [0, 8])
def test_wide_only_blocks_integer_bit_exact(brow, grid):
    """Several sectors, all on wide tiles (eight-wave workgroups), ragged
    edges and one K-split sector; grid 8 makes every workgroup loop over
    several tiles of the persistent task list."""
    dims = [(512, 512, 512), (300, 700, 260), (256, 96, 100), (700, 1200, 520), (64, 40, 300), (520, 256, 256)]
    con, a, b = _blocks(dims, brow, seed=31 + brow)
    plan = bst.Plan(con, tile_cols=256, split_k=12, grid_limit=grid).bind()
    s = plan.stats()
    print(f"[wide] blocks brow={brow} grid={grid} items={s['items']} split_tiles={s['split_tiles']} "
          f"wide_only={s['wide_only']}", flush=True)
    assert s["wide_only"] == 1 and s["split_tiles"] > 0
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
    assert s["wide_only"] == 1 and s["items_by_class"]["tail"] > 0
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


def test_wide_only_unaligned_bases_fall_back():
    """A plan of wide tiles only whose operand bases are off a 16-byte
    boundary runs on the general matrix-core tile (256-thread launch), K-split
    tiles included: integer values bit for bit."""
    con, a, b = _single(300, 700, 200, True, seed=41, ints=True)
    plan = bst.Plan(con, tile_cols=256, split_k=3).bind()
    s = plan.stats()
    assert s["wide_only"] == 1 and s["split_tiles"] > 0
    t = torch()
    A = to_dev(np.concatenate([[0.0], a]), "bf16")[1:]
    B = to_dev(np.concatenate([[0.0], b]), "bf16")[1:]
    assert A.data_ptr() % 16 != 0 and B.data_ptr() % 16 != 0
    addr, mask = c_addresses(con)
    Cd = t.tensor(canary(con, "bf16"), dtype=t.float32, device="cuda")
    print("[wide] wide-only plan, unaligned operand bases", flush=True)
    plan.contract(A, B, Cd)
    t.cuda.synchronize()
    got = Cd.cpu().numpy()
    check_canary(got, mask)
    ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
    assert np.array_equal(got[addr], ref[addr].astype(np.float32))
