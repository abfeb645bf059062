"""Single-sector GEMMs through the engine: tile-edge shapes (below, at and past
the 32/64/128/256 tile edges, ragged K), every operand orientation, padded and
unpadded leading dimensions.  Integer-valued inputs make every summation order
exact, so results must equal the plain product bit-for-bit (one sector is a
plain GEMM)."""
import numpy as np
import pytest

from workloads.layout import write_block
from workloads.model import Contraction, Index, Operand

from gpuhelp import have_gpu, to_dev, torch

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst

SHAPES = [(1, 1, 1), (7, 3, 5), (32, 16, 32), (64, 32, 64), (65, 17, 63), (128, 32, 128), (128, 33, 128),
          (129, 64, 127), (200, 40, 150), (256, 96, 256), (64, 1024, 64), (300, 7, 300), (17, 300, 9),
          (1100, 70, 1), (1100, 3, 16), (5, 130, 1030), (16, 65, 513), (17, 5, 700), (257, 33, 129),
          (384, 160, 96), (70, 48, 200),
          (300, 600, 200), (130, 520, 70)]


def _single(M, K, N, dtype, a_row, b_row, pad, seed, off=3):
    rng = np.random.default_rng(seed)
    fdt = np.float64 if dtype == "f64" else np.float32
    A = rng.integers(-2, 3, (M, K)).astype(fdt)
    B = rng.integers(-2, 3, (K, N)).astype(fdt)
    if a_row:
        lda = K + pad
        ars, acs, na = (lda, 0), (1, 0), M * lda
    else:
        lda = M + pad
        ars, acs, na = (1, 0), (lda, 0), K * lda
    if b_row:
        ldb = N + pad
        brs, bcs, nb = (ldb, 0), (1, 0), K * ldb
    else:
        ldb = K + pad
        brs, bcs, nb = (1, 0), (ldb, 0), N * ldb
    abuf, bbuf = np.zeros(na + off + 8, fdt), np.zeros(nb + off + 8, fdt)
    write_block(abuf, off, ars, acs, A)
    write_block(bbuf, off, brs, bcs, B)
    idx = lambda d: Index([[0]], [d])
    con = Contraction(idx(M), idx(K), idx(N), Operand([0], [0], [off], [ars], [acs], [0], na + off + 8),
                      Operand([0], [0], [off], [brs], [bcs], [0], nb + off + 8),
                      Operand([0], [0], [0], [(N, 0)], [(1, 0)], [0], M * N), dtype)
    return con, abuf, bbuf, A @ B


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f64"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_single_sector_exact(dtype, shape):
    t = torch()
    M, K, N = shape
    for a_row in (True, False):
        for b_row in (True, False):
            for pad, off in ((0, 3), (8, 3), (0, 0), (8, 8), ((-K) % 8 if a_row else (-M) % 8, 0)):
                con, abuf, bbuf, ref = _single(M, K, N, dtype, a_row, b_row, pad, M * 1000 + K * 10 + N, off)
                print(f"[tile] {dtype} {M}x{K}x{N} a_row={a_row} b_row={b_row} pad={pad} off={off}", flush=True)
                plan = bst.Plan(con).bind()
                cdt = t.float64 if dtype == "f64" else t.float32
                C = t.full((M * N,), float("nan"), dtype=cdt, device="cuda")
                plan.contract(to_dev(abuf, dtype), to_dev(bbuf, dtype), C)
                t.cuda.synchronize()
                got = C.cpu().numpy().reshape(M, N)
                assert np.array_equal(got, ref.astype(got.dtype)), (
                    f"{int(np.sum(got != ref))} of {M * N} elements differ")


def test_fast_path_selected():
    """Aligned, padded operands take the direct-to-LDS matrix-core tile (256 x 128)."""
    con, _, _, _ = _single(256, 256, 256, "bf16", True, True, 8, 1, 0)
    s = bst.Plan(con).stats()
    assert s["items_by_class"]["mfma_fast"] == 2
    con, _, _, _ = _single(256, 256, 256, "bf16", True, False, 8, 1, 0)
    assert bst.Plan(con).stats()["items_by_class"]["mfma_fast"] == 2
    con, _, _, _ = _single(256, 256, 256, "bf16", True, True, 0, 1, 3)
    assert bst.Plan(con).stats()["items_by_class"]["mfma"] == 4


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_matrix_core_class_for_fp32_fp64(dtype):
    """fp32 / fp64 groups of more than a few matrix-core steps run on 64 x 64 matrix-core tiles."""
    con, _, _, _ = _single(130, 20, 70, dtype, True, True, 0, 1, 0)
    s = bst.Plan(con).stats()
    assert s["items_by_class"]["mfma"] == 3 * 2 and s["items_by_class"]["generic"] == 0
    con, _, _, _ = _single(20, 20, 70, dtype, True, True, 0, 1, 0)
    assert bst.Plan(con).stats()["items_by_class"]["mfma"] == 2
    con, _, _, _ = _single(24, 4, 24, dtype, True, True, 0, 1, 0)
    assert bst.Plan(con).stats()["items_by_class"]["generic"] == 1


@pytest.mark.parametrize("dtype", ["bf16", "f32", "f64"])
def test_skinny_class(dtype):
    """Groups with at most 16 output rows or columns stream through the skinny tile."""
    # 256 threads x R lines per tile, R x (short extent rounded to 4/8/16) = 32
    budget = 32
    con, _, _, _ = _single(1300, 20, 16, dtype, True, True, 0, 1, 0)
    assert bst.Plan(con).stats()["items_by_class"]["skinny"] == -(-1300 // (256 * (budget // 16)))
    con, _, _, _ = _single(7, 20, 600, dtype, True, True, 0, 1, 0)
    assert bst.Plan(con).stats()["items_by_class"]["skinny"] == -(-600 // (256 * (budget // 8)))
    con, _, _, _ = _single(5000, 9, 1, dtype, True, True, 0, 1, 0)
    assert bst.Plan(con).stats()["items_by_class"]["skinny"] == -(-5000 // (256 * (budget // 4)))


@pytest.mark.parametrize("shape", [(128, 96, 128), (100, 640, 152), (64, 1030, 70), (33, 40, 24), (300, 600, 200)],
                         ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("tile_rows", [128, 256])
def test_tile_rows_forced(shape, tile_rows):
    """Both direct-to-LDS tile heights (128 rows: five-stage ring, waves of the
    idle row half compute nothing) on aligned operands, both B orientations:
    bit-exact on integer inputs."""
    t = torch()
    M, K, N = shape
    for b_row in (True, False):
        con, abuf, bbuf, ref = _single(M, K, N, "bf16", True, b_row, (-K) % 8, 2, 0)
        plan = bst.Plan(con, tile_rows=tile_rows).bind()
        assert plan.stats()["items_by_class"]["mfma_fast"] > 0
        print(f"[tile] bf16 {M}x{K}x{N} b_row={b_row} tile_rows={tile_rows}", flush=True)
        C = t.full((M * N,), float("nan"), dtype=t.float32, device="cuda")
        plan.contract(to_dev(abuf, "bf16"), to_dev(bbuf, "bf16"), C)
        t.cuda.synchronize()
        got = C.cpu().numpy().reshape(M, N)
        assert np.array_equal(got, ref.astype(got.dtype))
