"""Host-side tests of the C-ABI library: it loads, exports every symbol the
header declares, and its planner (no device needed) matches the oracle's
independent sector join and grouping bit-exactly and rejects malformed input
with the documented status codes."""
import os
import re

import numpy as np
import pytest

import oracle
from oracle.contract import AXIS_AUTO, AXIS_CONTRACT, AXIS_FREE_M, AXIS_FREE_N
from workloads import configs as C

bst = pytest.importorskip("block_sparse_tensor_amd")
from block_sparse_tensor_amd import _capi  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib_or_skip():
    if not os.path.exists(_capi.LIB_PATH):
        pytest.skip("libbsc.so not built")
    return _capi.lib()


def test_exports_every_declared_symbol():
    L = _lib_or_skip()
    hdr = open(os.path.join(ROOT, "include", "bsc.h")).read()
    declared = set(re.findall(r"\b(bsc_[a-z_]+)\s*\(", hdr))
    assert declared == set(_capi.EXPORTED)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings():
    L = _lib_or_skip()
    for code, name in _capi.STATUS.items():
        assert L.bsc_status_string(code).decode() == name


AXES = {"free_m": AXIS_FREE_M, "free_n": AXIS_FREE_N, "contract": AXIS_CONTRACT, "auto": AXIS_AUTO}


def _check_against_oracle(con, axis):
    p = bst.Plan(con, axis=axis)
    t, g, md = p.export()
    s = p.stats()
    assert np.array_equal(t, oracle.triples(con).astype(np.int32))
    oax, ogid, ogl = oracle.groups(con, AXES[axis])
    assert s["axis"] == oax
    assert np.array_equal(g, ogid.astype(np.int32))
    assert s["groups"] == len(ogl)
    assert s["useful_flops"] == oracle.useful_flops(con)
    assert s["alg_bytes"] == oracle.algorithmic_bytes(con)
    return p, s


@pytest.mark.parametrize("axis", list(AXES))
def test_planner_matches_oracle_configs(axis):
    _lib_or_skip()
    for con in [C.tiny_u1("diag").con, C.tiny_u1("flux1").con, C.tiny_u1("flux1_3leg").con, C.ragged_batch().con,
                C.blockdiag_bf16(values=False).con] + [s.con for s in C.rabc_u1().stages]:
        _check_against_oracle(con, axis)


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("axis", list(AXES))
def test_planner_matches_oracle_random(seed, axis):
    _lib_or_skip()
    prob = C.random_problem(2000 + seed, nq=1 + seed % 2, nkeys=(7, 6, 7), maxdim=6, qrange=1,
                            flux=[(0, 0), (1, -1), (1, 0)][seed % 3], density=0.8)
    _check_against_oracle(prob.con, axis)


def test_per_sector_stats():
    _lib_or_skip()
    con = C.ragged_batch().con
    p = bst.Plan(con, launch_mode="per_sector")
    s = p.stats()
    assert s["launches_per_contract"] == 4000 and s["launches_per_sector"] == 4000
    g = bst.Plan(con, axis="free_m").stats()
    assert g["launches_per_contract"] == 1
    assert s["launches_per_sector"] / g["launches_per_contract"] >= 50


def test_blockdiag_bf16_one_launch():
    _lib_or_skip()
    # padded rows: one grouped launch, every large group on the direct-to-LDS tile
    s = bst.Plan(C.blockdiag_bf16(values=False, ld_align=8, align=8).con).stats()
    assert s["launches_per_contract"] == 1 and s["launches_per_sector"] == 64 and s["pack_bytes"] == 0
    # the as-generated layout gathers nothing when told not to
    s = bst.Plan(C.blockdiag_bf16(values=False).con, layout="never_pack").stats()
    assert s["launches_per_contract"] == 1 and s["items_by_class"]["mfma_fast"] == 0


def test_alignment_gathers():
    """bf16 groups whose single-view operands have rows off 16-byte boundaries:
    the planner gathers the misaligned operands of the large groups (the
    modelled saving at the two tiles' rates exceeds the traffic) into 16-byte
    rows, which puts those groups on the direct-to-LDS tile; small groups
    stay where they are."""
    _lib_or_skip()
    prob = C.blockdiag_bf16(values=False)
    con = prob.con
    s = bst.Plan(con).stats()
    assert s["launches_per_contract"] == 2 and s["pack_gain_align_us"] > s["pack_cost_us"] > 0
    assert s["items_by_class"]["mfma_fast"] > 0 and s["items_by_class"]["mfma"] > 0
    # the gathered operands are the misaligned blocks of the groups above the
    # modelled break-even (M N / (M + N) > ~150 for square blocks)
    dims = [int(d) for d in con.m.dim]
    big = [d for d in dims if d % 8 != 0 and d > 320]
    assert s["mode_count"]["A"]["pack"] >= len(big) and s["mode_count"]["B"]["pack"] >= len(big)
    assert s["pack_bytes"] >= sum(2 * 2 * d * d for d in big)
    # fp32 / fp64 plans have no direct-to-LDS tile: nothing to align
    p32 = C.blockdiag_bf16(values=False)
    p32.con.dtype = "f32"
    assert bst.Plan(p32.con, dtype="f32").stats()["pack_gain_align_us"] == 0


def test_zero_blocks_counted():
    _lib_or_skip()
    ch = C.rabc_u1u1()
    for st in ch.stages:
        s = bst.Plan(st.con).stats()
        t = oracle.triples(st.con)
        nonempty = len({(int(m), int(n)) for m, k, n in t})
        assert s["zero_blocks"] == st.con.C.nblocks - nonempty
        assert s["zero_groups"] == s["zero_blocks"]


# ---------------------------------------------------------------------------
# error codes (every plan-time failure is forced from the host)
# ---------------------------------------------------------------------------

def _err(con, **kw):
    with pytest.raises(bst.BscError) as e:
        bst.Plan(con, **kw)
    return e.value.name


def test_error_charge():
    _lib_or_skip()
    p = C.tiny_u1("diag")
    p.con.A.col_key[0] = 1
    assert _err(p.con) == "BSC_ERR_CHARGE"


def test_error_flux():
    _lib_or_skip()
    p = C.tiny_u1("diag")
    p.con.C.flux[:] = 1
    p.con.C.row_key[:] = p.con.C.row_key  # same blocks now break the rule or the flux sum
    assert _err(p.con) in ("BSC_ERR_CHARGE",)


def test_error_overlap():
    _lib_or_skip()
    p = C.tiny_u1("diag")
    p.con.C.offset[1] = p.con.C.offset[0]
    assert _err(p.con) == "BSC_ERR_OVERLAP"


def test_error_overlap_interleaved():
    """Interleaved C views that collide only element-wise are caught."""
    _lib_or_skip()
    p = C.tiny_u1("diag")
    # block 0 is 8x4 row-major at offset 0: make block 1 (5x2) interleave into its columns
    p.con.C.offset[1] = 1
    p.con.C.row_stride[1] = (4, 0)
    assert _err(p.con) == "BSC_ERR_OVERLAP"


def test_interleaved_disjoint_accepted():
    """Two column-interleaved C views that never collide are legal."""
    _lib_or_skip()
    from workloads.model import Contraction, Index, Operand
    idx = Index([[0], [0]], [3, 3])
    one = Index([[0]], [2])
    A = Operand([0, 1], [0, 0], [0, 6], [(2, 0), (2, 0)], [(1, 0), (1, 0)], [0], 12)
    B = Operand([0], [0], [0], [(2, 0)], [(1, 0)], [0], 4)
    # C blocks (0,0) and (1,0) are 3x2 each, interleaved: columns of block 0 at even, block 1 at odd addresses
    Cop = Operand([0, 1], [0, 0], [0, 1], [(4, 0), (4, 0)], [(2, 0), (2, 0)], [0], 12)
    con = Contraction(idx, one, one, A, B, Cop, "f64")
    bst.Plan(con, axis="contract")


def test_error_missing_output():
    _lib_or_skip()
    p = C.tiny_u1("diag")
    keep = np.arange(p.con.C.nblocks) != 2
    for f in ("row_key", "col_key", "offset", "row_stride", "col_stride"):
        setattr(p.con.C, f, getattr(p.con.C, f)[keep])
    assert _err(p.con) == "BSC_ERR_MISSING_OUTPUT"


def test_error_bounds():
    _lib_or_skip()
    p = C.tiny_u1("diag")
    p.con.B.buffer_elems = int(p.con.B.offset[-1])
    assert _err(p.con) == "BSC_ERR_BOUNDS"
    p = C.tiny_u1("diag")
    p.con.A.offset[0] = -1
    assert _err(p.con) == "BSC_ERR_BOUNDS"


def test_error_shape():
    _lib_or_skip()
    p = C.tiny_u1("diag")
    p.con.A.row_key[1] = p.con.A.row_key[0]
    p.con.A.col_key[1] = p.con.A.col_key[0]
    assert _err(p.con) == "BSC_ERR_SHAPE"          # duplicate block
    p = C.tiny_u1("diag")
    p.con.A.row_stride[0] = (0, 0)
    assert _err(p.con) == "BSC_ERR_SHAPE"          # zero stride on a leg of extent 8
    p = C.tiny_u1("diag")
    p.con.A.row_key[0] = 17
    assert _err(p.con) == "BSC_ERR_SHAPE"          # key out of range
    p = C.tiny_u1("diag")
    p.con.m.dim[0] = 0
    assert _err(p.con) == "BSC_ERR_SHAPE"


def test_error_axis_none_grouped():
    _lib_or_skip()
    assert _err(C.tiny_u1().con, axis="none") == "BSC_ERR_ARG"


def test_contract_before_bind():
    L = _lib_or_skip()
    import ctypes
    p = bst.Plan(C.tiny_u1().con)
    st = L.bsc_contract(p._h, ctypes.c_void_p(16), ctypes.c_void_p(16), ctypes.c_void_p(16), None)
    assert _capi.STATUS[st] == "BSC_ERR_NOT_BOUND"


def test_bind_too_small():
    L = _lib_or_skip()
    import ctypes
    p = bst.Plan(C.tiny_u1().con)
    st = L.bsc_plan_bind(p._h, ctypes.c_void_p(4096), ctypes.c_size_t(1), None)
    assert _capi.STATUS[st] == "BSC_ERR_DEVICE_BYTES"


def test_empty_problem():
    _lib_or_skip()
    from workloads.model import Contraction, Index, Operand
    idx = Index(np.zeros((0, 1)), [])
    op = Operand([], [], [], np.zeros((0, 2)), np.zeros((0, 2)), [0], 0)
    s = bst.Plan(Contraction(idx, idx, idx, op, op, op, "f32")).stats()
    assert s["triples"] == 0 and s["items"] == 0 and s["launches_per_contract"] == 0


def _packed_operands(plan):
    m = plan.stats()["mode_count"]
    return m["A"]["pack"] + m["B"]["pack"]


def test_pack_cost_model_responds_to_constants():
    """AUTO packs a scattered operand when the gather is cheap against the
    set-up it saves, and never when the gather (or the extra launch) costs more."""
    from workloads import configs as C
    ch = C.small_chain(seed=4, layout="natural")
    con = ch.stages[0].con
    base = _packed_operands(bst.Plan(con, layout="force_pack"))
    assert base > 0
    cheap = bst.Plan(con, layout="auto", pack_gbps=1e12, t_seg_us=10.0, t_launch_us=1e-6)
    assert _packed_operands(cheap) == base
    assert cheap.stats()["launches_per_contract"] == 2
    dear = bst.Plan(con, layout="auto", pack_gbps=1e-3, t_seg_us=10.0, t_launch_us=1e-6)
    assert _packed_operands(dear) == 0 and dear.stats()["pack_bytes"] == 0
    no_launch = bst.Plan(con, layout="auto", pack_gbps=1e12, t_seg_us=10.0, t_launch_us=1e9)
    assert _packed_operands(no_launch) == 0 and no_launch.stats()["launches_per_contract"] == 1
    assert _packed_operands(bst.Plan(con, layout="never_pack", pack_gbps=1e12, t_seg_us=10.0)) == 0


def test_pack_never_applies_to_single_view_operands():
    """An operand that already is one strided view over the group is never copied."""
    from workloads import configs as C
    prob = C.blockdiag_bf16(ld_align=8, align=8, values=False)
    plan = bst.Plan(prob.con, layout="force_pack")
    assert _packed_operands(plan) == 0 and plan.stats()["launches_per_contract"] == 1


def test_pack_workspace_in_device_bytes():
    from workloads import configs as C
    ch = C.small_chain(seed=4, layout="natural")
    con = ch.stages[0].con
    never = bst.Plan(con, layout="never_pack")
    forced = bst.Plan(con, layout="force_pack")
    info, _ = forced.worklist()
    esz = 8 if con.dtype == "f64" else 4
    assert forced.device_bytes() >= info["off_workspace"] + info["workspace_elems"] * esz
    assert info["workspace_elems"] * esz >= forced.stats()["pack_bytes"]
    assert forced.device_bytes() > never.device_bytes()


def test_header_is_plain_c(tmp_path):
    """include/bsc.h is a C header: it compiles as pedantic C99 with no C++."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "h.c"
    src.write_text('#include "bsc.h"\nint main(void) { bsc_options o; bsc_options_default(&o); return o.accumulate; }\n')
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                        "-fsyntax-only", str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_probe_mfma_checks_arguments():
    """The matrix-core probe refuses bad arguments before touching a device."""
    from ctypes import byref, c_double, c_void_p
    L = bst._capi.lib() if hasattr(bst, "_capi") else None
    if L is None:
        pytest.skip("library not built")
    f = c_double()
    assert L.bsc_probe_mfma(2, 0, c_void_p(1), None, byref(f)) == -1      # iters < 1
    assert L.bsc_probe_mfma(2, 10, None, None, byref(f)) == -1             # NULL sink
    assert L.bsc_probe_mfma(2, 10, c_void_p(1), None, None) == -1          # NULL flops
