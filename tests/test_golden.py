"""A hand-worked example (tests/golden/hand_worked_u1.json): two output sectors,
a contracted charge carried by two keys (so one C block sums two products), a
B block stored column-major and C buffer elements outside every C block.  Its
expected C buffer, triples and useful flops were worked out by hand from the
definition C_mn = sum_k A_mk B_kn over charge-conserving sectors; they pin the
oracle on the CPU and the HIP engine (bit for bit: every value is a small
integer, exact in bf16, f32 and f64 under any summation order) on the GPU."""
import json
import os

import numpy as np
import pytest

import oracle
from workloads.layout import view_addresses
from workloads.model import Contraction, Index, Operand

from gpuhelp import have_gpu, run_engine

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_u1.json")


def load(dtype="f64"):
    g = json.load(open(GOLDEN))

    def index(d):
        return Index(np.array(d["charge"])[:, None], np.array(d["dim"]))

    m, k, n = index(g["m"]), index(g["k"]), index(g["n"])

    def operand(d, elems):
        bl = d["blocks"]
        return Operand([b["row"] for b in bl], [b["col"] for b in bl], [b["offset"] for b in bl],
                       [[b["row_stride"], 1] for b in bl], [[b["col_stride"], 1] for b in bl], [0], elems)

    con = Contraction(m, k, n, operand(g["A"], len(g["A"]["buffer"])), operand(g["B"], len(g["B"]["buffer"])),
                      operand(g["C"], len(g["C"]["buffer_before"])), dtype)
    return g, con


def test_fixture_blocks_sit_in_their_buffers():
    """The written-out block values are what the buffers hold at those views."""
    g, con = load()
    for name, idx_r, idx_c in (("A", con.m, con.k), ("B", con.k, con.n)):
        buf = np.array(g[name]["buffer"], np.float64)
        for b in g[name]["blocks"]:
            rows, cols = int(idx_r.dim[b["row"]]), int(idx_c.dim[b["col"]])
            addr = view_addresses(b["offset"], [b["row_stride"], 1], [b["col_stride"], 1], rows, cols)
            np.testing.assert_array_equal(buf[addr], np.array(b["values"], np.float64))


def test_oracle_matches_hand_worked_values():
    g, con = load()
    oracle.check_structure(con)
    got = oracle.contract(con, np.array(g["A"]["buffer"], np.float64), np.array(g["B"]["buffer"], np.float64),
                          np.array(g["C"]["buffer_before"], np.float64))
    np.testing.assert_array_equal(got, np.array(g["C"]["buffer_after"], np.float64))
    np.testing.assert_array_equal(oracle.triples(con), np.array(g["triples_mkn_sorted_by_m_n_k"]))
    assert oracle.useful_flops(con) == g["useful_flops"]


@pytest.mark.gpu
@pytest.mark.skipif(not have_gpu(), reason="needs a GPU")
@pytest.mark.parametrize("dtype", ["f64", "f32", "bf16"])
@pytest.mark.parametrize("axis,mode", [("auto", "grouped"), ("free_m", "grouped"), ("free_n", "grouped"),
                                       ("contract", "grouped"), ("none", "per_sector")])
def test_engine_matches_hand_worked_values(dtype, axis, mode):
    import block_sparse_tensor_amd as bst
    g, con = load(dtype)
    print(f"[golden] hand_worked_u1 dtype={dtype} axis={axis} mode={mode}", flush=True)
    plan = bst.Plan(con, axis=axis, launch_mode=mode).bind()
    t, _, _ = plan.export()
    np.testing.assert_array_equal(t, np.array(g["triples_mkn_sorted_by_m_n_k"]))
    assert plan.stats()["useful_flops"] == g["useful_flops"]
    got = run_engine(plan, np.array(g["A"]["buffer"]), np.array(g["B"]["buffer"]),
                     np.array(g["C"]["buffer_before"]), dtype)
    np.testing.assert_array_equal(got.astype(np.float64), np.array(g["C"]["buffer_after"], np.float64))
