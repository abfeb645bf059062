"""Generator check values: sector structures derived independently from the
configuration texts (dims, sector GEMM counts, useful flops, tail fractions)."""
import numpy as np

import oracle
from workloads import configs as C
from workloads.model import bf16_bits, bf16_round


def test_tiny_u1_dims_and_counts():
    p = C.tiny_u1()
    dm, dk, dn = p.info["dims"]
    assert dm.tolist() == [8, 5, 7, 1, 5]
    assert dk.tolist() == [2, 7, 7, 2, 1]
    assert dn.tolist() == [4, 2, 4, 6, 1]
    assert len(oracle.triples(p.con)) == 5 and oracle.useful_flops(p.con) == 694
    f = C.tiny_u1("flux1")
    assert len(oracle.triples(f.con)) == 4 and oracle.useful_flops(f.con) == 452


def test_ragged_batch_counts():
    p = C.ragged_batch()
    t = oracle.triples(p.con)
    assert len(t) == 4000
    fl = 2 * p.con.m.dim[t[:, 0]] * p.con.k.dim[t[:, 1]] * p.con.n.dim[t[:, 2]]
    assert int(fl.sum()) == 191006
    assert abs(float((fl <= 64).mean()) - 0.81825) < 1e-9
    assert oracle.algorithmic_bytes(p.con) == 276204


def test_rabc_u1_structure():
    ch = C.rabc_u1()
    D = ch.info["D"]
    assert D.tolist() == [1, 1, 1, 1, 2, 3, 4, 7, 9, 13, 17, 22, 28, 34, 41, 48, 55, 60, 64, 67, 68, 67,
                          64, 60, 55, 48, 41, 34, 28, 22, 17, 13, 9, 7, 4, 3, 2, 1, 1, 1, 1]
    assert [len(oracle.triples(s.con)) for s in ch.stages] == [804, 2586, 804]
    assert len(ch.info["W"]) == 64
    assert ch.stages[1].con.m.nkeys == 199
    t = oracle.triples(ch.stages[0].con)
    st = ch.stages[0].con
    fl = 2 * st.m.dim[t[:, 0]] * st.k.dim[t[:, 1]] * st.n.dim[t[:, 2]]
    assert abs(float((fl <= 1024).mean()) - 0.378) < 1e-3


def test_rabc_u1u1_structure():
    ch = C.rabc_u1u1()
    D = ch.info["D"]
    assert len(D) == 177 and int(D.sum()) == 4096 and int(D.max()) == 136 and int((D <= 4).sum()) == 76
    assert len(ch.info["W"]) == 28
    assert [len(oracle.triples(s.con)) for s in ch.stages] == [3778, 4541, 2570]


def test_blockdiag_bf16_structure():
    p = C.blockdiag_bf16(values=False)
    d = p.info["dims"]
    assert len(d) == 64 and int(d.sum()) == 16373 and int(d.max()) == 1024
    assert oracle.useful_flops(p.con) == 10183642630


def test_bf16_rounding_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-3], np.float32)
    r = bf16_round(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == np.float32(1.0 + 2 ** -6) and r[3] == 1.0
    assert r[4] == -2.5
    bf16_bits(r)  # exact after rounding
