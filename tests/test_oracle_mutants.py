"""Planted mistakes in the oracle, each caught by named pins.

Each mutant below plants one plausible mistake in the CPU oracle (on the CPU,
by replacing one of its helpers for the duration of a test) and runs pins from
test_oracle.py / test_golden.py against it; every listed pin must then fail
with an assertion.  This shows the pins are sharp enough to see a dropped
term, a wrong sign, a transposed operand, a wrong fused-leg index, a wrong
k-list or a wrong overwrite/accumulate mode, rather than only agreeing with
the oracle as it is.

Mutants:
  negate_b        B blocks read with the wrong sign;
  transpose_a     square A blocks read transposed (row and column swapped);
  transpose_b     square B blocks read transposed;
  swap_legs       a fused (outer, inner) index decoded as (inner, outer);
  drop_term       the A block with the largest k of every row that has two or
                  more is skipped (a dropped term of the k sum);
  short_klist     the last contracted key is left out of every k-list (an
                  off-by-one bound over the keys);
  accumulate      every contraction adds onto what C holds (overwrite mode lost).
"""
import sys

import numpy as np
import pytest

import oracle
import test_golden
import test_oracle as T

MOD = sys.modules["oracle.contract"]
ORIG = {name: getattr(MOD, name) for name in ("block", "_maps", "contract")}


class _Current:
    con = None


def _tracking_contract(accumulate_always=False):
    def contract(con, a, b, c=None, accumulate=False, check=True):
        prev, _Current.con = _Current.con, con
        try:
            return ORIG["contract"](con, a, b, c, accumulate or (accumulate_always and c is not None), check)
        finally:
            _Current.con = prev
    return contract


def _block_mutant(which, kind):
    orig = ORIG["block"]

    def block(buf, op, i, ridx, cidx):
        con = _Current.con
        target = con is not None and op is getattr(con, which)
        if not target:
            return orig(buf, op, i, ridx, cidx)
        v = orig(buf, op, i, ridx, cidx)
        if kind == "negate":
            return -v
        if kind == "transpose" and v.shape[0] == v.shape[1]:
            return np.ascontiguousarray(v.T)
        return v
    return block


def _swap_legs_block(buf, op, i, ridx, cidx):
    """Decode a fused (outer, inner) row or column index as (inner, outer)."""
    rk, ck = int(op.row_key[i]), int(op.col_key[i])
    R, C = int(ridx.dim[rk]), int(cidx.dim[ck])
    Ri = 1 if ridx.inner is None else int(ridx.inner[rk])
    Ci = 1 if cidx.inner is None else int(cidx.inner[ck])
    rs0, rs1 = (int(x) for x in op.row_stride[i])
    cs0, cs1 = (int(x) for x in op.col_stride[i])
    it = buf.itemsize
    v = np.lib.stride_tricks.as_strided(buf[int(op.offset[i]):], shape=(Ri, R // Ri, Ci, C // Ci),
                                        strides=(rs1 * it, rs0 * it, cs1 * it, cs0 * it), writeable=False)
    return np.array(v, dtype=np.float64).reshape(R, C)


def _drop_term_maps(con):
    a, b, c = ORIG["_maps"](con)
    by_row = {}
    for (m, k) in a:
        by_row.setdefault(m, []).append(k)
    for m, ks in by_row.items():
        if len(ks) >= 2:
            del a[(m, max(ks))]
    return a, b, c


def _short_klist_maps(con):
    a, b, c = ORIG["_maps"](con)
    last = con.k.nkeys - 1
    return a, {kn: i for kn, i in b.items() if kn[0] != last}, c


MUTANTS = {
    "negate_b": dict(block=_block_mutant("B", "negate")),
    "transpose_a": dict(block=_block_mutant("A", "transpose")),
    "transpose_b": dict(block=_block_mutant("B", "transpose")),
    "swap_legs": dict(block=_swap_legs_block),
    "drop_term": dict(_maps=_drop_term_maps),
    "short_klist": dict(_maps=_short_klist_maps),
    "accumulate": dict(accumulate_always=True),
}

# pins, by name: each a call of a test from test_oracle / test_golden
# a case with fused two-leg keys of both extents > 1 in operands (U(1), flux (1, -1), all blocks)
TWO_LEG_DUP = next(c for c in T.RANDOM_CASES if c["two_leg"] and c["density"] == 1.0 and c["nq"] == 1
                   and c["flux"] == (1, -1))
PINS = {
    "P1_dense": lambda: T.test_p1_dense_bruteforce_random(TWO_LEG_DUP),
    "P1_tiny_dense": lambda: T.test_p1_tiny_u1_dense("flux1_3leg"),
    "P3_identity": lambda: T.test_p3_identity_and_permutation("identity", 0),
    "P6_plain_gemm": lambda: T.test_p6_single_sector_is_plain_gemm((16, 16, 16), "rc"),
    "P7_triples": lambda: T.test_p7_triples_bruteforce(0),
    "P11_dense_einsum": lambda: T.test_p11_chain_vs_dense_einsum("coop"),
    "P11_identity_env": lambda: T.test_p11_identity_environment(),
    "golden": lambda: test_golden.test_oracle_matches_hand_worked_values(),
    "accumulate_adds": lambda: T.test_accumulate_adds(),
}

# (mutant, pin) pairs that must fail
CAUGHT = [
    ("negate_b", "P1_dense"), ("negate_b", "P3_identity"), ("negate_b", "P11_identity_env"), ("negate_b", "golden"),
    ("transpose_a", "golden"), ("transpose_a", "P6_plain_gemm"),
    ("transpose_b", "golden"), ("transpose_b", "P6_plain_gemm"), ("transpose_b", "P11_dense_einsum"),
    ("swap_legs", "P1_dense"), ("swap_legs", "P11_dense_einsum"),
    ("drop_term", "P1_dense"), ("drop_term", "golden"), ("drop_term", "P11_dense_einsum"),
    ("short_klist", "P1_dense"), ("short_klist", "P7_triples"), ("short_klist", "golden"),
    ("accumulate", "P1_dense"), ("accumulate", "golden"),
]


def _plant(monkeypatch, mutant):
    spec = MUTANTS[mutant]
    wrapped = _tracking_contract(spec.get("accumulate_always", False))
    monkeypatch.setattr(MOD, "contract", wrapped)
    monkeypatch.setattr(oracle, "contract", wrapped)
    for name in ("block", "_maps"):
        if name in spec:
            monkeypatch.setattr(MOD, name, spec[name])


@pytest.mark.parametrize("pin", sorted(PINS))
def test_pins_pass_unmutated(monkeypatch, pin):
    """The harness itself changes nothing: with the tracking wrapper only, every pin passes."""
    wrapped = _tracking_contract(False)
    monkeypatch.setattr(MOD, "contract", wrapped)
    monkeypatch.setattr(oracle, "contract", wrapped)
    PINS[pin]()


@pytest.mark.parametrize("mutant,pin", CAUGHT, ids=[f"{m}-{p}" for m, p in CAUGHT])
def test_planted_mistake_fails_pin(monkeypatch, mutant, pin):
    _plant(monkeypatch, mutant)
    with pytest.raises(AssertionError):
        PINS[pin]()
