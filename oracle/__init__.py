"""CPU oracle for block-sparse contractions over symmetry sectors.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
anything in this package: only the tests, `__graft_entry__.smoke()` and the
`cpu_baseline` leg of `bench.py` use it.  It shares no code with the HIP engine
(`block_sparse_tensor_amd`) and never imports it.

What it computes is the plain definition of the block GEMM from the uni20
"block coalescing" note (section "Why single-axis coalescing is hole-free"):
for every C block (m, n),  C_mn = sum over k of A_mk B_kn, taken over the k for
which both blocks exist, in float64, one sector at a time.  Coalescing is a
lowering that never changes the representation (same note, "Decisions made"),
so this uncoalesced loop is the reference result for every plan.

Pins (see tests/test_oracle.py): dense brute force on zero-filled materialised
matrices, identity/orthogonal special cases, exact linearity, plain-GEMM
reduction, brute-force sector enumeration, and the R/A/B/C chain against a dense
einsum and the identity-environment closed form.  The grouping re-derivation
(`groups`) is pinned by its structural invariants (partition, single axis,
hole-free, canonical order).  Operand-mode choice, tile classes and work order
affect only speed: parity unpinned, covered by coalesced == uncoalesced.
"""
from .contract import (  # noqa: F401
    OracleError, block, check_structure, contract, densify, groups,
    useful_flops, algorithmic_bytes, triples, run_chain,
)
