"""Plain containers for a block-sparse contraction's sector structure.

A matrix index is a list of keys (sectors).  Each key carries a charge vector
(U(1): one integer, U(1)xU(1): two), a dimension, and optionally an inner-leg
extent: a key of a fused multi-index such as (a', b) spans dim = outer * inner
elements, and element r of it is the pair (r // inner, r % inner).

An operand (A over (m,k), B over (k,n), C over (m,n)) is a list of blocks.  A
block is a strided view into one flat buffer: element (r, c) of block (row key,
col key) lives at

    offset + (r // Ri)*rs0 + (r % Ri)*rs1 + (c // Ci)*cs0 + (c % Ci)*cs1

where Ri, Ci are the inner extents of the row and column keys (1 for a single
leg).  This is the strided-view representation of a logical block over shared
storage that the uni20 "block coalescing" note describes (section "Expressed as
strided views over shared storage").

Nothing here computes a contraction.  These containers are shared by the seeded
generators, the CPU oracle and the GPU binding; they hold data only.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np


@dataclass
class Index:
    charge: np.ndarray                 # int32 [nkeys, nq]
    dim: np.ndarray                    # int64 [nkeys]
    inner: Optional[np.ndarray] = None  # int64 [nkeys] (dim % inner == 0) or None
    labels: Optional[list] = None      # human-readable key names (not used by the engine)

    def __post_init__(self):
        self.dim = np.ascontiguousarray(np.asarray(self.dim, dtype=np.int64))
        ch = np.asarray(self.charge, dtype=np.int32)
        nq = ch.shape[-1] if ch.ndim == 2 else (ch.size // max(1, len(self.dim)) or 1)
        self.charge = np.ascontiguousarray(ch.reshape(len(self.dim), nq))
        if self.inner is not None:
            self.inner = np.ascontiguousarray(np.asarray(self.inner, dtype=np.int64))

    @property
    def nkeys(self) -> int:
        return int(self.dim.shape[0])

    @property
    def nq(self) -> int:
        return int(self.charge.shape[1])

    def inner_of(self, key: int) -> int:
        return 1 if self.inner is None else int(self.inner[key])


@dataclass
class Operand:
    row_key: np.ndarray     # int32 [nb]
    col_key: np.ndarray     # int32 [nb]
    offset: np.ndarray      # int64 [nb]   (elements)
    row_stride: np.ndarray  # int64 [nb, 2] (outer, inner leg)
    col_stride: np.ndarray  # int64 [nb, 2]
    flux: np.ndarray        # int32 [nq]
    buffer_elems: int

    def __post_init__(self):
        nb = len(self.row_key)
        self.row_key = np.ascontiguousarray(np.asarray(self.row_key, dtype=np.int32))
        self.col_key = np.ascontiguousarray(np.asarray(self.col_key, dtype=np.int32))
        self.offset = np.ascontiguousarray(np.asarray(self.offset, dtype=np.int64))
        self.row_stride = np.ascontiguousarray(np.asarray(self.row_stride, dtype=np.int64).reshape(nb, 2))
        self.col_stride = np.ascontiguousarray(np.asarray(self.col_stride, dtype=np.int64).reshape(nb, 2))
        self.flux = np.ascontiguousarray(np.asarray(self.flux, dtype=np.int32).reshape(-1))
        self.buffer_elems = int(self.buffer_elems)

    @property
    def nblocks(self) -> int:
        return int(self.row_key.shape[0])


@dataclass
class Contraction:
    """C[m,n] = sum_k A[m,k] B[k,n] over the listed sectors (structure only)."""
    m: Index
    k: Index
    n: Index
    A: Operand
    B: Operand
    C: Operand
    dtype: str  # 'f64' | 'f32' | 'bf16' (bf16 inputs, fp32 C)


@dataclass
class Problem:
    """One contraction plus seeded input values.

    a, b hold the operand buffers.  For dtype 'bf16' they are float32 arrays whose
    values are exactly representable in bfloat16 (rounded to nearest even by the
    generator); `bf16_bits` gives the 16-bit patterns the device consumes.
    """
    name: str
    con: Contraction
    a: np.ndarray
    b: np.ndarray
    info: Dict = field(default_factory=dict)


@dataclass
class Stage:
    con: Contraction
    a_buf: str   # name of the buffer holding A
    b_buf: str
    c_buf: str
    label: str = ""


@dataclass
class Chain:
    """A sequence of contractions over named buffers (the R/A/B/C environment update)."""
    name: str
    stages: List[Stage]
    buffers: Dict[str, np.ndarray]      # input values; output buffers are zero-length placeholders
    sizes: Dict[str, int]               # element count of every buffer (inputs and outputs)
    dtype: str
    info: Dict = field(default_factory=dict)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    # NaN stays NaN (none are generated); infinities and normals round as integers do.
    return (r.astype(np.uint32)).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """16-bit patterns of float32 values that are already bfloat16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bfloat16-exact")
    return (u >> 16).astype(np.uint16)
