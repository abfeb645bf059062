"""Storage helpers for the seeded generators: placing blocks in flat buffers.

These only decide where block elements live and write generated values there;
they perform no contraction arithmetic.
"""
from __future__ import annotations

import numpy as np


def view_addresses(offset, rs, cs, rows, cols, ri=1, ci=1):
    """Element addresses [rows, cols] of a strided block view (2 legs per side)."""
    r = np.arange(rows, dtype=np.int64)
    c = np.arange(cols, dtype=np.int64)
    rp = (r // ri) * int(rs[0]) + (r % ri) * int(rs[1])
    cp = (c // ci) * int(cs[0]) + (c % ci) * int(cs[1])
    return int(offset) + rp[:, None] + cp[None, :]


def write_block(buf, offset, rs, cs, values, ri=1, ci=1):
    rows, cols = values.shape
    buf[view_addresses(offset, rs, cs, rows, cols, ri, ci)] = values


def round_up(x: int, a: int) -> int:
    return ((int(x) + a - 1) // a) * a


class Arena:
    """Bump allocator for block storage inside one flat buffer."""

    def __init__(self, align: int = 1):
        self.top = 0
        self.align = max(1, int(align))

    def take(self, n: int) -> int:
        off = round_up(self.top, self.align)
        self.top = off + int(n)
        return off
