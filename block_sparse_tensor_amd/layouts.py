"""Cross-stage layout planning for chains of contractions (host-side descriptor
rewriting; no device work).

The C library's bsc_plan_layout lays out one operand of one contraction so
that the contraction's coalescing groups address their members as single
strided views (uni20 "block coalescing", "Interleaved vs contiguous — the real
tradeoff is a copy": the zero-copy arrangement needs the coalesced axis laid
out interleaved; "Open questions": the axis may differ per stage).  In a
chain an intermediate is written by one stage and read by the next through a
different matrix view of the same tensor blocks (other legs fused into rows
and columns).  `relayout_chain` asks the library for the layout one stage
wants for each buffer (its writer or a reader, see below) and rewrites every
stage's view of that buffer to match:

* a tensor block is identified in every view by its first element's offset
  (views of one block all start there; the source layout must place blocks
  apart);
* each leg of a block (outer and inner part of its row and column keys, extent
  > 1) is identified by its stride in the source layout; the consumer's new
  view gives each such leg its new stride, and every other view of the block
  takes the new strides of the same legs.

So the chosen stage addresses the buffer as single views, and every other
stage reaches the same memory through its own leg order.
"""
from __future__ import annotations

import copy

import numpy as np

from .engine import Plan, plan_layout

# (coalescing axis, operand) pairs whose members a group addresses together:
# only for these does the layout decide between one view and several
_PANEL_ROLES = {("free_m", "A"), ("free_m", "C"), ("free_n", "B"), ("free_n", "C"), ("contract", "A"),
                ("contract", "B")}


def _legs(idx_r, idx_c, rk, ck, rs, cs):
    """[(extent, stride)] of the four legs of one block view (extent-1 legs dropped)."""
    R = int(idx_r.dim[rk])
    Cd = int(idx_c.dim[ck])
    Ri = 1 if idx_r.inner is None else int(idx_r.inner[rk])
    Ci = 1 if idx_c.inner is None else int(idx_c.inner[ck])
    legs = [(R // Ri, int(rs[0])), (Ri, int(rs[1])), (Cd // Ci, int(cs[0])), (Ci, int(cs[1]))]
    return [(e, s) for e, s in legs if e > 1]


def _views(con, which):
    """(row index, column index, operand) of operand `which` of a contraction."""
    return {"A": (con.m, con.k, con.A), "B": (con.k, con.n, con.B), "C": (con.m, con.n, con.C)}[which]


def relayout_chain(stages, align: int = 1, consumer=None, axes=None, prefer: str = "writer"):
    """stages: [(con, a_buf, b_buf, c_buf)] over named buffers (source layout);
    axes: the coalescing axis each stage will be planned with (default "auto").
    consumer: optional {buffer: (stage index, "A"|"B"|"C")} overriding which
    view a buffer's layout is planned for.  Default: a buffer some stage
    writes is laid out for its first writer when prefer="writer" and that
    writer's grouping coalesces its output (the epilogue then writes whole
    lines; on the environment updates this beat laying intermediates out for
    their readers), otherwise for the first stage that reads it in a role its
    grouping coalesces, else the first reader, else the first writer.
    Returns (new contractions, {buffer: new length}, {buffer: block map}) where
    a block map is {source offset: (new offset, {source stride: new stride})}."""
    uses = {}
    for i, (con, a, b, c) in enumerate(stages):
        for which, buf in (("A", a), ("B", b), ("C", c)):
            uses.setdefault(buf, []).append((i, which))
    chosen = dict(consumer or {})
    axis_of = {}

    def shapes_layout(i, which):
        # whether stage i's grouping coalesces its operand `which` (panel roles)
        if i not in axis_of:
            axis_of[i] = Plan(stages[i][0], axis=(axes[i] if axes else "auto")).stats()["axis_name"]
        return (axis_of[i], which) in _PANEL_ROLES

    if prefer not in ("writer", "reader"):
        raise ValueError("prefer must be 'writer' or 'reader'")
    for buf, us in uses.items():
        if buf not in chosen:
            reads = [u for u in us if u[1] != "C"]
            writes = [u for u in us if u[1] == "C"]
            shaped = [u for u in reads if shapes_layout(*u)]
            if prefer == "writer" and writes and shapes_layout(*writes[0]):
                chosen[buf] = writes[0]
            else:
                chosen[buf] = shaped[0] if shaped else (reads[0] if reads else us[0])

    maps, sizes = {}, {}
    for buf, (i, which) in chosen.items():
        con = stages[i][0]
        off, rs, cs, total = plan_layout(con, which, align=align, axis=(axes[i] if axes else "auto"))
        ir, ic, op = _views(con, which)
        bm = {}
        for j in range(len(op.row_key)):
            rk, ck = int(op.row_key[j]), int(op.col_key[j])
            old = _legs(ir, ic, rk, ck, np.reshape(op.row_stride, (-1, 2))[j], np.reshape(op.col_stride, (-1, 2))[j])
            new = _legs(ir, ic, rk, ck, rs[j], cs[j])
            strides = {}
            for (e, s_old), (_, s_new) in zip(old, new):
                if s_old in strides and strides[s_old] != s_new:
                    raise ValueError(f"{buf}: two legs of one block share a stride in the source layout")
                strides[s_old] = s_new
            bm[int(op.offset[j])] = (int(off[j]), strides)
        maps[buf] = bm
        sizes[buf] = total

    out = []
    for con, a, b, c in stages:
        nc = copy.deepcopy(con)
        for which, buf in (("A", a), ("B", b), ("C", c)):
            ir, ic, op = _views(nc, which)
            bm = maps[buf]
            rsa = np.array(np.reshape(op.row_stride, (-1, 2)), np.int64)
            csa = np.array(np.reshape(op.col_stride, (-1, 2)), np.int64)
            offs = np.array(op.offset, np.int64)
            for j in range(len(op.row_key)):
                key = int(offs[j])
                if key not in bm:
                    raise ValueError(f"{buf}: a block at offset {key} is absent from the planned view")
                new_off, strides = bm[key]
                rk, ck = int(op.row_key[j]), int(op.col_key[j])
                R, Cd = int(ir.dim[rk]), int(ic.dim[ck])
                Ri = 1 if ir.inner is None else int(ir.inner[rk])
                Ci = 1 if ic.inner is None else int(ic.inner[ck])
                ext = (R // Ri, Ri, Cd // Ci, Ci)
                src = (rsa[j, 0], rsa[j, 1], csa[j, 0], csa[j, 1])
                dst = []
                for e, s in zip(ext, src):
                    if e > 1:
                        if int(s) not in strides:
                            raise ValueError(f"{buf}: a leg of the block at offset {key} is not in the planned view")
                        dst.append(strides[int(s)])
                    else:
                        dst.append(1)
                offs[j] = new_off
                rsa[j] = dst[0:2]
                csa[j] = dst[2:4]
            op.offset, op.row_stride, op.col_stride = offs, rsa, csa
            op.buffer_elems = sizes[buf]
        out.append(nc)
    return out, sizes, maps


def move_blocks(src, con, which, new_con):
    """Copy the values of operand `which` from buffer `src` (laid out as in
    `con`) into a new buffer laid out as in `new_con` (host arrays)."""
    ir, ic, op = _views(con, which)
    _, _, nop = _views(new_con, which)
    dst = np.zeros(int(nop.buffer_elems), src.dtype)
    for j in range(len(op.row_key)):
        rk, ck = int(op.row_key[j]), int(op.col_key[j])
        a_old = _addresses(ir, ic, rk, ck, op, j)
        a_new = _addresses(ir, ic, rk, ck, nop, j)
        dst[a_new] = src[a_old]
    return dst


def _addresses(ir, ic, rk, ck, op, j):
    R, Cd = int(ir.dim[rk]), int(ic.dim[ck])
    Ri = 1 if ir.inner is None else int(ir.inner[rk])
    Ci = 1 if ic.inner is None else int(ic.inner[ck])
    rs = np.reshape(op.row_stride, (-1, 2))[j]
    cs = np.reshape(op.col_stride, (-1, 2))[j]
    r = np.arange(R)[:, None]
    c = np.arange(Cd)[None, :]
    return (int(op.offset[j]) + (r // Ri) * int(rs[0]) + (r % Ri) * int(rs[1]) + (c // Ci) * int(cs[0])
            + (c % Ci) * int(cs[1]))
