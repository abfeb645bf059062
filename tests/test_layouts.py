"""Host-side tests of layout planning: bsc_plan_layout (one operand of one
contraction laid out for its coalescing groups) and relayout_chain (every
buffer of a chain laid out for the stage that writes it or a stage that reads
it, every other view of the buffer rewritten to the same memory).

Pins: the layouts are valid descriptors (the planner accepts them, C stays
disjoint, panels and leading dimensions aligned), each group's members land
consecutively in ascending key order in their panel (checked against the
exported groups), workloads without membership conflicts become all single
views, and in a chain every view of a tensor element reaches the same new
address (the leg mapping is a bijection consistent across stages)."""
import copy

import numpy as np
import pytest

from workloads import configs as C
from workloads.layout import view_addresses

bst = pytest.importorskip("block_sparse_tensor_amd")
from block_sparse_tensor_amd import _capi  # noqa: E402


def _lib_or_skip():
    import os
    if not os.path.exists(_capi.LIB_PATH):
        pytest.skip("libbsc.so not built")


def _with_layout(con, which, align=1, **kw):
    off, rs, cs, tot = bst.plan_layout(con, which, align=align, **kw)
    c = copy.deepcopy(con)
    op = getattr(c, which)
    op.offset, op.row_stride, op.col_stride, op.buffer_elems = off, rs, cs, tot
    return c, (off, rs, cs, tot)


def _views_of(con, which):
    return {"A": (con.m, con.k, con.A), "B": (con.k, con.n, con.B), "C": (con.m, con.n, con.C)}[which]


def _block_addresses(con, which, j):
    ir, ic, op = _views_of(con, which)
    r, c = int(op.row_key[j]), int(op.col_key[j])
    ri = 1 if ir.inner is None else int(ir.inner[r])
    ci = 1 if ic.inner is None else int(ic.inner[c])
    return view_addresses(int(op.offset[j]), np.reshape(op.row_stride, (-1, 2))[j],
                          np.reshape(op.col_stride, (-1, 2))[j], int(ir.dim[r]), int(ic.dim[c]), ri, ci)


def _modes(con, **kw):
    s = bst.Plan(con, **kw).stats()
    return {k: (v["view"], v["pack"], v["segments"]) for k, v in s["mode_count"].items()}, s


CASES = {
    "tiny": lambda: C.tiny_u1("diag").con,
    "ragged": lambda: C.ragged_batch().con,
    "blockdiag": lambda: C.blockdiag_bf16(values=False).con,
    "rabc_u1_s1": lambda: C.rabc_u1(layout="natural").stages[0].con,
    "rabc_u1_s2": lambda: C.rabc_u1(layout="natural").stages[1].con,
    "rabc_u1u1_s1": lambda: C.rabc_u1u1(layout="natural").stages[0].con,
    "rand": lambda: C.random_problem(4).con,
}


@pytest.mark.parametrize("case", sorted(CASES))
@pytest.mark.parametrize("which", ["A", "B", "C"])
@pytest.mark.parametrize("align", [1, 8])
def test_layout_is_valid_and_aligned(case, which, align):
    _lib_or_skip()
    con = CASES[case]()
    new, (off, rs, cs, tot) = _with_layout(con, which, align=align)
    _modes(new)                                  # the planner accepts it (bounds, C disjointness)
    ir, ic, op = _views_of(new, which)
    seen = np.zeros(tot, bool)
    for j in range(len(op.row_key)):
        a = _block_addresses(new, which, j).ravel()
        assert a.min() >= 0 and a.max() < tot
        assert not seen[a].any()                 # blocks of the operand never overlap
        seen[a] = True
        assert rs[j][1] % align == 0             # leading dimension
        assert cs[j][1] == 1
    assert tot % align == 0


def _group_members(con, which, **kw):
    """{group: sorted [(panel key, along key)]} of operand `which`, from the plan's export."""
    p = bst.Plan(con, **kw)
    t, g, _ = p.export()
    axis = p.stats()["axis_name"]
    out = {}
    for (m, k, n), gid in zip(t, g):
        r, c = {"A": (m, k), "B": (k, n), "C": (m, n)}[which]
        out.setdefault(int(gid), set()).add((int(r), int(c)))
    return axis, out


@pytest.mark.parametrize("case", ["ragged", "rabc_u1_s1", "rabc_u1u1_s1", "rabc_u1_s2", "rand"])
@pytest.mark.parametrize("which", ["A", "B", "C"])
def test_members_consecutive_in_panels(case, which):
    """Every group whose blocks of this operand were free when it was placed
    finds them consecutive in ascending key order; with single-member-set
    workloads that is every group."""
    _lib_or_skip()
    con = CASES[case]()
    new, (off, rs, cs, tot) = _with_layout(con, which)
    axis, members = _group_members(con, which)
    stack_rows = {("free_m", "A"), ("free_m", "C"), ("contract", "B")}
    side = {("free_n", "B"), ("free_n", "C"), ("contract", "A")}
    if (axis, which) not in stack_rows | side:
        return
    _, _, op = _views_of(con, which)
    index = {(int(r), int(c)): j for j, (r, c) in enumerate(zip(op.row_key, op.col_key))}
    ir, ic, _ = _views_of(con, which)
    consecutive = 0
    for gid, blocks in members.items():
        panels = {}
        for r, c in blocks:
            pk, ak = (c, r) if (axis, which) in stack_rows else (r, c)
            panels.setdefault(pk, []).append(ak)
        for pk, aks in panels.items():
            aks.sort()
            js = [index[(ak, pk) if (axis, which) in stack_rows else (pk, ak)] for ak in aks]
            ok = True
            for j0, j1, ak in zip(js, js[1:], aks):
                step = (int(ir.dim[ak]) * int(rs[j0][1])) if (axis, which) in stack_rows else int(ic.dim[ak])
                ok &= int(off[j1]) == int(off[j0]) + step
            consecutive += ok
    assert consecutive > 0


@pytest.mark.parametrize("case", ["tiny", "ragged", "blockdiag", "rabc_u1_s1", "rabc_u1u1_s1", "rabc_u1_s2"])
def test_all_views_after_layout(case):
    """Workloads whose groups never share a panel with conflicting members:
    after laying out A, B and C every group addresses every operand as one
    view (no segments, and no gathers needed for stride irregularity)."""
    _lib_or_skip()
    con = CASES[case]()
    before, _ = _modes(con)
    for w in "ABC":
        con, _ = _with_layout(con, w)
    after, s = _modes(con, layout="never_pack")
    for op in "ABC":
        assert after[op][2] == 0, (op, before, after)
        assert after[op][0] >= before[op][0]


def test_layout_errors():
    _lib_or_skip()
    con = C.tiny_u1("diag").con
    with pytest.raises(bst.BscError) as e:
        bst.plan_layout(con, "A", align=0)
    assert e.value.name == "BSC_ERR_ARG"
    bad = copy.deepcopy(con)
    bad.A.row_key = np.array(bad.A.row_key).copy()
    bad.A.row_key[0] = 99
    with pytest.raises(bst.BscError) as e:
        bst.plan_layout(bad, "A")
    assert e.value.name == "BSC_ERR_SHAPE"
    bad = copy.deepcopy(con)
    bad.C.offset = np.array(bad.C.offset).copy()
    bad.C.offset[1] = bad.C.offset[0]          # the other operands must be valid
    with pytest.raises(bst.BscError) as e:
        bst.plan_layout(bad, "A")
    assert e.value.name == "BSC_ERR_OVERLAP"
    new, _ = _with_layout(bad, "C")             # the selected operand's own layout is ignored
    _modes(new)


# ---------------------------------------------------------------------------
# chains
# ---------------------------------------------------------------------------

def _chain_stages(ch):
    return [(st.con, st.a_buf, st.b_buf, st.c_buf) for st in ch.stages]


@pytest.mark.parametrize("make", [lambda: C.small_chain(seed=3, layout="natural"),
                                  lambda: C.small_chain(seed=4, layout="coop"),
                                  lambda: C.rabc_u1(layout="natural")], ids=["small_natural", "small_coop", "rabc_u1"])
def test_chain_views_agree(make):
    """Every view of every tensor element, in every stage, reaches one new
    address, distinct elements reach distinct addresses, and every stage plans."""
    _lib_or_skip()
    ch = make()
    st = _chain_stages(ch)
    new, sizes, _ = bst.layouts.relayout_chain(st)
    where = {buf: {} for buf in sizes}          # old address -> new address
    for (old, a, b, c), nc in zip(st, new):
        for which, buf in zip("ABC", (a, b, c)):
            _, _, op = _views_of(old, which)
            for j in range(len(op.row_key)):
                o = _block_addresses(old, which, j).ravel()
                n = _block_addresses(nc, which, j).ravel()
                assert n.min() >= 0 and n.max() < sizes[buf]
                m = where[buf]
                for x, y in zip(o.tolist(), n.tolist()):
                    assert m.setdefault(x, y) == y
    for buf, m in where.items():
        vals = list(m.values())
        assert len(set(vals)) == len(vals), buf
    for nc in new:
        bst.Plan(nc)


def test_chain_relayout_removes_gathers_and_segments():
    """The U(1) update in its natural layout walks per-member pieces in stage
    1 and has several views per group in stage 2; laid out for the readers,
    every group sees its members as one view."""
    _lib_or_skip()
    ch = C.rabc_u1(layout="natural")
    st = _chain_stages(ch)
    new, _, _ = bst.layouts.relayout_chain(st, prefer="reader")
    m0, s0 = _modes(st[0][0])
    m1, s1 = _modes(new[0])
    assert m0["A"][2] > 0 and m1["A"] == (s1["groups"] - s1["zero_groups"], 0, 0)
    # stage 2: in the natural layout many groups' members are several views
    # (gathering them is possible; the calibrated model finds it does not pay);
    # laid out for the readers far fewer are, and nothing is gathered
    before = bst.Plan(st[1][0], layout="force_pack").stats()["pack_bytes"]
    after = bst.Plan(new[1], layout="force_pack").stats()["pack_bytes"]
    assert before > 0 and after < before
    _, s1 = _modes(new[1])
    assert s1["launches_per_contract"] == 1 and s1["pack_bytes"] == 0


def test_move_blocks_round_trip():
    _lib_or_skip()
    ch = C.small_chain(seed=3, layout="natural")
    st = _chain_stages(ch)
    new, _, _ = bst.layouts.relayout_chain(st)
    e = ch.buffers[st[0][1]]
    moved = bst.layouts.move_blocks(e, st[0][0], "A", new[0])
    back = bst.layouts.move_blocks(moved, new[0], "A", st[0][0])
    _, mask = _mask_of(st[0][0], "A")
    assert np.array_equal(back[mask], np.asarray(e)[mask])


def _mask_of(con, which):
    _, _, op = _views_of(con, which)
    mask = np.zeros(op.buffer_elems, bool)
    for j in range(len(op.row_key)):
        mask[_block_addresses(con, which, j).ravel()] = True
    return None, mask


def test_chain_writer_first_outputs_are_views():
    """By default an intermediate is laid out for the stage that writes it:
    every stage's output groups then write single views (the natural layout
    makes stage 1 write per-member pieces), and the inputs are still laid out
    for their readers (stage 1 reads E as single views)."""
    _lib_or_skip()
    ch = C.rabc_u1u1(layout="natural")
    st = _chain_stages(ch)
    new, _, _ = bst.layouts.relayout_chain(st)
    m0, _ = _modes(st[0][0])
    assert m0["C"][2] > 0 and m0["A"][2] > 0
    for i, nc in enumerate(new):
        m, s = _modes(nc, layout="never_pack")
        assert m["C"][2] == 0, (i, m)
    m, s = _modes(new[0])
    assert m["A"][2] == 0


def test_layout_empty_operand_and_no_products():
    """An operand with no blocks gets an empty layout; with no sector products
    the other operands are still laid out (every block in its panel, disjoint)."""
    _lib_or_skip()
    con = copy.deepcopy(C.tiny_u1("diag").con)
    op = con.A
    op.row_key, op.col_key = np.zeros(0, np.int32), np.zeros(0, np.int32)
    op.offset, op.row_stride, op.col_stride = np.zeros(0, np.int64), np.zeros((0, 2), np.int64), np.zeros((0, 2), np.int64)
    off, rs, cs, tot = bst.plan_layout(con, "A")
    assert len(off) == 0 and tot == 0
    new, (off, rs, cs, tot) = _with_layout(con, "C", align=4)
    m, s = _modes(new)
    assert s["triples"] == 0 and s["zero_blocks"] == con.C.nblocks
    seen = np.zeros(tot, bool)
    for j in range(con.C.nblocks):
        a = _block_addresses(new, "C", j).ravel()
        assert not seen[a].any()
        seen[a] = True
