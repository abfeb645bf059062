"""Host-side check of the device work list: decode the image bsc_plan_bind
uploads and replay the kernel's addressing in numpy.  Every address a kernel
would read or write is bounds-checked, every C element inside a view is
written exactly once per launch sequence, and the replayed result matches the
oracle.  This runs the kernels' index arithmetic on the CPU before any GPU run."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

bst = pytest.importorskip("block_sparse_tensor_amd")

DVIEW = np.dtype([("off", "<i8"), ("sa0", "<i8"), ("sa1", "<i8"), ("sb0", "<i8"), ("sb1", "<i8"),
                  ("ia", "<i4"), ("ib", "<i4"), ("begin", "<i4"), ("len", "<i4")])
DGROUP = np.dtype([(n, "<i4") for n in ("M", "N", "K", "nrun", "run0", "ncp", "cp0", "flags")])
DRUN = np.dtype([(n, "<i4") for n in ("K", "nap", "ap0", "nbp", "bp0", "flags", "kbase", "pad")])
DTASK = np.dtype([(n, "<i4") for n in ("cls", "group", "m0", "n0")])
DFAST = np.dtype([(n, "<i8") for n in ("a_base", "a_rs", "a_ks", "b_base", "b_ks", "b_ns", "c_base", "c_rs", "c_cs")] +
                 [(n, "<i4") for n in ("mlen", "nlen", "K", "flags", "group", "split", "nsplit", "counter")] +
                 [("part", "<i8")])
DPACK = np.dtype([(n, "<i8") for n in ("off", "sa0", "sa1", "sb0", "sb1", "dst")] +
                 [(n, "<i4") for n in ("ia", "ib", "rows", "cols", "ld", "src", "dmode", "pad")])
R_A_WS, R_B_WS = 128, 256          # run reads A / B from the pack workspace
F_A_WS, F_B_WS = 4, 8              # dense record reads A / B from the pack workspace
G_C_ALONG_N, G_ACCUMULATE = 1, 2
T_GENERIC, T_MFMA, T_TAIL, T_ZERO = 0, 1, 2, 3
TILE = {T_GENERIC: (64, 64), T_ZERO: (64, 64), T_MFMA: (128, 128), 4: (256, 128), 5: (256, 128),
        12: (256, 256), 13: (256, 256)}
TILE_MFMA_F = (64, 64)   # fp32 / fp64 matrix-core tile

assert DVIEW.itemsize == 56 and DGROUP.itemsize == 32 and DRUN.itemsize == 32 and DTASK.itemsize == 16
assert DFAST.itemsize == 112 and DPACK.itemsize == 80
SPLIT_TILE = 256 * 128   # fp32 elements of one K-slice partial tile of the 256 x 128 tile
T_DENSE_N, T_DENSE_K = 4, 5
T_WIDE_N, T_WIDE_K = 12, 13       # wide tile (one workgroup per CU): 256 x 256, 128 x 64 waves at <= 128 columns
T_DIRECT = (T_DENSE_N, T_DENSE_K, T_WIDE_N, T_WIDE_K)


def split_tile_elems(cls, mlen, nlen, wide_only=False):
    """fp32 elements the kernel strides per K-slice partial tile: the 256 x 128
    tile's (128 x 128 for a tile of at most 128 rows, which runs as four 64 x 64
    waves), a wide tile's 256 x 256 (four waves of 128 x 64 at <= 128 columns:
    256 x 128), and on eight waves (a plan of wide tiles and tail bundles only)
    256 x 256, or 128 x 256 for a tile of at most 128 rows."""
    if cls in (T_WIDE_N, T_WIDE_K):
        if wide_only:
            return (128 if mlen <= 128 else 256) * 256
        return 256 * 256 if nlen > 128 else SPLIT_TILE
    return 128 * 128 if mlen <= 128 else SPLIT_TILE
T_MFMA_DENSE = 9                  # fp32 / fp64 record-addressed matrix-core tile
T_SKINNY_DENSE = (10, 11)         # record-addressed skinny items (long axis M / N)
T_SKINNY_M, T_SKINNY_N = 7, 8    # long axis M (at most 16 columns) / long axis N (at most 16 rows)


def skinny_long(dtype, short):
    """Long-axis extent of a skinny tile: 256 threads x R lines, R x (short
    extent rounded up to 4, 8 or 16) = 32 accumulators."""
    yb = 4 if short <= 4 else (8 if short <= 8 else 16)
    return 256 * (32 // yb)


def decode(plan):
    info, img = plan.worklist()
    tab = lambda dt, n, off: np.frombuffer(img, dtype=dt, count=n, offset=off)
    return (info, tab(DGROUP, info["n_groups"], info["off_groups"]), tab(DRUN, info["n_runs"], info["off_runs"]),
            tab(DVIEW, info["n_apieces"], info["off_apieces"]), tab(DVIEW, info["n_bpieces"], info["off_bpieces"]),
            tab(DVIEW, info["n_cpieces"], info["off_cpieces"]), tab(DTASK, info["n_tasks"], info["off_tasks"]),
            tab(DFAST, info["n_dense"], info["off_dense"]))


def decode_tail(plan):
    info, img = plan.worklist()
    return np.frombuffer(img, dtype=DFAST, count=info["n_tail"], offset=info["off_tail"])


def tail_lanes(mn):
    p = 1
    while 2 * p * mn <= 64:
        p *= 2
    return p


def decode_packs(plan):
    info, img = plan.worklist()
    tab = lambda dt, n, off: np.frombuffer(img, dtype=dt, count=n, offset=off)
    return info, tab(DPACK, info["n_packs"], info["off_packs"]), tab(DTASK, info["n_pack_tasks"], info["off_pack_tasks"])


def pack_piece(d, bf16):
    """The kernel's piece shape (tr rows by tc columns) for a gather: up to
    4096 elements of at most 64 columns; a straight bf16 gather (both sides
    unit-stride along the same axis) takes up to 16384 elements with lines of
    up to 1024 along that axis."""
    s_k = d["ib"] == 1 and (d["sb0"] == 1 or d["cols"] == 1)
    s_f = d["ia"] == 1 and (d["sa0"] == 1 or d["rows"] == 1)
    mode = (1 if s_k else 0) if d["dmode"] == 0 else (2 if s_f else 0)
    tc = 1
    if bf16 and mode == 1:
        while tc < d["cols"] and tc < 1024:
            tc *= 2
        return 16384 // tc, tc
    if bf16 and mode == 2:
        lr = 1
        while lr < d["rows"] and lr < 1024:
            lr *= 2
        while tc < d["cols"] and tc * lr < 16384:
            tc *= 2
        return min(16384 // tc, 4096), tc
    while tc < d["cols"] and tc < 64:
        tc *= 2
    return min(4096 // tc, 1024), tc


def replay_packs(plan, con, a64, b64):
    """The gather launch: every pack task copies its 64 x 64 piece of a gather
    from A or B into the workspace.  Every workspace element is written at most
    once; returns the workspace and the mask of written elements."""
    info, packs, ptasks = decode_packs(plan)
    ws = np.full(info["workspace_elems"], np.nan)
    hit = np.zeros(info["workspace_elems"], np.int64)
    bf16 = plan.stats()["dtype"] == 2
    for t in ptasks:
        d = packs[t["group"]]
        tr, tc = pack_piece(d, bf16)
        assert t["m0"] % tr == 0 and t["n0"] % tc == 0
        x = np.arange(t["m0"], min(t["m0"] + tr, d["rows"]))
        y = np.arange(t["n0"], min(t["n0"] + tc, d["cols"]))
        assert len(x) and len(y)
        src = d["off"] + (x[:, None] // d["ia"]) * d["sa0"] + (x[:, None] % d["ia"]) * d["sa1"] + \
            (y[None, :] // d["ib"]) * d["sb0"] + (y[None, :] % d["ib"]) * d["sb1"]
        buf = a64 if d["src"] == 0 else b64
        assert src.min() >= 0 and src.max() < buf.size
        if d["dmode"] == 0:
            dst = d["dst"] + x[:, None] * d["ld"] + y[None, :]
        else:
            dst = d["dst"] + y[None, :] * d["ld"] + x[:, None]
        assert dst.min() >= 0 and dst.max() < ws.size
        ws[dst] = buf[src]
        np.add.at(hit, dst.ravel(), 1)
    assert hit.max(initial=0) <= 1, "a workspace element is gathered twice"
    return ws, hit > 0


def rec_addr(pieces, x, y):
    """Address of element (x along the piece axis, y along the other) for arrays x, y."""
    begins = pieces["begin"]
    p = np.searchsorted(begins, x, side="right") - 1
    v = pieces[p]
    xl = x - v["begin"]
    assert np.all(xl >= 0) and np.all(xl < v["len"]), "row/column outside its piece"
    base = v["off"] + (xl // v["ia"]) * v["sa0"] + (xl % v["ia"]) * v["sa1"]
    return base[:, None] + (y[None, :] // v["ib"][:, None]) * v["sb0"][:, None] + \
        (y[None, :] % v["ib"][:, None]) * v["sb1"][:, None]


def replay(plan, con, a, b, c0, accumulate=False):
    info, groups, runs, ap, bp, cp, tasks, dense = decode(plan)
    c = np.array(c0, dtype=np.float64)
    written = np.zeros(c.size, np.int64)
    a64, b64 = np.asarray(a, np.float64), np.asarray(b, np.float64)
    ws, ws_written = replay_packs(plan, con, a64, b64)
    splits = {}   # K-split tiles by counter: the partials of their slices
    # a plan of wide tiles, tail bundles and no-ops (at least one wide tile)
    wide_only = plan.stats()["wide_only"] == 1
    assert wide_only == (bool(np.isin(tasks["cls"], (T_WIDE_N, T_WIDE_K)).any()) and
                         bool(np.isin(tasks["cls"], (T_WIDE_N, T_WIDE_K, T_TAIL, 6)).all()))
    tail = decode_tail(plan)
    # a tail bundle: entries group .. group + m0 - 1 of the tail table, one whole group per wave
    expanded = []
    for t in tasks:
        if t["cls"] == T_TAIL:
            assert 1 <= t["m0"] <= 4 and 0 <= t["group"] and t["group"] + t["m0"] <= len(tail)
            for e in range(int(t["group"]), int(t["group"] + t["m0"])):
                f = tail[e]
                mn = int(f["mlen"]) * int(f["nlen"])
                lanes = tail_lanes(mn)
                assert mn <= 256 and f["K"] <= 512 and f["mlen"] + f["nlen"] <= 1024
                assert -(-mn // (64 // lanes)) * -(-int(f["K"]) // lanes) <= 64, "tail lane work"
                # record-addressed tail group: bases and strides, the whole group at once
                assert f["nsplit"] == 1 and 2 * mn * int(f["K"]) <= 1024
                g = groups[f["group"]]
                assert g["M"] == f["mlen"] and g["N"] == f["nlen"] and g["K"] == f["K"] and g["nrun"] == 1
                expanded.append(("tail_dense", f))
        else:
            expanded.append(t)
    for t in expanded:
        if isinstance(t, tuple):
            f = t[1]
            i = np.arange(f["mlen"])[:, None]
            j = np.arange(f["nlen"])[None, :]
            k = np.arange(f["K"])
            aad = f["a_base"] + i * f["a_rs"] + k[None, :] * f["a_ks"]
            bad = f["b_base"] + k[:, None] * f["b_ks"] + j * f["b_ns"]
            cad = f["c_base"] + i * f["c_rs"] + j * f["c_cs"]
            abuf = ws if f["flags"] & F_A_WS else a64
            bbuf = ws if f["flags"] & F_B_WS else b64
            for ad, n in ((aad, abuf.size), (bad, bbuf.size), (cad, con.C.buffer_elems)):
                assert ad.min() >= 0 and ad.max() < n
            acc = abuf[aad] @ bbuf[bad]
            if f["flags"] & G_ACCUMULATE:
                acc = acc + c[cad]
            c[cad] = acc
            np.add.at(written, cad.ravel(), 1)
            continue
        if t["cls"] == 6:      # no-op placeholder
            continue
        if t["cls"] in T_DIRECT + (T_MFMA_DENSE,) + T_SKINNY_DENSE:
            # dense tile: bases and strides only (the kernel's addressing)
            f = dense[t["group"]]
            i = np.arange(f["mlen"])[:, None]
            j = np.arange(f["nlen"])[None, :]
            k = np.arange(f["K"])
            if t["cls"] in (T_DENSE_N, T_WIDE_N):
                assert f["b_ns"] == 1 or f["nlen"] == 1
            if t["cls"] in T_DIRECT:
                assert f["a_ks"] == 1 or f["K"] == 1
                tm, tn = TILE[int(t["cls"])]
                assert 1 <= f["mlen"] <= tm and 1 <= f["nlen"] <= tn
            if t["cls"] in (T_DENSE_K, T_WIDE_K):
                assert f["b_ks"] == 1 or f["K"] == 1
            aad = f["a_base"] + i * f["a_rs"] + k[None, :] * f["a_ks"]
            bad = f["b_base"] + k[:, None] * f["b_ks"] + j * f["b_ns"]
            cad = f["c_base"] + i * f["c_rs"] + j * f["c_cs"]
            abuf = ws if f["flags"] & F_A_WS else a64
            bbuf = ws if f["flags"] & F_B_WS else b64
            for ad, n in ((aad, abuf.size), (bad, bbuf.size), (cad, con.C.buffer_elems)):
                assert ad.min() >= 0 and ad.max() < n
            for ad, flag in ((aad, F_A_WS), (bad, F_B_WS)):
                if f["flags"] & flag:
                    assert ws_written[ad].all(), "a tile reads a workspace element no gather wrote"
            acc = abuf[aad] @ bbuf[bad]
            if f["nsplit"] > 1:
                # K-slice of a split tile: its partial waits for the other slices
                assert t["cls"] in T_DIRECT and 0 <= f["split"] < f["nsplit"]
                assert 0 <= f["counter"] < info["n_counters"]
                pt = split_tile_elems(int(t["cls"]), int(f["mlen"]), int(f["nlen"]), wide_only)
                assert 0 <= f["part"] and f["part"] + f["nsplit"] * pt <= info["partial_elems"]
                slot = splits.setdefault(int(f["counter"]), {"n": int(f["nsplit"]), "part": int(f["part"]),
                                                             "cad": cad, "f": f, "p": {}, "pt": pt})
                assert slot["n"] == f["nsplit"] and slot["part"] == f["part"] and np.array_equal(slot["cad"], cad)
                assert int(f["split"]) not in slot["p"], "a K-slice appears twice"
                slot["p"][int(f["split"])] = (acc, aad[0, :], int(f["K"]))
                continue
            if f["flags"] & G_ACCUMULATE:
                acc = acc + c[cad]
            c[cad] = acc
            np.add.at(written, cad.ravel(), 1)
            continue
        g = groups[t["group"]]
        if t["cls"] == T_TAIL:
            TM, TN = int(g["M"]), int(g["N"])
        elif t["cls"] == T_SKINNY_M:
            TM, TN = skinny_long(con.dtype, int(g["N"])), max(1, int(g["N"]))
        elif t["cls"] == T_SKINNY_N:
            TM, TN = max(1, int(g["M"])), skinny_long(con.dtype, int(g["M"]))
        else:
            TM, TN = TILE_MFMA_F if (t["cls"] == T_MFMA and con.dtype != "bf16") else TILE[int(t["cls"])]
        m0, n0 = int(t["m0"]), int(t["n0"])
        assert 0 <= m0 < g["M"] and 0 <= n0 < g["N"]
        rows = np.arange(m0, min(m0 + TM, g["M"]))
        cols = np.arange(n0, min(n0 + TN, g["N"]))
        acc = np.zeros((len(rows), len(cols)))
        kseen = 0
        for r in range(g["nrun"]):
            run = runs[g["run0"] + r]
            assert run["kbase"] == kseen
            kseen += run["K"]
            ks = np.arange(run["K"])
            aad = rec_addr(ap[run["ap0"]:run["ap0"] + run["nap"]], rows, ks)
            bad = rec_addr(bp[run["bp0"]:run["bp0"] + run["nbp"]], cols, ks)
            abuf = ws if run["flags"] & R_A_WS else a64
            bbuf = ws if run["flags"] & R_B_WS else b64
            assert aad.min(initial=0) >= 0 and aad.max(initial=-1) < abuf.size
            assert bad.min(initial=0) >= 0 and bad.max(initial=-1) < bbuf.size
            for ad, flag in ((aad, R_A_WS), (bad, R_B_WS)):
                if run["flags"] & flag:
                    assert ws_written[ad].all(), "a tile reads a workspace element no gather wrote"
            acc += abuf[aad] @ bbuf[bad].T
        assert kseen == g["K"]
        cps = cp[g["cp0"]:g["cp0"] + g["ncp"]]
        if g["flags"] & G_C_ALONG_N:
            cad = rec_addr(cps, cols, rows).T
        else:
            cad = rec_addr(cps, rows, cols)
        assert cad.min() >= 0 and cad.max() < con.C.buffer_elems
        if g["flags"] & G_ACCUMULATE:
            acc = acc + c[cad]
        c[cad] = acc
        np.add.at(written, cad.ravel(), 1)
    # K-split tiles: every slice once, slices cover consecutive K ranges, the
    # partials summed in slice order
    parts_used = np.zeros(info["partial_elems"], np.int64)
    for slot in splits.values():
        n, f = slot["n"], slot["f"]
        assert sorted(slot["p"]) == list(range(n)), "a K-slice is missing"
        krow = np.concatenate([slot["p"][s][1] for s in range(n)])   # A addresses along k of the first row
        assert len(krow) == len(np.unique(krow)) and np.all(np.diff(krow) == f["a_ks"])
        assert all(slot["p"][s][2] % 32 == 0 for s in range(n - 1)), "only the last slice may end in a partial chunk"
        parts_used[slot["part"]:slot["part"] + n * slot["pt"]] += 1
        acc = slot["p"][0][0]
        for s in range(1, n):
            acc = acc + slot["p"][s][0]
        cad = slot["cad"]
        if f["flags"] & G_ACCUMULATE:
            acc = acc + c[cad]
        c[cad] = acc
        np.add.at(written, cad.ravel(), 1)
    assert parts_used.max(initial=0) <= 1, "two split tiles share partial storage"
    return c, written


CASES = [("tiny_u1", lambda: C.tiny_u1().con, lambda: C.tiny_u1()),
         ("tiny_u1-flux1", None, lambda: C.tiny_u1("flux1")),
         ("tiny_u1-3leg", None, lambda: C.tiny_u1("flux1_3leg")),
         ("ragged_batch", None, lambda: C.ragged_batch())]


@pytest.mark.parametrize("axis", ["auto", "free_m", "free_n", "contract"])
@pytest.mark.parametrize("name", ["tiny_u1", "tiny_u1-flux1", "tiny_u1-3leg", "ragged_batch"])
def test_replay_configs(name, axis):
    prob = dict((n, f) for n, _, f in CASES)[name]()
    _check(prob.con, prob.a, prob.b, axis)


@pytest.mark.parametrize("seed", range(16))
@pytest.mark.parametrize("axis", ["auto", "free_m", "free_n", "contract", "per_sector"])
def test_replay_random(seed, axis):
    prob = C.random_problem(5000 + seed, nq=1 + seed % 2, nkeys=(6, 6, 6), maxdim=12, qrange=1,
                            flux=[(0, 0), (1, -1), (1, 0)][seed % 3], density=0.8)
    _check(prob.con, prob.a, prob.b, axis)


@pytest.mark.parametrize("layout", ["coop", "natural"])
@pytest.mark.parametrize("axis", ["auto", "free_m", "free_n", "contract"])
def test_replay_small_chain(layout, axis):
    ch = C.small_chain(seed=4, layout=layout)
    bufs = {k: np.asarray(v, np.float64) for k, v in ch.buffers.items()}
    ref = oracle.run_chain(ch)
    for st in ch.stages:
        c0 = np.zeros(ch.sizes[st.c_buf])
        plan = bst.Plan(st.con, axis=axis)
        got, written = replay(plan, st.con, bufs[st.a_buf], bufs[st.b_buf], c0)
        np.testing.assert_allclose(got, ref[st.c_buf], rtol=1e-12, atol=1e-12)
        bufs[st.c_buf] = got


def test_replay_rabc_u1_stages():
    ch = C.rabc_u1()
    bufs = {k: np.asarray(v, np.float64) for k, v in ch.buffers.items()}
    ref = oracle.run_chain(ch)
    for st in ch.stages:
        plan = bst.Plan(st.con)
        got, written = replay(plan, st.con, bufs[st.a_buf], bufs[st.b_buf], np.zeros(ch.sizes[st.c_buf]))
        err = np.linalg.norm(got - ref[st.c_buf]) / np.linalg.norm(ref[st.c_buf])
        assert err < 1e-13
        bufs[st.c_buf] = got


def _check(con, a, b, axis):
    kw = dict(launch_mode="per_sector") if axis == "per_sector" else dict(axis=axis)
    plan = bst.Plan(con, **kw)
    c0 = np.full(con.C.buffer_elems, -3.5)
    got, written = replay(plan, con, a, b, c0)
    ref = oracle.contract(con, a, b, c0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    in_view = np.zeros(con.C.buffer_elems, bool)
    from gpuhelp import c_addresses
    addr, in_view = c_addresses(con)
    assert np.all(written[~in_view] == 0)
    if axis != "per_sector":
        assert np.all(written[in_view] == 1)   # one owner per C element
    else:
        assert np.all(written[in_view] >= 1)


@pytest.mark.parametrize("la", [1, 8])
def test_replay_bf16_dense_tiles(la):
    """bf16 block-diagonal structures: aligned layouts take the dense tile records."""
    prob = C.blockdiag_bf16(ld_align=la, align=la)
    # replay a subset of the sectors to keep it quick: rebuild with the first 12 keys
    import copy
    con = prob.con
    plan = bst.Plan(con)
    s = plan.stats()
    if la == 8:
        assert s["items_by_class"]["mfma_fast"] > 0
    got, written = replay(plan, con, prob.a, prob.b, np.zeros(con.C.buffer_elems))
    ref = oracle.contract(con, prob.a, prob.b, np.zeros(con.C.buffer_elems), check=False)
    assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


@pytest.mark.parametrize("seed", range(6))
def test_replay_dense_random(seed):
    """Aligned random single-view groups (both B orientations, accumulate too)."""
    from workloads.layout import write_block
    from workloads.model import Contraction, Index, Operand
    rng = np.random.default_rng(seed)
    M, K, N = (int(x) for x in rng.integers(40, 300, 3))
    lda, ldb = (K + 7) // 8 * 8, (N + 7) // 8 * 8
    brow = seed % 2 == 0
    A = rng.standard_normal((M, K)); B = rng.standard_normal((K, N))
    abuf = np.zeros(M * lda + 16); bbuf = np.zeros(K * ldb + N * ldb + 16)
    write_block(abuf, 8, (lda, 0), (1, 0), A)
    if brow:
        write_block(bbuf, 8, (ldb, 0), (1, 0), B); brs, bcs = (ldb, 0), (1, 0)
    else:
        ldk = (K + 7) // 8 * 8
        write_block(bbuf, 8, (1, 0), (ldk, 0), B); brs, bcs = (1, 0), (ldk, 0)
    idx = lambda d: Index([[0]], [d])
    con = Contraction(idx(M), idx(K), idx(N), Operand([0], [0], [8], [(lda, 0)], [(1, 0)], [0], abuf.size),
                      Operand([0], [0], [8], [brs], [bcs], [0], bbuf.size),
                      Operand([0], [0], [5], [(N + 3, 0)], [(1, 0)], [0], 5 + M * (N + 3)), "bf16")
    for acc in (False, True):
        plan = bst.Plan(con, accumulate=acc)
        assert plan.stats()["items_by_class"]["mfma_fast"] > 0
        c0 = np.full(con.C.buffer_elems, 0.5)
        got, written = replay(plan, con, abuf, bbuf, c0)
        ref = oracle.contract(con, abuf, bbuf, c0, accumulate=acc)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def _dense_con(M, K, N, brow):
    """One aligned bf16 GEMM block: A row-major, B row- or column-major."""
    from workloads.model import Contraction, Index, Operand
    lda, ldb, ldk = (K + 7) // 8 * 8, (N + 7) // 8 * 8, (K + 7) // 8 * 8
    brs, bcs = ((ldb, 0), (1, 0)) if brow else ((1, 0), (ldk, 0))
    na, nb = M * lda + 16, K * ldb + N * ldb + 16
    idx = lambda d: Index([[0]], [d])
    return Contraction(idx(M), idx(K), idx(N), Operand([0], [0], [8], [(lda, 0)], [(1, 0)], [0], na),
                       Operand([0], [0], [8], [brs], [bcs], [0], nb),
                       Operand([0], [0], [5], [(N + 3, 0)], [(1, 0)], [0], 5 + M * (N + 3)), "bf16")


def _dense_single(seed, M, K, N, brow):
    from workloads.layout import write_block
    rng = np.random.default_rng(seed)
    con = _dense_con(M, K, N, brow)
    A = rng.standard_normal((M, K)); B = rng.standard_normal((K, N))
    abuf, bbuf = np.zeros(con.A.buffer_elems), np.zeros(con.B.buffer_elems)
    write_block(abuf, 8, con.A.row_stride[0], con.A.col_stride[0], A)
    write_block(bbuf, 8, con.B.row_stride[0], con.B.col_stride[0], B)
    return con, abuf, bbuf


@pytest.mark.parametrize("split_k", [1, 2, 3, 5])
@pytest.mark.parametrize("brow", [True, False])
def test_replay_split_k(split_k, brow):
    """K-split tiles: slices cover K in order, every slice once, partial
    storage disjoint, and the summed partials give the oracle's result (also
    when accumulating)."""
    con, abuf, bbuf = _dense_single(40 + split_k, 300, 333, 150, brow)
    for acc in (False, True):
        plan = bst.Plan(con, accumulate=acc, split_k=split_k)
        s = plan.stats()
        tiles = 2 * 2   # 256 x 128 tiles over 300 x 150
        assert s["split_tiles"] == tiles and s["items_by_class"]["mfma_fast"] == tiles * -(-11 // split_k)
        info, *_ = decode(plan)
        assert info["n_counters"] == tiles and info["partial_elems"] == tiles * -(-11 // split_k) * SPLIT_TILE
        assert plan.device_bytes() >= info["off_partials"] + 4 * info["partial_elems"]
        c0 = np.full(con.C.buffer_elems, 0.5)
        got, written = replay(plan, con, abuf, bbuf, c0, accumulate=acc)
        ref = oracle.contract(con, abuf, bbuf, c0, accumulate=acc)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
        assert written.max() == 1


def test_half_row_tiles_policy():
    """With at most one 256 x 128 tile per CU, direct-to-LDS groups whose K
    chain is long (>= 16 chunks of 32) and above 1.5x one slot's share of the
    plan's work get 128-row tiles."""
    # 1024^3: 32 chunks, share 32 * 32 / 512 = 2 -> 8 x 8 tiles of 128 x 128
    assert bst.Plan(_dense_con(1024, 1024, 1024, True)).stats()["items_by_class"]["mfma_fast"] == 64
    # the block-diagonal bf16 workload has 362 tiles of 256 x 128 (more than the CUs): none halved
    prob = C.blockdiag_bf16(ld_align=8, align=8, values=False)
    assert bst.Plan(prob.con).stats()["items_by_class"]["mfma_fast"] == \
        bst.Plan(prob.con, tile_rows=256).stats()["items_by_class"]["mfma_fast"]
    # 4096^3: share 128 chunks = the chain -> 256-row tiles
    assert bst.Plan(_dense_con(4096, 4096, 4096, True)).stats()["items_by_class"]["mfma_fast"] == 512
    # K = 480 (15 chunks): never
    assert bst.Plan(_dense_con(1024, 480, 1024, True)).stats()["items_by_class"]["mfma_fast"] == 32
    # per-sector launches keep 256-row tiles
    s = bst.Plan(_dense_con(1024, 1024, 1024, True), launch_mode="per_sector").stats()
    assert s["items_by_class"]["mfma_fast"] == 32
    # forced heights
    assert bst.Plan(_dense_con(1024, 1024, 1024, True), tile_rows=256).stats()["items_by_class"]["mfma_fast"] == 32
    assert bst.Plan(_dense_con(1024, 480, 1024, True), tile_rows=128).stats()["items_by_class"]["mfma_fast"] == 64
    with pytest.raises(bst.BscError):
        bst.Plan(_dense_con(64, 64, 64, True), tile_rows=64)


def test_split_k_policy():
    """Automatic K split: only tiles whose K chain is far above both 64 chunks
    and one slot's share of the plan's work; never in per-sector mode, with
    split_k=-1, or for fp32."""
    prob = C.blockdiag_bf16(ld_align=8, align=8, values=False)
    assert bst.Plan(prob.con).stats()["split_tiles"] == 0          # K <= 1024
    assert bst.Plan(prob.con, split_k=8).stats()["split_tiles"] > 0
    assert bst.Plan(prob.con, split_k=8, launch_mode="per_sector").stats()["split_tiles"] == 0
    for shape in ((4096, 4096, 4096), (2048, 2048, 2048), (1024, 1024, 1024)):
        assert bst.Plan(_dense_con(*shape, True)).stats()["split_tiles"] == 0
    # 256 x 32768 x 128 (1024 chunks): two 128-row tiles (long chain), each
    # cut into slices of 64 chunks
    con = _dense_con(256, 32768, 128, True)
    s = bst.Plan(con).stats()
    assert s["split_tiles"] == 2 and s["items_by_class"]["mfma_fast"] == 2 * 16
    s = bst.Plan(con, split_k=-1).stats()
    assert s["split_tiles"] == 0 and s["items_by_class"]["mfma_fast"] == 2
    assert bst.Plan(con, split_k=100).stats()["items_by_class"]["mfma_fast"] == 2 * 11
    # fp32 tiles are never split
    con32 = _dense_con(256, 32768, 128, True)
    con32.dtype = "f32"
    assert bst.Plan(con32, split_k=4).stats()["split_tiles"] == 0
    with pytest.raises(bst.BscError):
        bst.Plan(con, split_k=-2)


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("axis", ["free_m", "free_n", "contract"])
def test_replay_force_pack_random(seed, axis):
    """Every scattered operand gathered into the workspace: the gathers cover
    exactly what the tiles read, and the result is the oracle's."""
    prob = C.random_problem(7000 + seed, nq=1 + seed % 2, nkeys=(6, 6, 6), maxdim=12, qrange=1,
                            flux=[(0, 0), (1, -1), (1, 0)][seed % 3], density=0.8)
    plan = bst.Plan(prob.con, axis=axis, layout="force_pack")
    c0 = np.full(prob.con.C.buffer_elems, -3.5)
    got, written = replay(plan, prob.con, prob.a, prob.b, c0)
    ref = oracle.contract(prob.con, prob.a, prob.b, c0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    s = plan.stats()
    modes = s["mode_count"]
    assert modes["A"]["segments"] == 0 and modes["B"]["segments"] == 0
    if modes["A"]["pack"] + modes["B"]["pack"]:
        assert s["launches_per_contract"] == 2 and s["pack_bytes"] > 0


@pytest.mark.parametrize("layout", ["force_pack", "auto"])
def test_replay_pack_natural_chain(layout):
    """The natural-layout environment update with gathers, stage by stage."""
    ch = C.small_chain(seed=4, layout="natural")
    bufs = {k: np.asarray(v, np.float64) for k, v in ch.buffers.items()}
    ref = oracle.run_chain(ch)
    for st in ch.stages:
        plan = bst.Plan(st.con, layout=layout)
        got, written = replay(plan, st.con, bufs[st.a_buf], bufs[st.b_buf], np.zeros(ch.sizes[st.c_buf]))
        np.testing.assert_allclose(got, ref[st.c_buf], rtol=1e-12, atol=1e-12)
        bufs[st.c_buf] = got


def _wide_tasks(plan):
    _, _, _, _, _, _, tasks, _ = decode(plan)
    return tasks[np.isin(tasks["cls"], (T_WIDE_N, T_WIDE_K))]


@pytest.mark.parametrize("la", [8])
def test_replay_bf16_wide_tiles(la):
    """The bf16 block-diagonal workload on the wide tile (tile_cols=256): every
    direct-to-LDS group takes wide tiles of at most 256 x 256, replayed exactly."""
    prob = C.blockdiag_bf16(ld_align=la, align=la)
    con = prob.con
    plan = bst.Plan(con, tile_cols=256)
    wt = _wide_tasks(plan)
    assert len(wt) > 0 and plan.stats()["launches_per_contract"] == 1
    got, written = replay(plan, con, prob.a, prob.b, np.zeros(con.C.buffer_elems))
    ref = oracle.contract(con, prob.a, prob.b, np.zeros(con.C.buffer_elems), check=False)
    assert np.linalg.norm(got - ref) <= 1e-12 * np.linalg.norm(ref)


@pytest.mark.parametrize("shape", [(256, 1024, 256), (300, 600, 200), (100, 640, 152), (520, 1000, 260),
                                   (64, 1030, 70), (33, 40, 24), (257, 96, 257)])
@pytest.mark.parametrize("brow", [True, False])
@pytest.mark.parametrize("split_k", [-1, 3])
def test_replay_wide_single(shape, brow, split_k):
    """Single aligned GEMM blocks on the wide tile, both B orientations, with
    and without K-slices (partials strided by the kernel's tile size)."""
    M, K, N = shape
    con, a, b = _dense_single(11 + M + N, M, K, N, brow)
    plan = bst.Plan(con, tile_cols=256, split_k=split_k)
    wt = _wide_tasks(plan)
    assert len(wt) == plan.stats()["items"]
    if split_k > 0 and K > 3 * 32:
        assert plan.stats()["split_tiles"] > 0
    c0 = np.full(con.C.buffer_elems, 0.5)
    got, written = replay(plan, con, a, b, c0)
    ref = oracle.contract(con, a, b, c0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_wide_only_plans():
    """Plans of wide tiles, tail bundles and no-ops say so (their launch runs
    eight-wave workgroups); a wide plan with other tiles, and every plan on the
    256 x 128 tile, does not."""
    con, _, _ = _dense_single(3, 1024, 1024, 1024, True)
    assert bst.Plan(con, tile_cols=256).stats()["wide_only"] == 1
    assert bst.Plan(con, tile_cols=256, split_k=3).stats()["wide_only"] == 1
    assert bst.Plan(con).stats()["wide_only"] == 0
    prob = C.blockdiag_bf16(ld_align=8, align=8, values=False)
    assert bst.Plan(prob.con, tile_cols=256).stats()["wide_only"] == 1   # wide tiles and tail bundles
    assert bst.Plan(prob.con).stats()["wide_only"] == 0
    prob = C.blockdiag_bf16(values=False)                                 # unpadded: four general tiles too
    assert bst.Plan(prob.con, tile_cols=256).stats()["wide_only"] == 0


def test_wide_half_rows_policy():
    """Wide plans cut the groups whose K chain is far above one CU's share
    into 128-row wide tiles: on the bf16 block-diagonal workload only the
    1024^3 sector (32 tiles of 128 x 256); tile_rows forces either height."""
    prob = C.blockdiag_bf16(ld_align=8, align=8, values=False)
    _, _, _, _, _, _, tk, fa = decode(bst.Plan(prob.con, tile_cols=256))
    w = [t for t in range(len(tk)) if tk[t]["cls"] in (T_WIDE_N, T_WIDE_K)]
    cut = [t for t in w if fa[t]["K"] == 1024]
    assert len(cut) == 32 and all(fa[t]["mlen"] == 128 for t in cut)
    assert all(fa[t]["mlen"] > 128 or fa[t]["K"] < 1024 for t in w if t not in cut)
    _, _, _, _, _, _, tk2, fa2 = decode(bst.Plan(prob.con, tile_cols=256, tile_rows=256))
    assert all(fa2[t]["mlen"] > 128 for t in range(len(tk2)) if tk2[t]["cls"] in (T_WIDE_N, T_WIDE_K)
               and fa2[t]["K"] == 1024)


def test_tile_cols_option_checked():
    with pytest.raises(bst.BscError):
        bst.Plan(_dense_con(64, 64, 64, True), tile_cols=192)


@pytest.mark.parametrize("name", ["ragged_batch", "tiny_u1", "small_chain"])
def test_tail_bundles_cover_tiny_groups(name):
    """Tiny groups go to tail bundles (one group per wave, at most four per
    bundle), every one of them exactly once, and the replay matches the oracle."""
    if name == "small_chain":
        ch = C.small_chain(seed=3, layout="natural")
        cases = [(st.con, None) for st in ch.stages]
        bufs = oracle.run_chain(ch)
        cases = [(st.con, (bufs[st.a_buf], bufs[st.b_buf])) for st in ch.stages]
    else:
        prob = C.ragged_batch() if name == "ragged_batch" else C.tiny_u1()
        cases = [(prob.con, (prob.a, prob.b))]
    seen = 0
    for con, (a, b) in cases:
        plan = bst.Plan(con)
        tasks = decode(plan)[6]
        tail = decode_tail(plan)
        n_bundles = int(np.sum(tasks["cls"] == T_TAIL))
        assert plan.stats()["items_by_class"]["tail"] == n_bundles
        assert len(tail) == len(np.unique(tail["group"])), "a group in two bundles"
        seen += len(tail)
        got, written = replay(plan, con, a, b, np.zeros(con.C.buffer_elems))
        ref = oracle.contract(con, a, b, np.zeros(con.C.buffer_elems), check=False)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    assert seen > 0


def test_chiplet_placement():
    """Task t runs on chiplet t % 8.  A group of at most 32 tiles (one per CU of
    a chiplet) costing at most twice a chiplet's share stays on one chiplet; a
    larger group is cut over several.  The 32 tiles of the bf16 block-diagonal
    workload's 1024^3 sector share one chiplet and run without a CU partner."""
    prob = C.blockdiag_bf16(ld_align=8, align=8, values=False)
    info, groups, runs, ap, bp, cp, tasks, fast = decode(bst.Plan(prob.con))
    direct = [t for t in range(len(tasks)) if tasks[t]["cls"] in (T_DENSE_N, T_DENSE_K)]
    by_group = {}
    for t in direct:
        by_group.setdefault(int(fast[t]["group"]), []).append(t)
    assert max(len(v) for v in by_group.values()) == 32
    for g, ts in by_group.items():
        if len(ts) <= 32:
            assert len({t % 8 for t in ts}) == 1, g
    big = [t for t in direct if fast[t]["K"] == 1024]
    assert len(big) == 32 and len({t % 8 for t in big}) == 1
    # slot d of a chiplet's queue is task 8 d + x; slots d and d + 32 share a CU
    for t in big:
        d = t // 8
        assert d < 32
        partner = t + 8 * 32
        assert partner >= len(tasks) or tasks[partner]["cls"] == 6   # T_NOP
    # 4096^3: 512 tiles over all eight chiplets
    _, _, _, _, _, _, tk, _ = decode(bst.Plan(_dense_con(4096, 4096, 4096, True)))
    cl = [t % 8 for t in range(len(tk)) if tk[t]["cls"] in T_DIRECT]
    assert len(cl) == 512 and set(cl) == set(range(8))
