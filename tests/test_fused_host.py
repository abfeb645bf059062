"""Host checks of the fused two-stage plan (bsc_fused_*): planning, its
statistics and error paths, and a host replay of its device work list.

The replay decodes the image bsc_fused_bind would upload (bsc_fused_worklist)
and evaluates it as the kernel does: every 16 x 16 tile of a group, every
product A_p B_p of the group in order, summed per stage-1 block and the block
weighted by its W entries into the outputs it feeds.  With integer-valued
operands every summation order is exact, so the replayed T2 must equal the
oracle's two-stage result bit for bit; a planner mistake (a product fed to the
wrong output, a wrong weight index, a tile missed or written twice, a
transposed view) changes it."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import c_addresses

bst = pytest.importorskip("block_sparse_tensor_amd")

GROUP = np.dtype([("M", "<i4"), ("N", "<i4"), ("nchan", "<i4"), ("chan0", "<i4"), ("nout", "<i4"),
                  ("out0", "<i4"), ("wbase", "<i4"), ("flags", "<i4"), ("nblk", "<i4"), ("pad0", "<i4"),
                  ("pad1", "<i4"), ("pad2", "<i4")])
CHAN = np.dtype([("a_off", "<i8"), ("a_rs", "<i8"), ("a_ks", "<i8"), ("b_off", "<i8"), ("b_ks", "<i8"),
                 ("b_ns", "<i8"), ("K", "<i4"), ("wrow", "<i2"), ("last", "<i2")])
OUT = np.dtype([("c_off", "<i8"), ("c_rs", "<i8"), ("c_cs", "<i8")])
TASK = np.dtype([("group", "<i4"), ("i0", "<i4"), ("j0", "<i4"), ("oc", "<i4")])
PART = np.dtype([(n, "<i4") for n in ("i0", "j0", "ml", "nl", "M", "N", "nchan", "chan0", "no", "out0", "wbase",
                                      "wstride", "nblk", "flags", "part", "nparts")] + [("first", CHAN), ("npass", "<i4"),
                                                                                       ("reduce", "<i4")])
TILE = 16
G_ACCUMULATE = 2


def _lib_ok():
    try:
        bst._capi.lib()
        return True
    except Exception:
        return False


pytestmark = pytest.mark.skipif(not _lib_ok(), reason="libbsc.so not built")


def decode(fp):
    s, img = fp.worklist()
    assert PART.itemsize == 128 and GROUP.itemsize == 48 and CHAN.itemsize == 56
    arr = lambda off, dt, n: np.frombuffer(img, dt, count=n, offset=off)
    return (s, arr(s["off_groups"], GROUP, s["groups"]), arr(s["off_chans"], CHAN, s["channels"]),
            arr(s["off_outs"], OUT, s["outputs"]), arr(s["off_widx"], np.int32, (s["off_tasks"] - s["off_widx"]) // 4),
            arr(s["off_tasks"], TASK, s["items"]), arr(s["off_parts"], PART, s["n_parts"]),
            arr(s["off_pchans"], CHAN, s["n_pchans"]))


def replay(fp, A1, B1, W, C2):
    """Evaluate the fused work list on the host (float64) from the per-wave
    part records the kernel reads, workgroup by workgroup as the kernel does;
    C2 is updated in place.  Also checks the records against the tasks and
    groups, and that the tasks cover every tile and output chunk once."""
    s, groups, chans, outs, widx, tasks, parts, pchans = decode(fp)
    NO = s["outs_per_task"]
    assert NO in (1, 4, 8, 16) and len(parts) % 4 == 0
    assert s["tile_blocks"] in (1, 2)
    TILE = 16 * s["tile_blocks"]
    assert s["groups"] == 0 or max(int(g["nblk"]) for g in groups) * NO <= 256

    def part_sum(pr):
        """The part's products in order, each finished stage-1 block weighted
        into the task's outputs (list over the outputs) and its block rows."""
        ii = np.arange(pr["i0"], pr["i0"] + pr["ml"])[:, None]
        jj = np.arange(pr["j0"], pr["j0"] + pr["nl"])[None, :]
        acc = [np.zeros((ii.shape[0], jj.shape[1])) for _ in range(int(pr["no"]))]
        t1 = np.zeros((ii.shape[0], jj.shape[1]))
        rows = []
        for c in range(int(pr["nchan"])):
            ch = pr["first"] if c == 0 else pchans[int(pr["chan0"]) + c]
            if c == 0:
                assert ch == pchans[int(pr["chan0"])]
            kk = np.arange(int(ch["K"]))
            a = A1[ch["a_off"] + ii * ch["a_rs"] + kk[None, :] * ch["a_ks"]]
            b = B1[ch["b_off"] + kk[:, None] * ch["b_ks"] + jj * ch["b_ns"]]
            t1 = t1 + a @ b
            if not ch["last"]:
                continue
            r = int(ch["wrow"])
            rows.append(r)
            for o in range(int(pr["no"])):
                wi = int(widx[int(pr["wbase"]) + r * int(pr["wstride"]) + o])
                if wi >= 0:
                    acc[o] += W[wi] * t1
            t1 = np.zeros_like(t1)
        assert not t1.any(), "a part ends inside a stage-1 block"
        return acc, rows, ii, jj

    ti = 0   # parts appear in task order
    for wgi in range(len(parts) // 4):
        prs = parts[4 * wgi: 4 * wgi + 4]
        npass, reduce = int(prs[0]["npass"]), int(prs[0]["reduce"])
        assert all(int(p["npass"]) == npass and int(p["reduce"]) == reduce for p in prs)
        assert reduce == int(any(p["nparts"] > 1 for p in prs))
        w = 0
        while w < 4:
            pr = prs[w]
            if pr["nparts"] == 0:
                assert all(q["nparts"] == 0 for q in prs[w:]), "idle slots end the workgroup"
                break
            S = int(pr["nparts"])
            assert pr["part"] == 0 and w + S <= 4, "a task's parts start a run of slots"
            t = tasks[ti]
            g = groups[t["group"]]
            o0 = int(t["oc"]) * NO
            assert 1 <= S <= max(1, min(4, int(g["nblk"])))
            total, rows_all = None, []
            for p in range(S):
                q = prs[w + p]
                assert q["part"] == p and q["nparts"] == S
                assert (q["i0"], q["j0"], q["M"], q["N"]) == (t["i0"], t["j0"], g["M"], g["N"])
                assert q["ml"] == min(TILE, g["M"] - t["i0"]) and q["nl"] == min(TILE, g["N"] - t["j0"])
                assert (q["nblk"], q["flags"]) == (g["nblk"], g["flags"])
                assert q["no"] == min(NO, int(g["nout"]) - o0) and q["out0"] == g["out0"] + o0
                assert q["wbase"] == g["wbase"] + o0 and q["wstride"] == g["nout"]
                acc, rows, ii, jj = part_sum(q)
                assert rows == list(range(p, int(g["nblk"]), S)), "a part's stage-1 blocks"
                rows_all += rows
                total = acc if total is None else [x + y for x, y in zip(total, acc)]
            assert sorted(rows_all) == list(range(int(g["nblk"])))
            assert npass >= (int(pr["no"]) + 3) // 4
            for o in range(int(pr["no"])):
                out = outs[int(pr["out0"]) + o]
                ad = out["c_off"] + ii * out["c_rs"] + jj * out["c_cs"]
                C2[ad] = total[o] + (C2[ad] if pr["flags"] & G_ACCUMULATE else 0.0)
            ti += 1
            w += S
    assert ti == len(tasks), "a task has no parts"
    # every tile and output chunk of every group is a task, once
    seen = {(int(t["group"]), int(t["i0"]), int(t["j0"]), int(t["oc"])) for t in tasks}
    assert len(seen) == len(tasks)
    for gi, g in enumerate(groups):
        for oc in range(max(1, -(-int(g["nout"]) // NO))):
            for i0 in range(0, int(g["M"]), TILE):
                for j0 in range(0, int(g["N"]), TILE):
                    assert (gi, i0, j0, oc) in seen, ("task missing", gi, i0, j0, oc)
    return C2


def _wide_chain():
    # fp32, bond 1024 in 4 charges, one-column W: 32 x 32 wave tiles when asked
    return C.small_chain(seed=3, layout="coop", dtype="f32", total=1024, qmax=4, sigma=2.0, w=1, values="int")


CASES = {
    # name: (chain, split bound, wave tile edge)
    "small-coop": (lambda: C.small_chain(seed=3, layout="coop", values="int"), 0, 0),
    "small-natural": (lambda: C.small_chain(seed=5, layout="natural", values="int", dtype="f32"), 0, 0),
    "rabc_u1": (lambda: C.rabc_u1(layout="coop", values="int"), 0, 0),
    # every charge zero: 4 products per stage-1 block, 20 blocks and 20 outputs
    # per stage-2 row (outputs over three tasks), K over two chunks; unsplit,
    # 80 products per wave (past the 64 lane-held records)
    "neutral-natural-unsplit": (lambda: C.neutral_chain(layout="natural"), 1, 0),
    "neutral-coop-f32-split": (lambda: C.neutral_chain(seed=4, layout="coop", dtype="f32"), 0, 0),
    "wide-coop-f32-tile32": (_wide_chain, 0, 32),
}


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("accumulate", [False, True])
def test_fused_replay_equals_two_stage_oracle(name, accumulate):
    make, split, tile = CASES[name]
    ch = make()
    s1, s2 = ch.stages[0], ch.stages[1]
    fp = bst.FusedPlan(s1.con, s2.con, accumulate=accumulate, split=split, tile_cols=tile)
    assert fp.stats()["tile_blocks"] == (2 if tile == 32 else 1)
    bufs = {k: np.asarray(v, np.float64) for k, v in ch.buffers.items()}
    rng = np.random.default_rng(11)
    c0 = rng.integers(-3, 4, ch.sizes[s2.c_buf]).astype(np.float64) if accumulate else np.zeros(ch.sizes[s2.c_buf])
    t1 = oracle.contract(s1.con, bufs[s1.a_buf], bufs[s1.b_buf], np.zeros(ch.sizes[s1.c_buf]))
    want = oracle.contract(s2.con, t1, bufs[s2.b_buf], c0.copy(), accumulate=accumulate)
    got = replay(fp, bufs[s1.a_buf], bufs[s1.b_buf], bufs[s2.b_buf], c0.copy())
    _, mask = c_addresses(s2.con)
    assert np.array_equal(got[mask], want[mask])
    assert np.array_equal(got[~mask], c0[~mask]), "a write outside the stage-2 output views"


def test_fused_stats_count_the_two_stages():
    ch = C.small_chain(seed=3, layout="coop", values="int")
    s1, s2 = ch.stages[0].con, ch.stages[1].con
    fp = bst.FusedPlan(s1, s2)
    s = fp.stats()
    t1 = oracle.triples(s1)
    assert s["channels"] == len(t1)          # every stage-1 product feeds stage 2 here
    assert s["stage1_flops"] == oracle.useful_flops(s1)
    assert s["useful_flops"] == oracle.useful_flops(s1) + oracle.useful_flops(s2)
    assert s["groups"] == len(np.unique(s2.C.row_key))
    assert s["outputs"] == s2.C.nblocks
    assert s["terms"] == len(oracle.triples(s2))
    assert s["launches_per_contract"] == 1 and s["launches_issued"] == 0
    esz = 8
    want_bytes = (oracle.algorithmic_bytes(s1) - _c_bytes(s1, esz)   # stage-1 A, B
                  + s2.B.nblocks * esz + _c_bytes(s2, esz))
    assert s["alg_bytes"] == want_bytes


def _c_bytes(con, esz):
    return int(sum(con.m.dim[r] * con.n.dim[c] for r, c in zip(con.C.row_key, con.C.col_key))) * esz


def test_fused_refuses_what_it_cannot_fuse():
    ch = C.small_chain(seed=3, layout="coop")
    s1, s2, s3 = (st.con for st in ch.stages)
    with pytest.raises(bst.BscError) as e:
        bst.FusedPlan(s1, s2, dtype="bf16")
    assert e.value.name == "BSC_ERR_UNSUPPORTED"
    # stage 3's B is the MPS tensor, not a matrix of scalars
    with pytest.raises(bst.BscError) as e:
        bst.FusedPlan(s2, s3)
    assert e.value.name in ("BSC_ERR_UNSUPPORTED", "BSC_ERR_ARG")
    # a stage 2 whose A is not stage 1's output (another chain's T1 layout)
    other = C.small_chain(seed=3, layout="natural")
    with pytest.raises(bst.BscError) as e:
        bst.FusedPlan(s1, other.stages[1].con)
    assert e.value.name in ("BSC_ERR_UNSUPPORTED", "BSC_ERR_ARG")


def test_fused_reports_stage_errors():
    ch = C.small_chain(seed=3, layout="coop")
    s1, s2 = ch.stages[0].con, ch.stages[1].con
    bad = C.small_chain(seed=3, layout="coop").stages[0].con
    bad.A.offset[0] = -1
    with pytest.raises(bst.BscError) as e:
        bst.FusedPlan(bad, s2)
    assert e.value.name == "BSC_ERR_BOUNDS" and "stage 1" in str(e.value)
    bad2 = C.small_chain(seed=3, layout="coop").stages[1].con
    bad2.C.offset[0] = bad2.C.buffer_elems
    with pytest.raises(bst.BscError) as e:
        bst.FusedPlan(s1, bad2)
    assert e.value.name == "BSC_ERR_BOUNDS" and "stage 2" in str(e.value)


def test_fused_device_entry_points_check_arguments():
    ch = C.small_chain(seed=3, layout="coop")
    fp = bst.FusedPlan(ch.stages[0].con, ch.stages[1].con)
    L = bst._capi.lib()
    from ctypes import c_size_t, c_void_p
    assert L.bsc_fused_bind(fp._h, None, c_size_t(0), None) == -1
    assert L.bsc_fused_contract(None, None, None, None, None, None) == -1
    assert L.bsc_fused_worklist(fp._h, None, c_size_t(0)) == -1
    # unbound plan: refused before anything is enqueued
    st = L.bsc_fused_contract(fp._h, c_void_p(1), c_void_p(1), c_void_p(1), c_void_p(1), None)
    assert st in (-8, -7)


def test_fused_split_bound_is_honoured():
    ch = C.neutral_chain(layout="natural")
    s1, s2 = ch.stages[0].con, ch.stages[1].con
    for split, most in ((1, 1), (2, 2), (0, 4)):
        parts = decode(bst.FusedPlan(s1, s2, split=split))[6]
        assert parts["nparts"].max() == most, split
    assert decode(bst.FusedPlan(s1, s2, split=1))[6]["nchan"].max() > 64
    with pytest.raises(bst.BscError) as e:
        bst.FusedPlan(s1, s2, split=-1)
    assert e.value.name == "BSC_ERR_ARG"


def test_fused_wave_tile_choice():
    """32 x 32 wave tiles: fp32 with at most 4 outputs per task only, chosen
    automatically when they add little padding and still make enough tasks."""
    big = C.small_chain(seed=3, layout="coop", dtype="f32", total=2048, qmax=4, sigma=2.0, w=1)
    wide = _wide_chain()
    f64 = C.small_chain(seed=3, layout="coop", values="int")
    tb = lambda ch, t: bst.FusedPlan(ch.stages[0].con, ch.stages[1].con, tile_cols=t).stats()["tile_blocks"]
    assert tb(big, 0) == 2 and tb(big, 16) == 1
    assert tb(wide, 0) == 1 and tb(wide, 32) == 2      # too few 32 x 32 tasks to pick by itself
    assert tb(f64, 32) == 1                            # fp64 accumulators do not fit
    s_wide = bst.FusedPlan(wide.stages[0].con, wide.stages[1].con, tile_cols=32).stats()
    s_narrow = bst.FusedPlan(wide.stages[0].con, wide.stages[1].con, tile_cols=16).stats()
    assert s_wide["items"] < s_narrow["items"]
    for bad in (-16, 8, 64):
        with pytest.raises(bst.BscError) as e:
            bst.FusedPlan(wide.stages[0].con, wide.stages[1].con, tile_cols=bad)
        assert e.value.name == "BSC_ERR_ARG"
