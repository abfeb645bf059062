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
G_C_ALONG_N, G_ACCUMULATE = 1, 2
T_GENERIC, T_MFMA, T_TAIL, T_ZERO = 0, 1, 2, 3
TILE = {T_GENERIC: (64, 64), T_ZERO: (64, 64), T_MFMA: (128, 128)}

assert DVIEW.itemsize == 56 and DGROUP.itemsize == 32 and DRUN.itemsize == 32 and DTASK.itemsize == 16


def decode(plan):
    info, img = plan.worklist()
    tab = lambda dt, n, off: np.frombuffer(img, dtype=dt, count=n, offset=off)
    return (info, tab(DGROUP, info["n_groups"], info["off_groups"]), tab(DRUN, info["n_runs"], info["off_runs"]),
            tab(DVIEW, info["n_apieces"], info["off_apieces"]), tab(DVIEW, info["n_bpieces"], info["off_bpieces"]),
            tab(DVIEW, info["n_cpieces"], info["off_cpieces"]), tab(DTASK, info["n_tasks"], info["off_tasks"]))


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
    info, groups, runs, ap, bp, cp, tasks = decode(plan)
    c = np.array(c0, dtype=np.float64)
    written = np.zeros(c.size, np.int64)
    for t in tasks:
        g = groups[t["group"]]
        TM, TN = TILE[int(t["cls"])]
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
            assert aad.min(initial=0) >= 0 and aad.max(initial=-1) < con.A.buffer_elems
            assert bad.min(initial=0) >= 0 and bad.max(initial=-1) < con.B.buffer_elems
            acc += np.asarray(a, np.float64)[aad] @ np.asarray(b, np.float64)[bad].T
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
    return c, written


CASES = [("cfg1", lambda: C.cfg1().con, lambda: C.cfg1()),
         ("cfg1-flux1", None, lambda: C.cfg1("flux1")),
         ("cfg1-3leg", None, lambda: C.cfg1("flux1_3leg")),
         ("cfg2", None, lambda: C.cfg2())]


@pytest.mark.parametrize("axis", ["auto", "free_m", "free_n", "contract"])
@pytest.mark.parametrize("name", ["cfg1", "cfg1-flux1", "cfg1-3leg", "cfg2"])
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


def test_replay_cfg3_stages():
    ch = C.cfg3()
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
