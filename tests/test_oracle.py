"""Pins for the CPU oracle: checks against facts the mathematics fixes, never
against the oracle's own formula retyped.

P1  dense brute force on zero-filled materialised matrices (values placed by the
    generator's independent writer, products formed on the dense arrays), plus a
    pure-Python fixed-order scalar loop that is bit-identical in sector and dense
    form because the dense form only adds exact zeros;
P3  identity / permutation B blocks give C = A exactly;
P4  square orthogonal B blocks preserve the Frobenius norm;
P5  exact scaling by powers of two, additivity;
P6  one sector (trivial symmetry) is a plain GEMM;
P7  the sector join equals brute-force enumeration over every key triple;
P9  C elements outside every C view are untouched; rule breaks are rejected;
P11 the R/A/B/C chain equals a dense einsum, and an identity environment with a
    left-orthonormal A gives E' = identity.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle.contract import AXIS_CONTRACT, AXIS_FREE_M, AXIS_FREE_N, AXIS_NONE, AXIS_AUTO
from workloads import configs as C
from workloads.layout import view_addresses, write_block
from workloads.model import Contraction, Index, Operand

# ----------------------------------------------------------------------------
# helpers that never go through the oracle's view reader
# ----------------------------------------------------------------------------


def _starts(idx):
    return np.concatenate([[0], np.cumsum(idx.dim)]).astype(np.int64)


def _inner(idx, key):
    return 1 if idx.inner is None else int(idx.inner[key])


def _addr(op, i, ridx, cidx):
    r, c = int(op.row_key[i]), int(op.col_key[i])
    return view_addresses(op.offset[i], op.row_stride[i], op.col_stride[i], int(ridx.dim[r]), int(cidx.dim[c]),
                          _inner(ridx, r), _inner(cidx, c))


def _plant_dense(prob, rng):
    """Draw dense zero-filled A~, B~ with values only inside listed blocks, and
    write each block into fresh buffers with the generator's writer."""
    con = prob.con
    out = []
    for op, ridx, cidx in ((con.A, con.m, con.k), (con.B, con.k, con.n)):
        rs, cs = _starts(ridx), _starts(cidx)
        dense = np.zeros((rs[-1], cs[-1]))
        buf = np.full(op.buffer_elems, np.nan)
        for i in range(op.nblocks):
            r, c = int(op.row_key[i]), int(op.col_key[i])
            v = rng.standard_normal((rs[r + 1] - rs[r], cs[c + 1] - cs[c]))
            dense[rs[r]:rs[r + 1], cs[c]:cs[c + 1]] = v
            write_block(buf, op.offset[i], op.row_stride[i], op.col_stride[i], v, _inner(ridx, r), _inner(cidx, c))
        out += [dense, buf]
    return out


def _read_c(con, cbuf):
    """C blocks read with the generator's address helper: {(m,n): array}."""
    return {(int(con.C.row_key[i]), int(con.C.col_key[i])): cbuf[_addr(con.C, i, con.m, con.n)]
            for i in range(con.C.nblocks)}


RANDOM_CASES = [
    dict(seed=s, nq=nq, flux=fl, two_leg=tl, density=de)
    for s, (nq, fl, tl, de) in enumerate(itertools.product([1, 2], [(0, 0), (1, -1), (1, 0)], [False, True], [1.0, 0.6]))
]


# ----------------------------------------------------------------------------
# P1: dense brute force
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("case", RANDOM_CASES, ids=lambda c: f"s{c['seed']}-q{c['nq']}-f{c['flux']}-2l{c['two_leg']}-d{c['density']}")
def test_p1_dense_bruteforce_random(case):
    prob = C.random_problem(case["seed"] + 100, nq=case["nq"], nkeys=(5, 6, 5), maxdim=9, qrange=1,
                            flux=case["flux"], two_leg=case["two_leg"], density=case["density"])
    con = prob.con
    rng = np.random.default_rng(case["seed"])
    Ad, abuf, Bd, bbuf = _plant_dense(prob, rng)
    canary = np.full(con.C.buffer_elems, -7.25)
    out = oracle.contract(con, abuf, bbuf, canary)
    Cd = Ad @ Bd
    rs, cs = _starts(con.m), _starts(con.n)
    got = _read_c(con, out)
    touched = np.zeros(con.C.buffer_elems, bool)
    for i in range(con.C.nblocks):
        m, n = int(con.C.row_key[i]), int(con.C.col_key[i])
        ref = Cd[rs[m]:rs[m + 1], cs[n]:cs[n + 1]]
        np.testing.assert_allclose(got[(m, n)], ref, rtol=1e-13, atol=1e-13)
        touched[_addr(con.C, i, con.m, con.n).ravel()] = True
    # P9: nothing outside the C views moved
    assert np.all(out[~touched] == -7.25)
    # the dense product has no mass outside listed C blocks (charge conservation)
    mask = np.zeros_like(Cd, bool)
    for i in range(con.C.nblocks):
        m, n = int(con.C.row_key[i]), int(con.C.col_key[i])
        mask[rs[m]:rs[m + 1], cs[n]:cs[n + 1]] = True
    assert np.all(Cd[~mask] == 0.0)


def _scalar_sector(con, A, B):
    amap = {(int(r), int(c)): A[i] for i, (r, c) in enumerate(zip(con.A.row_key, con.A.col_key))}
    bmap = {(int(r), int(c)): B[i] for i, (r, c) in enumerate(zip(con.B.row_key, con.B.col_key))}
    out = {}
    for i in range(con.C.nblocks):
        m, n = int(con.C.row_key[i]), int(con.C.col_key[i])
        R, N = int(con.m.dim[m]), int(con.n.dim[n])
        blk = [[0.0] * N for _ in range(R)]
        for k in range(con.k.nkeys):
            if (m, k) in amap and (k, n) in bmap:
                a, b = amap[(m, k)], bmap[(k, n)]
                for r in range(R):
                    for c in range(N):
                        s = blk[r][c]
                        for kk in range(int(con.k.dim[k])):
                            s += a[r][kk] * b[kk][c]
                        blk[r][c] = s
        out[(m, n)] = blk
    return out


def _scalar_dense(Ad, Bd, r0, r1, c0, c1):
    return [[sum_fixed(Ad[r], Bd[:, c]) for c in range(c0, c1)] for r in range(r0, r1)]


def sum_fixed(row, col):
    s = 0.0
    for x, y in zip(row.tolist(), col.tolist()):
        s += x * y
    return s


@pytest.mark.parametrize("seed", range(6))
def test_p1_scalar_loop_bit_identical(seed):
    prob = C.random_problem(seed + 300, nq=1, nkeys=(3, 4, 3), maxdim=5, qrange=1, two_leg=True, density=0.8)
    con = prob.con
    rng = np.random.default_rng(seed)
    Ad, abuf, Bd, bbuf = _plant_dense(prob, rng)
    rs, ks, cs = _starts(con.m), _starts(con.k), _starts(con.n)
    Ab = [Ad[rs[r]:rs[r + 1], ks[c]:ks[c + 1]].tolist() for r, c in zip(con.A.row_key, con.A.col_key)]
    Bb = [Bd[ks[r]:ks[r + 1], cs[c]:cs[c + 1]].tolist() for r, c in zip(con.B.row_key, con.B.col_key)]
    sec = _scalar_sector(con, Ab, Bb)
    for (m, n), blk in sec.items():
        den = _scalar_dense(Ad, Bd, rs[m], rs[m + 1], cs[n], cs[n + 1])
        assert blk == den, (m, n)   # bit-identical: the dense loop only adds exact zeros
    out = _read_c(con, oracle.contract(con, abuf, bbuf))
    for key, blk in sec.items():
        np.testing.assert_allclose(out[key], np.array(blk).reshape(out[key].shape), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("variant", ["diag", "flux1", "flux1_3leg"])
def test_p1_tiny_u1_dense(variant):
    p = C.tiny_u1(variant)
    out = oracle.contract(p.con, p.a, p.b)
    Cd = oracle.densify(p.con.C, out, p.con.m, p.con.n)
    # dense product formed from the generator's own buffers via independent addresses
    con = p.con
    Ad = np.zeros((con.m.dim.sum(), con.k.dim.sum()))
    Bd = np.zeros((con.k.dim.sum(), con.n.dim.sum()))
    for op, buf, dense, ri, ci in ((con.A, p.a, Ad, con.m, con.k), (con.B, p.b, Bd, con.k, con.n)):
        r0, c0 = _starts(ri), _starts(ci)
        for i in range(op.nblocks):
            r, c = int(op.row_key[i]), int(op.col_key[i])
            dense[r0[r]:r0[r + 1], c0[c]:c0[c + 1]] = buf[_addr(op, i, ri, ci)]
    np.testing.assert_allclose(Cd, Ad @ Bd, rtol=1e-14, atol=1e-14)


def test_tiny_u1_flux_encodings_agree():
    a = oracle.contract(C.tiny_u1("flux1").con, C.tiny_u1("flux1").a, C.tiny_u1("flux1").b)
    p3 = C.tiny_u1("flux1_3leg")
    b = oracle.contract(p3.con, p3.a, p3.b)
    assert np.array_equal(a, b)
    assert len(oracle.triples(p3.con)) == 4 and oracle.useful_flops(p3.con) == 452


# ----------------------------------------------------------------------------
# P3 / P4 / P5 / P6: special cases and closed forms
# ----------------------------------------------------------------------------

def _with_b(prob, kind, rng):
    """Replace B by square blocks on the (k, k) diagonal: identity, a permutation
    or an orthogonal matrix; n is a copy of k and C lists every allowed block."""
    con = prob.con
    k = con.k
    n = Index(k.charge.copy(), k.dim.copy(), None if k.inner is None else k.inner.copy())
    off, rs, cs, mats = [], [], [], []
    top = 0
    b = []
    for key in range(k.nkeys):
        d = int(k.dim[key])
        if kind == "identity":
            Mx = np.eye(d)
        elif kind == "perm":
            Mx = np.eye(d)[rng.permutation(d)]
        else:
            Mx, _ = np.linalg.qr(rng.standard_normal((d, d)))
        off.append(top)
        rs.append((d, 0))
        cs.append((1, 0))
        b.append(Mx.ravel())
        mats.append(Mx)
        top += d * d
    # single-leg views over the key dims (inner extents dropped for n and the B rows)
    k1 = Index(k.charge.copy(), k.dim.copy())
    n1 = Index(k.charge.copy(), k.dim.copy())
    Bop = Operand(np.arange(k.nkeys), np.arange(k.nkeys), off, rs, cs, np.zeros(k.nq, np.int32), top)
    # A with single-leg column views: rebuild A's col strides for single legs is not
    # possible in general, so keep A as is but require its k keys to be single-leg
    m = con.m
    cpairs = [(i, j) for i in range(m.nkeys) for j in range(n1.nkeys)
              if np.array_equal(m.charge[i] - n1.charge[j], con.A.flux)]
    coff, crs, ccs = [], [], []
    top_c = 0
    for (i, j) in cpairs:
        R, N = int(m.dim[i]), int(n1.dim[j])
        coff.append(top_c)
        crs.append((N, 0) if m.inner_of(i) == 1 else (N * m.inner_of(i), N))
        ccs.append((1, 0))
        top_c += R * N
    Cop = Operand([p[0] for p in cpairs], [p[1] for p in cpairs], coff, crs, ccs, con.A.flux.copy(), top_c)
    con2 = Contraction(m, k1, n1, con.A, Bop, Cop, con.dtype)
    return con2, np.concatenate(b) if b else np.zeros(0), mats


@pytest.mark.parametrize("kind", ["identity", "perm"])
@pytest.mark.parametrize("seed", range(4))
def test_p3_identity_and_permutation(kind, seed):
    prob = C.random_problem(seed + 500, nq=1, nkeys=(5, 5, 5), maxdim=8, qrange=1, two_leg=False, flux=(1, 0))
    rng = np.random.default_rng(seed)
    con, bbuf, mats = _with_b(prob, kind, rng)
    out = oracle.contract(con, prob.a, bbuf)
    got = _read_c(con, out)
    amap = {(int(r), int(c)): i for i, (r, c) in enumerate(zip(con.A.row_key, con.A.col_key))}
    for (m, n), blk in got.items():
        if (m, n) in amap:
            a = prob.a[_addr(con.A, amap[(m, n)], con.m, con.k)]
            assert np.array_equal(blk, a @ mats[n]) if kind == "perm" else np.array_equal(blk, a)
            if kind == "perm":
                # a permutation only moves columns: exact
                assert np.array_equal(blk, a[:, np.argmax(mats[n], axis=0)])
        else:
            assert np.all(blk == 0.0)


@pytest.mark.parametrize("seed", range(4))
def test_p4_orthogonal_preserves_norm(seed):
    prob = C.random_problem(seed + 600, nq=1, nkeys=(6, 5, 5), maxdim=10, qrange=1, two_leg=False)
    rng = np.random.default_rng(seed)
    con, bbuf, _ = _with_b(prob, "orth", rng)
    out = oracle.contract(con, prob.a, bbuf)
    ca = sum(float(np.sum(prob.a[_addr(con.A, i, con.m, con.k)] ** 2)) for i in range(con.A.nblocks))
    cc = sum(float(np.sum(v ** 2)) for v in _read_c(con, out).values())
    assert abs(np.sqrt(cc) - np.sqrt(ca)) <= 1e-13 * np.sqrt(ca)


@pytest.mark.parametrize("seed", range(4))
def test_p5_linearity(seed):
    prob = C.random_problem(seed + 700, nq=2, nkeys=(5, 5, 5), maxdim=8, qrange=1)
    con = prob.con
    base = oracle.contract(con, prob.a, prob.b)
    for p in (-3, 1, 5):
        scaled = oracle.contract(con, prob.a * 2.0 ** p, prob.b)
        assert np.array_equal(scaled, base * 2.0 ** p)
    rng = np.random.default_rng(seed)
    a2 = rng.standard_normal(prob.a.shape)
    s = oracle.contract(con, prob.a + a2, prob.b)
    t = base + oracle.contract(con, a2, prob.b)
    np.testing.assert_allclose(s, t, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", [(7, 5, 3), (1, 9, 4), (13, 1, 6), (16, 16, 16)])
@pytest.mark.parametrize("orient", ["rr", "rc", "cr", "cc"])
def test_p6_single_sector_is_plain_gemm(shape, orient):
    M, K, N = shape
    rng = np.random.default_rng(M * 100 + K * 10 + N)
    A = rng.standard_normal((M, K))
    B = rng.standard_normal((K, N))
    lda, ldb = K + 3, N + 2
    abuf = np.full(M * lda + K * lda + 8, np.nan)
    bbuf = np.full(K * ldb + N * ldb + 8, np.nan)
    if orient[0] == "r":
        ars, acs = (lda, 0), (1, 0)
    else:
        ars, acs = (1, 0), (M + 2, 0)
    if orient[1] == "r":
        brs, bcs = (ldb, 0), (1, 0)
    else:
        brs, bcs = (1, 0), (K + 1, 0)
    write_block(abuf, 2, ars, acs, A)
    write_block(bbuf, 1, brs, bcs, B)
    idx = lambda d: Index([[0]], [d])
    con = Contraction(idx(M), idx(K), idx(N),
                      Operand([0], [0], [2], [ars], [acs], [0], abuf.size),
                      Operand([0], [0], [1], [brs], [bcs], [0], bbuf.size),
                      Operand([0], [0], [0], [(N, 0)], [(1, 0)], [0], M * N), "f64")
    out = oracle.contract(con, abuf, bbuf)
    np.testing.assert_allclose(out.reshape(M, N), np.matmul(A, B), rtol=1e-14, atol=1e-14)


def test_accumulate_adds():
    p = C.tiny_u1("diag")
    first = oracle.contract(p.con, p.a, p.b)
    twice = oracle.contract(p.con, p.a, p.b, first, accumulate=True)
    np.testing.assert_allclose(twice, 2 * first, rtol=1e-15, atol=0)


# ----------------------------------------------------------------------------
# P7: sector join and grouping structure
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(8))
def test_p7_triples_bruteforce(seed):
    prob = C.random_problem(seed + 800, nq=1 + seed % 2, nkeys=(6, 7, 6), maxdim=4, qrange=1, density=0.7)
    con = prob.con
    A = {(int(r), int(c)) for r, c in zip(con.A.row_key, con.A.col_key)}
    B = {(int(r), int(c)) for r, c in zip(con.B.row_key, con.B.col_key)}
    brute = [(m, k, n) for m in range(con.m.nkeys) for n in range(con.n.nkeys) for k in range(con.k.nkeys)
             if (m, k) in A and (k, n) in B]
    assert oracle.triples(con).tolist() == [list(t) for t in brute]
    fl = sum(2 * int(con.m.dim[m]) * int(con.k.dim[k]) * int(con.n.dim[n]) for m, k, n in brute)
    assert oracle.useful_flops(con) == fl


def _check_groups(con, axis):
    t = oracle.triples(con)
    ax, gid, gl = oracle.groups(con, axis)
    A = {(int(r), int(c)) for r, c in zip(con.A.row_key, con.A.col_key)}
    B = {(int(r), int(c)) for r, c in zip(con.B.row_key, con.B.col_key)}
    L = {}
    for m, k, n in t.tolist():
        L.setdefault((m, n), []).append(k)
    # partition: each triple is in exactly one group, and that group holds it
    seen = set()
    for i, (m, k, n) in enumerate(t.tolist()):
        rows, cols, kl = gl[gid[i]]
        assert m in rows and n in cols and k in kl
        seen.add((m, k, n))
    assert len(seen) == len(t)
    covered = sum(len(r) * len(c) * len(kl) for r, c, kl in gl)
    assert covered == len(t)                       # hole-free: no (m,k,n) of a group is missing
    for rows, cols, kl in gl:
        assert list(kl) == sorted(kl) and list(rows) == sorted(rows) and list(cols) == sorted(cols)
        if ax == AXIS_FREE_M:
            assert len(cols) == 1
        elif ax == AXIS_FREE_N:
            assert len(rows) == 1
        else:
            assert len(rows) == 1 and len(cols) == 1
        if ax == AXIS_NONE:
            assert len(kl) == 1
        for m in rows:
            for k in kl:
                assert (m, k) in A
        for k in kl:
            for n in cols:
                assert (k, n) in B
        if ax != AXIS_NONE:   # per-sector groups hold one k of a possibly longer list
            for m in rows:
                for n in cols:
                    assert L[(m, n)] == list(kl)
    # maximal: no two free-axis groups share their key
    if ax == AXIS_FREE_M:
        keys = [(c[0], kl) for r, c, kl in gl]
        assert len(keys) == len(set(keys))
        assert [(c[0], r[0]) for r, c, kl in gl] == sorted((c[0], r[0]) for r, c, kl in gl)
    if ax == AXIS_FREE_N:
        keys = [(r[0], kl) for r, c, kl in gl]
        assert len(keys) == len(set(keys))
        assert [(r[0], c[0]) for r, c, kl in gl] == sorted((r[0], c[0]) for r, c, kl in gl)
    if ax == AXIS_CONTRACT:
        assert [(r[0], c[0]) for r, c, kl in gl] == sorted(L)
    return ax, gl


@pytest.mark.parametrize("axis", [AXIS_NONE, AXIS_FREE_M, AXIS_FREE_N, AXIS_CONTRACT, AXIS_AUTO])
@pytest.mark.parametrize("seed", range(5))
def test_p7_groups_invariants(axis, seed):
    prob = C.random_problem(seed + 900, nq=1, nkeys=(7, 6, 7), maxdim=3, qrange=1, density=0.8)
    _check_groups(prob.con, axis)


def test_groups_on_configs():
    ax, gl = _check_groups(C.ragged_batch().con, AXIS_FREE_M)
    assert len(gl) == 500 and all(len(r) == 8 for r, c, kl in gl)
    ch = C.rabc_u1()
    ax, gl = _check_groups(ch.stages[0].con, AXIS_AUTO)
    assert ax == AXIS_FREE_M
    ax, gl = _check_groups(ch.stages[1].con, AXIS_AUTO)
    assert ax == AXIS_CONTRACT


def test_auto_rule_threshold():
    """AUTO picks CONTRACT exactly when more than 1/4 of non-empty C blocks sum over >1 k."""
    for seed in range(12):
        prob = C.random_problem(seed + 1000, nq=1, nkeys=(5, 6, 5), maxdim=2, qrange=1, density=0.5)
        t = oracle.triples(prob.con).tolist()
        L = {}
        for m, k, n in t:
            L.setdefault((m, n), []).append(k)
        multi = sum(1 for v in L.values() if len(v) > 1)
        ax, _, _ = oracle.groups(prob.con, AXIS_AUTO)
        assert (ax == AXIS_CONTRACT) == (len(L) > 0 and 4 * multi > len(L))


# ----------------------------------------------------------------------------
# P9: rejected descriptors
# ----------------------------------------------------------------------------

def _tiny():
    p = C.tiny_u1("diag")
    return p


def test_rejects_charge_violation():
    p = _tiny()
    p.con.A.col_key[0] = 1
    with pytest.raises(oracle.OracleError):
        oracle.contract(p.con, p.a, p.b)


def test_rejects_overlap():
    p = _tiny()
    p.con.C.offset[1] = p.con.C.offset[0]
    with pytest.raises(oracle.OracleError):
        oracle.contract(p.con, p.a, p.b)


def test_rejects_missing_output():
    p = _tiny()
    keep = np.arange(p.con.C.nblocks) != 2
    for f in ("row_key", "col_key", "offset", "row_stride", "col_stride"):
        setattr(p.con.C, f, getattr(p.con.C, f)[keep])
    with pytest.raises(oracle.OracleError):
        oracle.contract(p.con, p.a, p.b)


def test_rejects_out_of_bounds():
    p = _tiny()
    p.con.B.buffer_elems = int(p.con.B.offset[-1])
    with pytest.raises(oracle.OracleError):
        oracle.contract(p.con, p.a, p.b)


def test_rejects_bad_flux():
    p = _tiny()
    p.con.C.flux[:] = 1
    with pytest.raises(oracle.OracleError):
        oracle.contract(p.con, p.a, p.b)


# ----------------------------------------------------------------------------
# P11: the R/A/B/C chain
# ----------------------------------------------------------------------------

def _dense_tensors(ch):
    info = ch.info
    D = info["D"]
    st = np.concatenate([[0], np.cumsum(D)])
    S, d, w = len(D), len(info["local_q"]), len(info["mpo_q"])
    m = int(st[-1])
    E = np.zeros((m, w, m))
    A = np.zeros((m, d, m))
    W = np.zeros((w, d, d, w))
    for (a, ww, ap), v in info["E"].items():
        E[st[a]:st[a + 1], ww, st[ap]:st[ap + 1]] = v
    for (a, s, b), v in info["A"].items():
        A[st[a]:st[a + 1], s, st[b]:st[b + 1]] = v
    for (ww, s, sp, wp), v in info["W"].items():
        W[ww, s, sp, wp] = v
    return st, E, A, W


def _ep_blocks(ch, buf):
    D = ch.info["D"]
    out = {}
    for key in ch.info["Ep_blocks"]:
        off, rs, cs = ch.info["Ep_loc"][key]
        out[key] = buf[view_addresses(off, (rs, 0), (cs, 0), D[key[0]], D[key[2]])]
    return out


@pytest.mark.parametrize("layout", ["coop", "natural"])
def test_p11_chain_vs_dense_einsum(layout):
    ch = C.small_chain(seed=11, layout=layout)
    bufs = oracle.run_chain(ch)
    st, E, A, W = _dense_tensors(ch)
    # one einsum over the dense tensors; the contraction path may keep intermediates
    # (numpy's default memory cap would otherwise force the naive 8-index loop)
    expr = "awc,asb,wstv,ctd->bvd"
    path = np.einsum_path(expr, E, A, W, A, optimize=("greedy", 1e9))[0]
    Ep = np.einsum(expr, E, A, W, A, optimize=path)
    got = _ep_blocks(ch, bufs["Ep"])
    mask = np.zeros(Ep.shape, bool)
    for (b, wp, bp), v in got.items():
        ref = Ep[st[b]:st[b + 1], wp, st[bp]:st[bp + 1]]
        np.testing.assert_allclose(v, ref, rtol=1e-12, atol=1e-12)
        mask[st[b]:st[b + 1], wp, st[bp]:st[bp + 1]] = True
    assert np.all(Ep[~mask] == 0.0)  # no weight outside E''s charge-allowed blocks


def test_p11_identity_environment():
    ch = C.small_chain(seed=5, layout="coop", values="identity", w=1)
    bufs = oracle.run_chain(ch)
    got = _ep_blocks(ch, bufs["Ep"])
    assert got
    for (b, wp, bp), v in got.items():
        ref = np.eye(v.shape[0]) if b == bp else np.zeros_like(v)
        np.testing.assert_allclose(v, ref, atol=1e-13)
