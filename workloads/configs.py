"""Seeded synthetic sector structures shaped like the workloads of the uni20
"block coalescing" note (Summary: block-sparse contractions split into many
small per-sector GEMMs; section "One mechanism, three payoffs": the R/A/B/C
environment update is the consumer).  The note's own calibrated R/A/B/C data is
not public, so these generators stand in for it.

Every generator uses numpy's PCG64 (`np.random.default_rng(seed)`) and draws in
the order written.  Blocks are enumerated in canonical order (sorted by their
sector tuple) and their values are drawn row-major per block.

Conventions (also used by the engine and the oracle):
  * charge rule: block (r, c) of an operand X may exist iff
    q_row(r) - q_col(c) == flux_X (componentwise), and a product has
    flux_A + flux_B;
  * a fused multi-index key carries the signed sum of its legs' charges.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np

from .layout import Arena, round_up, write_block
from .model import Chain, Contraction, Index, Operand, Problem, Stage, bf16_round


# ----------------------------------------------------------------------------
# small helpers
# ----------------------------------------------------------------------------

def _operand(blocks, flux, nq, buffer_elems):
    """blocks: list of (row_key, col_key, offset, (rs0, rs1), (cs0, cs1))."""
    if blocks:
        rk, ck, off, rs, cs = zip(*blocks)
    else:
        rk = ck = off = ()
        rs = cs = np.zeros((0, 2), np.int64)
    return Operand(np.array(rk, np.int32), np.array(ck, np.int32), np.array(off, np.int64),
                   np.array(rs, np.int64).reshape(-1, 2), np.array(cs, np.int64).reshape(-1, 2),
                   np.array(flux, np.int32).reshape(nq), buffer_elems)


def _rowmajor(pairs, rdim, cdim, align=1, ld_align=1, arena=None):
    """Row-major contiguous blocks in the given order.  Returns (blocks, size)."""
    arena = arena or Arena(align)
    out = []
    for (r, c) in pairs:
        R, C = int(rdim[r]), int(cdim[c])
        ld = round_up(C, ld_align)
        off = arena.take(R * ld)
        out.append((r, c, off, (ld, 0), (1, 0)))
    return out, arena.top


def _fill(buf, blocks, rdim, cdim, draw, rinner=None, cinner=None):
    """Draw values per block (canonical order, row-major) and place them."""
    for (r, c, off, rs, cs) in blocks:
        R, C = int(rdim[r]), int(cdim[c])
        ri = 1 if rinner is None else int(rinner[r])
        ci = 1 if cinner is None else int(cinner[c])
        write_block(buf, off, rs, cs, draw((R, C)), ri, ci)


def _round_dims(raw, qkeys, total):
    """d = max(1, rint(raw)), then +-1 corrections cycling over sectors in
    (-raw, charge) order until the dimensions sum to `total`."""
    d = np.maximum(1, np.rint(raw)).astype(np.int64)
    order = sorted(range(len(raw)), key=lambda i: (-raw[i], tuple(int(v) for v in np.atleast_1d(qkeys[i]))))
    step = 1 if d.sum() < total else -1
    i = 0
    while d.sum() != total:
        j = order[i % len(order)]
        if step > 0 or d[j] > 1:
            d[j] += step
        i += 1
        if i > 100 * len(order) * max(1, abs(total)):
            raise RuntimeError("dimension rounding did not converge")
    return d


# ----------------------------------------------------------------------------
# config 1: tiny U(1) block-sparse GEMM, fp64
# ----------------------------------------------------------------------------

def tiny_u1(variant: str = "diag", seed: int = 1001) -> Problem:
    """Five U(1) sectors q=-2..2 per index, dims uniform in 1..8.

    variant 'diag'      : A, B, C diagonal (q_m = q_k = q_n), 5 sector GEMMs;
    variant 'flux1'     : A has flux +1 (q_m - q_k = +1), C flux +1, 4 sector GEMMs;
    variant 'flux1_3leg': the same tensors written as three-leg tensors whose extra
                          leg x (one key, charge +1, dim 1) is fused into the row
                          multi-index (m, x) of A and C, so every operand has flux 0.
    """
    rng = np.random.default_rng(seed)
    dm = rng.integers(1, 9, 5)
    dk = rng.integers(1, 9, 5)
    dn = rng.integers(1, 9, 5)
    q = np.arange(-2, 3)
    m, k, n = Index(q[:, None], dm), Index(q[:, None], dk), Index(q[:, None], dn)
    fa = 0 if variant == "diag" else 1
    a_pairs = [(i, j) for i in range(5) for j in range(5) if q[i] - q[j] == fa]
    b_pairs = [(i, i) for i in range(5)]
    c_pairs = [(i, j) for i in range(5) for j in range(5) if q[i] - q[j] == fa]
    Ab, na = _rowmajor(a_pairs, dm, dk)
    Bb, nb = _rowmajor(b_pairs, dk, dn)
    Cb, nc = _rowmajor(c_pairs, dm, dn)
    a = np.zeros(na)
    b = np.zeros(nb)
    _fill(a, Ab, dm, dk, lambda s: rng.standard_normal(s))
    _fill(b, Bb, dk, dn, lambda s: rng.standard_normal(s))
    flux_a, flux_c = [fa], [fa]
    if variant == "flux1_3leg":
        # row multi-index (m, x): x has charge +1 and enters with the opposite sign
        m = Index((q - 1)[:, None], dm)
        flux_a, flux_c = [0], [0]
    elif variant not in ("diag", "flux1"):
        raise ValueError(variant)
    con = Contraction(m, k, n, _operand(Ab, flux_a, 1, na), _operand(Bb, [0], 1, nb),
                      _operand(Cb, flux_c, 1, nc), "f64")
    return Problem(f"tiny_u1-{variant}", con, a, b, {"dims": (dm, dk, dn)})


# ----------------------------------------------------------------------------
# config 2: tail-heavy ragged batch, fp32
# ----------------------------------------------------------------------------

def ragged_batch(seed: int = 1002, ngroups: int = 500, per_group: int = 8, p: float = 0.35, cap: int = 64) -> Problem:
    """4000 independent sector GEMMs with geometric(p) dims capped at 64; every
    8 consecutive GEMMs share one (K, N, B) so they stack along M."""
    rng = np.random.default_rng(seed)
    K = np.minimum(rng.geometric(p, ngroups), cap)
    N = np.minimum(rng.geometric(p, ngroups), cap)
    M = np.minimum(rng.geometric(p, ngroups * per_group), cap)
    g = np.arange(ngroups * per_group) // per_group
    m = Index(g[:, None], M)
    k = Index(np.arange(ngroups)[:, None], K)
    n = Index(np.arange(ngroups)[:, None], N)
    a_pairs = [(i, int(g[i])) for i in range(len(M))]
    b_pairs = [(j, j) for j in range(ngroups)]
    Ab, na = _rowmajor(a_pairs, M, K)
    Bb, nb = _rowmajor(b_pairs, K, N)
    Cb, nc = _rowmajor(a_pairs, M, N)
    a = np.zeros(na, np.float32)
    b = np.zeros(nb, np.float32)
    draw = lambda s: rng.uniform(-1.0, 1.0, s).astype(np.float32)
    _fill(a, Ab, M, K, draw)
    _fill(b, Bb, K, N, draw)
    con = Contraction(m, k, n, _operand(Ab, [0], 1, na), _operand(Bb, [0], 1, nb),
                      _operand(Cb, [0], 1, nc), "f32")
    return Problem("ragged_batch-ragged", con, a, b, {"M": M, "N": N, "K": K})


# ----------------------------------------------------------------------------
# config 5: large block-sparse GEMM, bf16 inputs / fp32 accumulate
# ----------------------------------------------------------------------------

def blockdiag_bf16_dims(reading: str = "i_scaled", seed: int = 1005):
    rng = np.random.default_rng(seed)
    if reading == "i_scaled":
        main = np.clip(np.rint(rng.lognormal(5.0, 0.6, 45)), 16, 1024)
        tail = rng.integers(1, 5, 19)
        c = (16384 - tail.sum()) / main.sum()
        main = np.clip(np.rint(main * c), 16, 1024)
    elif reading in ("ii_scaled", "ii_literal"):
        main = np.clip(np.rint(rng.lognormal(5.0, 0.6, 64)), 16, 1024)
        tail = rng.integers(1, 5, 19)
        if reading == "ii_scaled":
            c = (16384 - tail.sum()) / main.sum()
            main = np.clip(np.rint(main * c), 16, 1024)
    else:
        raise ValueError(reading)
    dims = np.concatenate([main, tail]).astype(np.int64)
    perm = rng.permutation(len(dims))
    return dims[perm], rng


def blockdiag_bf16(reading: str = "i_scaled", seed: int = 1005, ld_align: int = 1, align: int = 1,
         values: bool = True, int_values: bool = False) -> Problem:
    """U(1) sectors q=0..S-1 sharing one dimension list for m, k and n, flux 0, so
    every operand is block diagonal.  Dims are lognormal(5, 0.6) clipped to
    16..1024 (rescaled so the dense equivalent is ~16384) plus tail sectors of
    dim 1..4.  Values N(0, 0.02) drawn in fp32 and rounded to bf16 (RNE).

    ld_align / align pad each block's leading dimension / start offset (in
    elements); 1 gives plain contiguous row-major blocks.  int_values draws
    integers in {-2..2} instead (exact in bf16; with K <= 1024 every partial
    sum is an integer below 2^24, so any summation order is exact in fp32)."""
    dims, rng = blockdiag_bf16_dims(reading, seed)
    S = len(dims)
    q = np.arange(S)
    idx = Index(q[:, None], dims)
    pairs = [(i, i) for i in range(S)]
    Ab, na = _rowmajor(pairs, dims, dims, align, ld_align)
    Bb, nb = _rowmajor(pairs, dims, dims, align, ld_align)
    Cb, nc = _rowmajor(pairs, dims, dims, align, ld_align)
    a = np.zeros(na, np.float32)
    b = np.zeros(nb, np.float32)
    if values and int_values:
        draw = lambda s: rng.integers(-2, 3, s).astype(np.float32)
        _fill(a, Ab, dims, dims, draw)
        _fill(b, Bb, dims, dims, draw)
    elif values:
        draw = lambda s: bf16_round((rng.standard_normal(s) * 0.02).astype(np.float32))
        _fill(a, Ab, dims, dims, draw)
        _fill(b, Bb, dims, dims, draw)
    con = Contraction(idx, idx, idx, _operand(Ab, [0], 1, na), _operand(Bb, [0], 1, nb),
                      _operand(Cb, [0], 1, nc), "bf16")
    return Problem(f"blockdiag_bf16-{reading}" + ("-int" if int_values else ""), con, a, b, {"dims": dims})


# ----------------------------------------------------------------------------
# configs 3 and 4: the R/A/B/C environment update as a chain of block GEMMs
# ----------------------------------------------------------------------------

def _bond_u1(total=1024, qmax=20, sigma=6.0):
    q = np.arange(-qmax, qmax + 1)
    w = np.exp(-q.astype(float) ** 2 / (2 * sigma ** 2))
    raw = total * w / w.sum()
    return q[:, None].astype(np.int64), _round_dims(raw, q[:, None], total)


def _bond_u1u1(total=4096, half=7, sigma=2.2, threshold=0.5):
    x = np.arange(-half, half + 1)
    X, Y = np.meshgrid(x, x, indexing="ij")
    w = np.exp(-(X.astype(float) ** 2 + Y.astype(float) ** 2) / (2 * sigma ** 2))
    raw = total * w / w.sum()
    pop = raw >= threshold
    q = np.stack([X[pop], Y[pop]], axis=1).astype(np.int64)
    return q, _round_dims(raw[pop], q, total)


def rabc_chain(bond_q, bond_dim, local_q, mpo_q, mpo_pairs, dtype, rng, layout="coop",
               values="normal", name="rabc", ld_align=1):
    """E'[b,w',b'] = sum E[a,w,a'] A[a,s,b] W[w,s,s',w'] A*[a',s',b'] as three stages:

      (1) T1[(w,a'),(s,b)]  = sum_a     E^T[(w,a'),a]   A[a,(s,b)]
      (2) T2[(a',b),(s',w')] = sum_(w,s) T1[(a',b),(w,s)] W[(w,s),(s',w')]
      (3) E'[(b,w'),b']     = sum_(a',s') T2[(b,w'),(a',s')] A*[(a',s'),b']

    Tensor rules: E: q_a = q_w + q_a';  A: q_b = q_a + q_s;
    W: q_w + q_s = q_s' + q_w';  E': q_b = q_w' + q_b'.  Real dtypes, so A* = A.

    layout 'coop'   : layouts chosen so the expected coalescing groups are
                      stride-addressable (E per a-sector with (w,a') interleaved
                      along columns, A per b-sector as a fused (a,s) x b matrix,
                      T1 per (a',b) with (w,s) slowest, T2 per (b,w') with (a',s')
                      concatenated along columns, E' like E);
    layout 'natural': every tensor block contiguous row-major in its own leg
                      order, blocks in sorted order.
    values 'normal' : N(0,1) entries;
    values 'identity': E = identity, W = identity on the local space (needs w = 1),
                      A left-orthonormal per b-sector (QR of a Gaussian matrix);
    values 'int'    : integer entries in {-1, 0, 1} for E, A and W, so every
                      product and partial sum of the three stages is an integer
                      (exact in fp32 while its magnitude stays below 2^24).
    """
    bond_q = np.asarray(bond_q, np.int64)
    local_q = np.asarray(local_q, np.int64).reshape(len(local_q), -1)
    mpo_q = np.asarray(mpo_q, np.int64).reshape(len(mpo_q), -1)
    nq = bond_q.shape[1]
    S, d, w = len(bond_dim), len(local_q), len(mpo_q)
    D = np.asarray(bond_dim, np.int64)
    sec = {tuple(bond_q[i]): i for i in range(S)}
    tq = lambda v: tuple(int(x) for x in v)
    fdt = np.float64 if dtype == "f64" else np.float32

    # --- tensor block lists -------------------------------------------------
    E_blocks = [(a, ww, ap) for a in range(S) for ww in range(w) for ap in range(S)
                if tq(bond_q[a]) == tq(mpo_q[ww] + bond_q[ap])]
    A_blocks = [(a, s, b) for a in range(S) for s in range(d) for b in range(S)
                if tq(bond_q[b]) == tq(bond_q[a] + local_q[s])]
    W_elems = [(ww, s, sp, wp) for ww in range(w) for s in range(d) for sp in range(d) for wp in range(w)
               if (ww, wp) in set(map(tuple, mpo_pairs)) and tq(mpo_q[ww] + local_q[s]) == tq(local_q[sp] + mpo_q[wp])]

    # --- values ---------------------------------------------------------------
    Ev, Av, Wv = {}, {}, {}
    if values == "normal":
        for (a, ww, ap) in E_blocks:
            Ev[(a, ww, ap)] = rng.standard_normal((D[a], D[ap]))
        for (a, s, b) in A_blocks:
            Av[(a, s, b)] = rng.standard_normal((D[a], D[b]))
        for e in W_elems:
            Wv[e] = rng.standard_normal()
    elif values == "int":
        for (a, ww, ap) in E_blocks:
            Ev[(a, ww, ap)] = rng.integers(-1, 2, (D[a], D[ap])).astype(np.float64)
        for (a, s, b) in A_blocks:
            Av[(a, s, b)] = rng.integers(-1, 2, (D[a], D[b])).astype(np.float64)
        for e in W_elems:
            Wv[e] = float(rng.integers(-1, 2))
    elif values == "identity":
        if w != 1:
            raise ValueError("identity values need an MPO bond of dimension 1")
        for (a, ww, ap) in E_blocks:
            Ev[(a, ww, ap)] = np.eye(D[a]) if a == ap else np.zeros((D[a], D[ap]))
        for e in W_elems:
            Wv[e] = 1.0 if e[1] == e[2] else 0.0
        for b in range(S):
            rows = [(a, s) for (a, s, bb) in A_blocks if bb == b]
            R = int(sum(D[a] for a, _ in rows))
            if R < D[b]:
                raise ValueError("bond sector too large for a left-orthonormal A")
            Q, _ = np.linalg.qr(rng.standard_normal((R, D[b])))
            r0 = 0
            for (a, s) in rows:
                Av[(a, s, b)] = Q[r0:r0 + D[a]]
                r0 += D[a]
    else:
        raise ValueError(values)
    Ev = {kk: v.astype(fdt) for kk, v in Ev.items()}
    Av = {kk: v.astype(fdt) for kk, v in Av.items()}
    Wv = {kk: fdt(v) for kk, v in Wv.items()}

    # --- stage indices ----------------------------------------------------------
    # stage 1: m=(w,a'), k=a, n=(s,b)
    m1 = [(ww, ap) for ww in range(w) for ap in range(S)]
    m1_id = {key: i for i, key in enumerate(m1)}
    n1 = [(s, b) for s in range(d) for b in range(S)]
    n1_id = {key: i for i, key in enumerate(n1)}
    idx_m1 = Index(np.array([mpo_q[ww] + bond_q[ap] for ww, ap in m1]), [D[ap] for _, ap in m1], labels=m1)
    idx_k1 = Index(bond_q, D)
    idx_n1 = Index(np.array([bond_q[b] - local_q[s] for s, b in n1]), [D[b] for _, b in n1], labels=n1)
    T1_keys = sorted({(m1_id[(ww, ap)], n1_id[(s, b)])
                      for (a, ww, ap) in E_blocks for (a2, s, b) in A_blocks if a2 == a})
    T1_blocks = [(m1[mi][0], m1[mi][1], n1[ni][0], n1[ni][1]) for mi, ni in T1_keys]  # (w,a',s,b)

    # stage 2: m=(a',b), k=(w,s), n=(s',w')
    m2 = sorted({(ap, b) for (_, ap, _, b) in T1_blocks})
    m2_id = {key: i for i, key in enumerate(m2)}
    k2 = [(ww, s) for ww in range(w) for s in range(d)]
    k2_id = {key: i for i, key in enumerate(k2)}
    n2 = [(sp, wp) for sp in range(d) for wp in range(w)]
    n2_id = {key: i for i, key in enumerate(n2)}
    idx_m2 = Index(np.array([bond_q[ap] - bond_q[b] for ap, b in m2]).reshape(len(m2), nq),
                   [D[ap] * D[b] for ap, b in m2], inner=[D[b] for _, b in m2], labels=m2)
    idx_k2 = Index(np.array([-(mpo_q[ww] + local_q[s]) for ww, s in k2]), np.ones(len(k2), np.int64), labels=k2)
    idx_n2 = Index(np.array([-(local_q[sp] + mpo_q[wp]) for sp, wp in n2]), np.ones(len(n2), np.int64), labels=n2)
    T2_keys = sorted({(m2_id[(ap, b)], n2_id[(sp, wp)])
                      for (ww, ap, s, b) in T1_blocks for (w2, s2, sp, wp) in W_elems if (w2, s2) == (ww, s)})
    T2_blocks = [(m2[mi][0], m2[mi][1], n2[ni][0], n2[ni][1]) for mi, ni in T2_keys]  # (a',b,s',w')

    # stage 3: m=(b,w'), k=(a',s'), n=b'
    m3 = sorted({(b, wp) for (_, b, _, wp) in T2_blocks})
    m3_id = {key: i for i, key in enumerate(m3)}
    k3 = [(ap, sp) for ap in range(S) for sp in range(d)]
    k3_id = {key: i for i, key in enumerate(k3)}
    idx_m3 = Index(np.array([bond_q[b] - mpo_q[wp] for b, wp in m3]).reshape(len(m3), nq), [D[b] for b, _ in m3], labels=m3)
    idx_k3 = Index(np.array([bond_q[ap] + local_q[sp] for ap, sp in k3]), [D[ap] for ap, _ in k3], labels=k3)
    idx_n3 = Index(bond_q, D)
    Ep_keys = sorted({(m3_id[(b, wp)], bp)
                      for (ap, b, sp, wp) in T2_blocks for (a, s, bp) in A_blocks if (a, s) == (ap, sp)})
    Ep_blocks = [(m3[mi][0], m3[mi][1], bp) for mi, bp in Ep_keys]  # (b,w',b')

    # --- storage ----------------------------------------------------------------
    # per-tensor maps: block -> (offset, row stride, col stride) of the block as a
    # (first-leg-group x second-leg-group) matrix in the tensor's own leg order
    Eloc, Aloc, Wloc, T1loc, T2loc, Eploc = {}, {}, {}, {}, {}, {}
    if layout == "coop":
        ar = Arena()
        for a in range(S):   # E per a-sector: D_a x [(w,a') in m1 order]
            cols = [(ww, ap) for (ww, ap) in m1 if (a, ww, ap) in Ev]
            ld = round_up(sum(D[ap] for _, ap in cols), ld_align)
            base = ar.take(D[a] * ld)
            c0 = 0
            for (ww, ap) in cols:
                Eloc[(a, ww, ap)] = (base + c0, ld, 1)
                c0 += D[ap]
        nE = ar.top
        ar = Arena()
        for b in range(S):   # A per b-sector: [(a,s) in k3 order] x D_b
            rows = [(a, s) for (a, s) in k3 if (a, s, b) in Av]
            ld = round_up(D[b], ld_align)
            base = ar.take(sum(D[a] for a, _ in rows) * ld)
            r0 = 0
            for (a, s) in rows:
                Aloc[(a, s, b)] = (base + r0 * ld, ld, 1)
                r0 += D[a]
        nA = ar.top
        ar = Arena()
        T1_by_pair: Dict[Tuple[int, int], list] = {}
        for (ww, ap, s, b) in T1_blocks:
            T1_by_pair.setdefault((ap, b), []).append((ww, s))
        for (ap, b) in sorted(T1_by_pair):   # per (a',b): [(w,s) slot][D_a'][D_b]
            slots = sorted(T1_by_pair[(ap, b)], key=lambda t: k2_id[t])
            ld = round_up(D[b], ld_align)
            base = ar.take(len(slots) * D[ap] * ld)
            for i, (ww, s) in enumerate(slots):
                T1loc[(ww, ap, s, b)] = (base + i * D[ap] * ld, ld, 1)
        nT1 = ar.top
        ar = Arena()
        T2_by_row: Dict[Tuple[int, int], list] = {}
        for (ap, b, sp, wp) in T2_blocks:
            T2_by_row.setdefault((b, wp), []).append((ap, sp))
        for (b, wp) in sorted(T2_by_row):    # per (b,w'): D_b x [(a',s') in k3 order]
            cols = sorted(T2_by_row[(b, wp)], key=lambda t: k3_id[t])
            ld = round_up(sum(D[ap] for ap, _ in cols), ld_align)
            base = ar.take(D[b] * ld)
            c0 = 0
            for (ap, sp) in cols:
                # T2[a',b,s',w'] as an (a' x b) block: a' along columns (stride 1), b along rows (stride ld)
                T2loc[(ap, b, sp, wp)] = (base + c0, 1, ld)
                c0 += D[ap]
        nT2 = ar.top
        ar = Arena()
        Ep_by_b: Dict[int, list] = {}
        for (b, wp, bp) in Ep_blocks:
            Ep_by_b.setdefault(b, []).append((wp, bp))
        for b in sorted(Ep_by_b):           # E' per b-sector: D_b x [(w',b') in order]
            cols = sorted(Ep_by_b[b])
            ld = round_up(sum(D[bp] for _, bp in cols), ld_align)
            base = ar.take(D[b] * ld)
            c0 = 0
            for (wp, bp) in cols:
                Eploc[(b, wp, bp)] = (base + c0, ld, 1)
                c0 += D[bp]
        nEp = ar.top
    elif layout == "natural":
        def nat(keys, rdim, cdim):
            ar, loc = Arena(), {}
            for key in sorted(keys):
                R, C = int(rdim(key)), int(cdim(key))
                ld = round_up(C, ld_align)
                loc[key] = (ar.take(R * ld), ld, 1)
            return loc, ar.top
        Eloc, nE = nat(Ev.keys(), lambda t: D[t[0]], lambda t: D[t[2]])
        Aloc, nA = nat(Av.keys(), lambda t: D[t[0]], lambda t: D[t[2]])
        T1loc, nT1 = nat(T1_blocks, lambda t: D[t[1]], lambda t: D[t[3]])
        T2loc, nT2 = nat(T2_blocks, lambda t: D[t[0]], lambda t: D[t[1]])
        Eploc, nEp = nat(Ep_blocks, lambda t: D[t[0]], lambda t: D[t[2]])
    else:
        raise ValueError(layout)
    for i, e in enumerate(W_elems):
        Wloc[e] = i
    nW = len(W_elems)

    # --- buffers with values ----------------------------------------------------
    Ebuf = np.zeros(nE, fdt)
    for key, v in Ev.items():
        off, rs, cs = Eloc[key]
        write_block(Ebuf, off, (rs, 0), (cs, 0), v)
    Abuf = np.zeros(nA, fdt)
    for key, v in Av.items():
        off, rs, cs = Aloc[key]
        write_block(Abuf, off, (rs, 0), (cs, 0), v)
    Wbuf = np.zeros(nW, fdt)
    for key, v in Wv.items():
        Wbuf[Wloc[key]] = v

    # --- stage operands -----------------------------------------------------------
    zero = [0] * nq
    # stage 1: A-op = E^T over ((w,a'), a); B-op = A over (a, (s,b)); C = T1
    s1A = [(m1_id[(ww, ap)], a, Eloc[(a, ww, ap)][0], (Eloc[(a, ww, ap)][2], 0), (Eloc[(a, ww, ap)][1], 0))
           for (a, ww, ap) in sorted(E_blocks, key=lambda t: (m1_id[(t[1], t[2])], t[0]))]
    s1B = [(a, n1_id[(s, b)], Aloc[(a, s, b)][0], (Aloc[(a, s, b)][1], 0), (Aloc[(a, s, b)][2], 0))
           for (a, s, b) in sorted(A_blocks, key=lambda t: (t[0], n1_id[(t[1], t[2])]))]
    s1C = [(m1_id[(ww, ap)], n1_id[(s, b)], T1loc[(ww, ap, s, b)][0], (T1loc[(ww, ap, s, b)][1], 0),
            (T1loc[(ww, ap, s, b)][2], 0)) for (ww, ap, s, b) in T1_blocks]
    st1 = Contraction(idx_m1, idx_k1, idx_n1, _operand(s1A, zero, nq, nE), _operand(s1B, zero, nq, nA),
                      _operand(s1C, zero, nq, nT1), dtype)
    # stage 2: A-op = T1 over ((a',b), (w,s)) with two-leg rows (a' outer, b inner)
    s2A = sorted([(m2_id[(ap, b)], k2_id[(ww, s)], T1loc[(ww, ap, s, b)][0],
                   (T1loc[(ww, ap, s, b)][1], T1loc[(ww, ap, s, b)][2]), (1, 0))
                  for (ww, ap, s, b) in T1_blocks], key=lambda t: (t[0], t[1]))
    s2B = sorted([(k2_id[(ww, s)], n2_id[(sp, wp)], Wloc[(ww, s, sp, wp)], (1, 0), (1, 0))
                  for (ww, s, sp, wp) in W_elems], key=lambda t: (t[0], t[1]))
    s2C = [(m2_id[(ap, b)], n2_id[(sp, wp)], T2loc[(ap, b, sp, wp)][0],
            (T2loc[(ap, b, sp, wp)][1], T2loc[(ap, b, sp, wp)][2]), (1, 0)) for (ap, b, sp, wp) in T2_blocks]
    st2 = Contraction(idx_m2, idx_k2, idx_n2, _operand(s2A, zero, nq, nT1), _operand(s2B, zero, nq, nW),
                      _operand(s2C, zero, nq, nT2), dtype)
    # stage 3: A-op = T2 over ((b,w'), (a',s')): rows b, cols a'; B-op = A over ((a,s), b')
    s3A = sorted([(m3_id[(b, wp)], k3_id[(ap, sp)], T2loc[(ap, b, sp, wp)][0],
                   (T2loc[(ap, b, sp, wp)][2], 0), (T2loc[(ap, b, sp, wp)][1], 0))
                  for (ap, b, sp, wp) in T2_blocks], key=lambda t: (t[0], t[1]))
    s3B = sorted([(k3_id[(a, s)], bp, Aloc[(a, s, bp)][0], (Aloc[(a, s, bp)][1], 0), (Aloc[(a, s, bp)][2], 0))
                  for (a, s, bp) in A_blocks], key=lambda t: (t[0], t[1]))
    s3C = [(m3_id[(b, wp)], bp, Eploc[(b, wp, bp)][0], (Eploc[(b, wp, bp)][1], 0), (Eploc[(b, wp, bp)][2], 0))
           for (b, wp, bp) in Ep_blocks]
    st3 = Contraction(idx_m3, idx_k3, idx_n3, _operand(s3A, zero, nq, nT2), _operand(s3B, zero, nq, nA),
                      _operand(s3C, zero, nq, nEp), dtype)

    stages = [Stage(st1, "E", "A", "T1", "E^T A"), Stage(st2, "T1", "W", "T2", "T1 W"),
              Stage(st3, "T2", "A", "Ep", "T2 A*")]
    sizes = {"E": nE, "A": nA, "W": nW, "T1": nT1, "T2": nT2, "Ep": nEp}
    info = {"D": D, "bond_q": bond_q, "local_q": local_q, "mpo_q": mpo_q,
            "E": Ev, "A": Av, "W": Wv, "Ep_blocks": Ep_blocks, "Ep_loc": Eploc, "layout": layout}
    return Chain(name, stages, {"E": Ebuf, "A": Abuf, "W": Wbuf}, sizes, dtype, info)


U1_MPO_PAIRS = [(0, 0), (0, 1), (0, 2), (0, 3), (0, 4), (1, 4), (2, 4), (3, 4), (4, 4), (1, 1), (2, 2), (3, 3)]
U1U1_MPO_PAIRS = [(0, j) for j in range(6)] + [(i, 5) for i in range(1, 5)] + [(5, 5)]


def rabc_u1(seed: int = 1003, layout: str = "coop", values: str = "normal") -> Chain:
    """U(1) spin-chain environment update, fp64: bond m=1024 over 41 sectors
    (Gaussian dims, sigma = 6 sectors), LocalSpace d=4 with charges {-1,0,0,+1},
    MPO bond w=5 with 12 nonzero channel pairs."""
    rng = np.random.default_rng(seed)
    bq, bd = _bond_u1(1024, 20, 6.0)
    local = np.array([[-1], [0], [0], [1]])
    mpo = np.array([[0], [-1], [1], [0], [0]])
    return rabc_chain(bq, bd, local, mpo, U1_MPO_PAIRS, "f64", rng, layout, values,
                      name=f"rabc_u1-{layout}" + ("" if values == "normal" else f"-{values}"))


def rabc_u1u1(seed: int = 1004, layout: str = "natural", values: str = "normal") -> Chain:
    """U(1)xU(1) environment update, fp32: bond m=4096 over the populated part of
    a 15x15 charge grid (Gaussian dims, sigma 2.2 -> 177 sectors), local charges
    (n_up, n_dn), Hubbard-shaped MPO w=6 with 11 nonzero channel pairs."""
    rng = np.random.default_rng(seed)
    bq, bd = _bond_u1u1(4096, 7, 2.2, 0.5)
    local = np.array([[0, 0], [1, 0], [0, 1], [1, 1]])
    mpo = np.array([[0, 0], [-1, 0], [1, 0], [0, -1], [0, 1], [0, 0]])
    return rabc_chain(bq, bd, local, mpo, U1U1_MPO_PAIRS, "f32", rng, layout, values,
                      name=f"rabc_u1u1-{layout}" + ("" if values == "normal" else f"-{values}"))


def small_chain(seed: int = 7, layout: str = "coop", values: str = "normal", dtype: str = "f64",
                total: int = 64, qmax: int = 4, sigma: float = 2.0, w: int = 5) -> Chain:
    """A small R/A/B/C chain (bond ~64) for dense cross-checks."""
    rng = np.random.default_rng(seed)
    bq, bd = _bond_u1(total, qmax, sigma)
    local = np.array([[-1], [0], [0], [1]])
    if w == 5:
        mpo, pairs = np.array([[0], [-1], [1], [0], [0]]), U1_MPO_PAIRS
    elif w == 1:
        mpo, pairs = np.array([[0]]), [(0, 0)]
    else:
        raise ValueError(w)
    return rabc_chain(bq, bd, local, mpo, pairs, dtype, rng, layout, values, name=f"small-{layout}-{values}")


def neutral_chain(seed: int = 9, dims=(3, 37, 17, 40), layout: str = "natural", values: str = "int",
                  dtype: str = "f64", d: int = 4) -> Chain:
    """An environment-update chain whose charges are all zero, so every pair of
    blocks meets: several products per stage-1 block (one per bond sector),
    stage-2 rows of d x w stage-1 blocks and up to d x w outputs (w = 5, the
    U(1) MPO pairs), bond dims across several 16-wide tiles and 32-long chunks."""
    rng = np.random.default_rng(seed)
    bq = np.zeros((len(dims), 1), np.int64)
    local = np.zeros((d, 1), np.int64)
    mpo = np.zeros((5, 1), np.int64)
    return rabc_chain(bq, list(dims), local, mpo, U1_MPO_PAIRS, dtype, rng, layout, values,
                      name=f"neutral-{layout}-{values}")


# ----------------------------------------------------------------------------
# random structures for property tests
# ----------------------------------------------------------------------------

def random_problem(seed: int, nq: int = 1, nkeys=(4, 4, 4), maxdim: int = 12, qrange: int = 2,
                   dtype: str = "f64", flux=(0, 0), density: float = 1.0, two_leg: bool = True,
                   scatter: bool = True, int_values: bool = False, dup_charges: bool = True) -> Problem:
    """Random sector structure with random strided block layouts.

    Keys get random charges in [-qrange, qrange]^nq (repeats allowed), random dims
    1..maxdim and, with two_leg, sometimes an inner-leg extent.  Every
    charge-allowed block is present with probability `density` (C gets every
    allowed block).  With `scatter`, each block is stored as a 4-d array
    [outer_r, inner_r, outer_c, inner_c] in a random axis order, with random
    padding and random block order in the buffer.  int_values draws integers in
    {-2..2} (exact in every dtype)."""
    rng = np.random.default_rng(seed)
    fa = np.array(flux[0], np.int64).reshape(-1)
    fb = np.array(flux[1], np.int64).reshape(-1)
    if fa.size == 1:
        fa = np.repeat(fa, nq)
    if fb.size == 1:
        fb = np.repeat(fb, nq)

    def mk_index(nk):
        ch = rng.integers(-qrange, qrange + 1, (nk, nq))
        if not dup_charges:
            ch = np.unique(ch, axis=0)
            nk = len(ch)
        dims = rng.integers(1, maxdim + 1, nk)
        inner = np.ones(nk, np.int64)
        if two_leg:
            for i in range(nk):
                if rng.random() < 0.4:
                    ii = int(rng.integers(1, 4))
                    oo = int(rng.integers(1, 4))
                    inner[i] = ii
                    dims[i] = ii * oo
        return Index(ch, dims, inner if two_leg else None)

    m, k, n = mk_index(nkeys[0]), mk_index(nkeys[1]), mk_index(nkeys[2])
    allowed = lambda ri, ci, f: np.array_equal(ri - ci, f)
    a_pairs = [(i, j) for i in range(m.nkeys) for j in range(k.nkeys)
               if allowed(m.charge[i], k.charge[j], fa) and rng.random() < density]
    b_pairs = [(i, j) for i in range(k.nkeys) for j in range(n.nkeys)
               if allowed(k.charge[i], n.charge[j], fb) and rng.random() < density]
    c_pairs = [(i, j) for i in range(m.nkeys) for j in range(n.nkeys) if allowed(m.charge[i], n.charge[j], fa + fb)]

    def place(pairs, ri_idx, ci_idx):
        ar = Arena()
        order = list(range(len(pairs)))
        if scatter:
            rng.shuffle(order)
        loc = [None] * len(pairs)
        for p in order:
            r, c = pairs[p]
            R, C = int(ri_idx.dim[r]), int(ci_idx.dim[c])
            Ri, Ci = ri_idx.inner_of(r), ci_idx.inner_of(c)
            ext = [R // Ri, Ri, C // Ci, Ci]   # legs: outer_r, inner_r, outer_c, inner_c
            axes = list(range(4))
            if scatter:
                rng.shuffle(axes)
            pad = int(rng.integers(0, 3)) if scatter else 0
            strides = [0] * 4
            st = 1
            for ax in reversed(axes):      # last axis in `axes` is fastest
                strides[ax] = st
                st *= ext[ax] + (pad if ax == axes[0] else 0)
            size = st
            off = ar.take(size + (int(rng.integers(0, 3)) if scatter else 0))
            # strides must be >= 1 even along unit extents
            strides = [max(1, s) for s in strides]
            loc[p] = (r, c, off, (strides[0], strides[1]), (strides[2], strides[3]))
        return loc, ar.top

    Ab, na = place(a_pairs, m, k)
    Bb, nb = place(b_pairs, k, n)
    Cb, nc = place(c_pairs, m, n)
    fdt = np.float64 if dtype == "f64" else np.float32
    if int_values:
        draw = lambda s: rng.integers(-2, 3, s).astype(fdt)
    elif dtype == "bf16":
        draw = lambda s: bf16_round(rng.standard_normal(s).astype(np.float32))
    else:
        draw = lambda s: rng.standard_normal(s).astype(fdt)
    a = np.zeros(na, fdt)
    b = np.zeros(nb, fdt)
    _fill(a, Ab, m.dim, k.dim, draw, m.inner, k.inner)
    _fill(b, Bb, k.dim, n.dim, draw, k.inner, n.inner)
    con = Contraction(m, k, n, _operand(Ab, fa, nq, na), _operand(Bb, fb, nq, nb),
                      _operand(Cb, fa + fb, nq, nc), dtype)
    return Problem(f"random-{seed}", con, a, b, {})
