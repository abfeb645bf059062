"""Reference block-sparse contraction (float64, one sector at a time).

Test infrastructure only; see the package docstring.

Readings taken where the uni20 "block coalescing" note is silent (its tensor
document is not public):
  * charge rule: block (r, c) of operand X may exist iff
    q_row(r) - q_col(c) == flux_X componentwise; a product carries
    flux_A + flux_B;
  * several keys may carry equal charges (individually keyed LocalSpace states,
    section "Interleaved vs contiguous"), so a C block may sum over several k;
  * overwrite mode writes C_mn = sum_k A_mk B_kn and zero for a listed C block
    with no contributing k; accumulate mode adds to what C holds;
  * a product sector absent from C's block list is an error, never dropped;
  * elements of C's buffer outside every listed C block are left unchanged.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np
from numpy.lib.stride_tricks import as_strided


class OracleError(ValueError):
    pass


# --------------------------------------------------------------------------
# reading a block through its strided view
# --------------------------------------------------------------------------

def _inner(index, key):
    return 1 if index.inner is None else int(index.inner[key])


def block(buf: np.ndarray, op, i: int, ridx, cidx) -> np.ndarray:
    """Block i of operand `op` as a float64 (rows x cols) array (a copy).

    Element (r, c) sits at offset + (r//Ri)*rs0 + (r%Ri)*rs1 + (c//Ci)*cs0 + (c%Ci)*cs1:
    the block is the 4-d strided array [R/Ri, Ri, C/Ci, Ci] reshaped to (R, C)."""
    rk, ck = int(op.row_key[i]), int(op.col_key[i])
    R, C = int(ridx.dim[rk]), int(cidx.dim[ck])
    Ri, Ci = _inner(ridx, rk), _inner(cidx, ck)
    rs0, rs1 = (int(x) for x in op.row_stride[i])
    cs0, cs1 = (int(x) for x in op.col_stride[i])
    base = buf[int(op.offset[i]):]
    it = buf.itemsize
    v = as_strided(base, shape=(R // Ri, Ri, C // Ci, Ci),
                   strides=(rs0 * it, rs1 * it, cs0 * it, cs1 * it), writeable=False)
    return np.array(v, dtype=np.float64).reshape(R, C)


def _block_addresses(op, i, ridx, cidx) -> np.ndarray:
    rk, ck = int(op.row_key[i]), int(op.col_key[i])
    R, C = int(ridx.dim[rk]), int(cidx.dim[ck])
    Ri, Ci = _inner(ridx, rk), _inner(cidx, ck)
    rs0, rs1 = (int(x) for x in op.row_stride[i])
    cs0, cs1 = (int(x) for x in op.col_stride[i])
    ro, ri = np.divmod(np.arange(R), Ri)
    co, ci = np.divmod(np.arange(C), Ci)
    return int(op.offset[i]) + (ro * rs0 + ri * rs1)[:, None] + (co * cs0 + ci * cs1)[None, :]


# --------------------------------------------------------------------------
# structure checks
# --------------------------------------------------------------------------

def check_structure(con) -> None:
    """Raise OracleError if the descriptors break a rule the contraction relies on."""
    nq = con.m.nq
    if con.k.nq != nq or con.n.nq != nq:
        raise OracleError("charge arity differs between indices")
    for name, op, ridx, cidx in (("A", con.A, con.m, con.k), ("B", con.B, con.k, con.n), ("C", con.C, con.m, con.n)):
        seen = set()
        for i in range(op.nblocks):
            r, c = int(op.row_key[i]), int(op.col_key[i])
            if not (0 <= r < ridx.nkeys and 0 <= c < cidx.nkeys):
                raise OracleError(f"{name}: block {i} key out of range")
            if (r, c) in seen:
                raise OracleError(f"{name}: duplicate block ({r},{c})")
            seen.add((r, c))
            if not np.array_equal(ridx.charge[r] - cidx.charge[c], op.flux):
                raise OracleError(f"{name}: block ({r},{c}) breaks the charge rule")
            R, Cc = int(ridx.dim[r]), int(cidx.dim[c])
            Ri, Ci = _inner(ridx, r), _inner(cidx, c)
            legs = ((R // Ri, op.row_stride[i][0]), (Ri, op.row_stride[i][1]),
                    (Cc // Ci, op.col_stride[i][0]), (Ci, op.col_stride[i][1]))
            # a leg of extent > 1 needs a stride >= 1; a unit leg's stride is ignored but may not be negative
            if op.offset[i] < 0 or any(s < 0 or (e > 1 and s < 1) for e, s in legs):
                raise OracleError(f"{name}: block {i} has a bad stride or a negative offset")
            if _block_addresses(op, i, ridx, cidx).max() >= op.buffer_elems:
                raise OracleError(f"{name}: block {i} reaches past the buffer")
    if not np.array_equal(con.A.flux + con.B.flux, con.C.flux):
        raise OracleError("flux_C != flux_A + flux_B")
    owner = np.zeros(con.C.buffer_elems, dtype=np.int32)
    for i in range(con.C.nblocks):
        addr = _block_addresses(con.C, i, con.m, con.n).ravel()
        if len(np.unique(addr)) != addr.size:
            raise OracleError(f"C: block {i} aliases itself")
        owner[addr] += 1
    if np.any(owner > 1):
        raise OracleError("C: blocks overlap")


# --------------------------------------------------------------------------
# the sector join and the contraction itself
# --------------------------------------------------------------------------

def _maps(con):
    a = {(int(r), int(c)): i for i, (r, c) in enumerate(zip(con.A.row_key, con.A.col_key))}
    b = {(int(r), int(c)): i for i, (r, c) in enumerate(zip(con.B.row_key, con.B.col_key))}
    c = {(int(r), int(cc)): i for i, (r, cc) in enumerate(zip(con.C.row_key, con.C.col_key))}
    return a, b, c


def triples(con) -> np.ndarray:
    """All (m, k, n) with an A block (m,k) and a B block (k,n), sorted by (m, n, k).
    Raises OracleError if a product sector (m, n) is absent from C."""
    a, b, c = _maps(con)
    b_by_row: Dict[int, List[int]] = {}
    for (k, n) in b:
        b_by_row.setdefault(k, []).append(n)
    out = []
    for (m, k) in a:
        for n in b_by_row.get(k, ()):
            if (m, n) not in c:
                raise OracleError(f"product sector ({m},{n}) missing from C")
            out.append((m, k, n))
    out.sort(key=lambda t: (t[0], t[2], t[1]))
    return np.array(out, dtype=np.int64).reshape(-1, 3)


def useful_flops(con) -> int:
    t = triples(con)
    return int(sum(2 * int(con.m.dim[m]) * int(con.k.dim[k]) * int(con.n.dim[n]) for m, k, n in t))


def algorithmic_bytes(con) -> int:
    """Every A and B block read once, every C block written once."""
    ab = 8 if con.dtype == "f64" else (2 if con.dtype == "bf16" else 4)
    cb = 8 if con.dtype == "f64" else 4
    na = sum(int(con.m.dim[r]) * int(con.k.dim[c]) for r, c in zip(con.A.row_key, con.A.col_key))
    nb = sum(int(con.k.dim[r]) * int(con.n.dim[c]) for r, c in zip(con.B.row_key, con.B.col_key))
    nc = sum(int(con.m.dim[r]) * int(con.n.dim[c]) for r, c in zip(con.C.row_key, con.C.col_key))
    return ab * (na + nb) + cb * nc


def contract(con, a: np.ndarray, b: np.ndarray, c: np.ndarray = None, accumulate: bool = False,
             check: bool = True) -> np.ndarray:
    """C_mn (+)= sum_{k in L(m,n)} A_mk @ B_kn for every listed C block, float64.

    Returns a float64 copy of `c` (zeros if None) with the listed C blocks
    rewritten through their views; everything else is untouched."""
    if check:
        check_structure(con)
    amap, bmap, _ = _maps(con)
    b_by_row: Dict[int, List[Tuple[int, int]]] = {}
    for (k, n), i in bmap.items():
        b_by_row.setdefault(k, []).append((n, i))
    a_by_row: Dict[int, List[Tuple[int, int]]] = {}
    for (m, k), i in amap.items():
        a_by_row.setdefault(m, []).append((k, i))
    cmap = {(int(r), int(cc)) for r, cc in zip(con.C.row_key, con.C.col_key)}
    for m, lst in a_by_row.items():
        for k, _ in lst:
            for n, _ in b_by_row.get(k, ()):
                if (m, n) not in cmap:
                    raise OracleError(f"product sector ({m},{n}) missing from C")
    out = np.zeros(con.C.buffer_elems) if c is None else np.array(c, dtype=np.float64)
    a64 = np.asarray(a)
    b64 = np.asarray(b)
    for ci in range(con.C.nblocks):
        m, n = int(con.C.row_key[ci]), int(con.C.col_key[ci])
        acc = np.zeros((int(con.m.dim[m]), int(con.n.dim[n])))
        for k, ai in sorted(a_by_row.get(m, ())):
            bi = bmap.get((k, n))
            if bi is None:
                continue
            acc += block(a64, con.A, ai, con.m, con.k) @ block(b64, con.B, bi, con.k, con.n)
        addr = _block_addresses(con.C, ci, con.m, con.n)
        if accumulate:
            acc = acc + out[addr]
        out[addr] = acc
    return out


# --------------------------------------------------------------------------
# dense brute force
# --------------------------------------------------------------------------

def _key_starts(index):
    return np.concatenate([[0], np.cumsum(index.dim)]).astype(np.int64)


def densify(op, buf, ridx, cidx) -> np.ndarray:
    """Zero-filled dense matrix (sum of row dims x sum of col dims), keys in key order."""
    rs, cs = _key_starts(ridx), _key_starts(cidx)
    out = np.zeros((rs[-1], cs[-1]))
    for i in range(op.nblocks):
        r, c = int(op.row_key[i]), int(op.col_key[i])
        out[rs[r]:rs[r + 1], cs[c]:cs[c + 1]] = block(buf, op, i, ridx, cidx)
    return out



# --------------------------------------------------------------------------
# grouping re-derivation (single-axis coalescing rules)
# --------------------------------------------------------------------------

AXIS_NONE, AXIS_FREE_M, AXIS_FREE_N, AXIS_CONTRACT, AXIS_AUTO = 0, 1, 2, 3, 4


def groups(con, axis: int):
    """Single-axis coalescing groups, following the uni20 note's two directions
    (section "Why single-axis coalescing is hole-free"): free-axis grouping stacks
    output blocks that share the other output key and the same contracted-key
    list; contraction-axis grouping concatenates the k-list of one output block.

    Returns (resolved_axis, group_of_triple[T], groups) where groups is a list of
    (rows, cols, klist) tuples of key ids.  Canonical orders:
      NONE     one group per triple, in triple order (m, n, k);
      CONTRACT one group per output block with a non-empty k-list, in (m, n) order;
      FREE_M   members share n and the k-list, stacked by ascending m, groups in
               (n, first m) order;
      FREE_N   members share m and the k-list, stacked by ascending n, groups in
               (m, first n) order;
      AUTO     CONTRACT if more than a quarter of the non-empty output blocks
               have more than one k, else whichever free axis gives fewer groups
               (FREE_M on a tie)."""
    t = triples(con)
    L: Dict[Tuple[int, int], List[int]] = {}
    for m, k, n in t:
        L.setdefault((int(m), int(n)), []).append(int(k))
    for key in L:
        L[key].sort()
    if axis == AXIS_AUTO:
        multi = sum(1 for v in L.values() if len(v) > 1)
        if len(L) and 4 * multi > len(L):
            axis = AXIS_CONTRACT
        else:
            gm = len({(n, tuple(v)) for (m, n), v in L.items()})
            gn = len({(m, tuple(v)) for (m, n), v in L.items()})
            axis = AXIS_FREE_M if gm <= gn else AXIS_FREE_N
    glist = []
    if axis == AXIS_NONE:
        glist = [((int(m),), (int(n),), (int(k),)) for m, k, n in t]
    elif axis == AXIS_CONTRACT:
        glist = [((m,), (n,), tuple(L[(m, n)])) for (m, n) in sorted(L)]
    elif axis == AXIS_FREE_M:
        bucket: Dict = {}
        for (m, n), v in L.items():
            bucket.setdefault((n, tuple(v)), []).append(m)
        glist = sorted(((tuple(sorted(ms)), (n,), kl) for (n, kl), ms in bucket.items()),
                       key=lambda g: (g[1][0], g[0][0]))
    elif axis == AXIS_FREE_N:
        bucket = {}
        for (m, n), v in L.items():
            bucket.setdefault((m, tuple(v)), []).append(n)
        glist = sorted((((m,), tuple(sorted(ns)), kl) for (m, kl), ns in bucket.items()),
                       key=lambda g: (g[0][0], g[1][0]))
    else:
        raise OracleError(f"unknown axis {axis}")
    gid = np.empty(len(t), dtype=np.int64)
    if axis == AXIS_NONE:
        gid[:] = np.arange(len(t))
    else:
        where = {}
        for g, (rows, cols, kl) in enumerate(glist):
            for m in rows:
                for n in cols:
                    where[(m, n)] = g
        for i, (m, k, n) in enumerate(t):
            gid[i] = where[(int(m), int(n))]
    return axis, gid, glist


# --------------------------------------------------------------------------
# chains
# --------------------------------------------------------------------------

def run_chain(chain, accumulate: bool = False) -> Dict[str, np.ndarray]:
    """Run every stage of a Chain in order; returns all buffers as float64."""
    bufs = {k: np.asarray(v, dtype=np.float64) for k, v in chain.buffers.items()}
    for st in chain.stages:
        c0 = bufs.get(st.c_buf)
        if c0 is None:
            c0 = np.zeros(chain.sizes[st.c_buf])
        bufs[st.c_buf] = contract(st.con, bufs[st.a_buf], bufs[st.b_buf], c0, accumulate)
    return bufs
