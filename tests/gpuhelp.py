"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
engine through the C-ABI binding, and compare with the oracle.

Two float checks run on every result:

* the global relative Frobenius error over the union of C blocks, in float64,
  against the dtype tolerance (1e-12 fp64, 1e-5 fp32, 2e-2 bf16 inputs with
  fp32 accumulation);
* a per-C-block check, so that small blocks (tail sectors that hold a
  negligible share of the global norm) cannot hide a wrong result:
  ||C_b - C_ref,b||_F / ||(|A| |B|)_b||_F <= the same tolerance, where
  (|A| |B|)_b is the block computed by the oracle from the absolute values of
  the operands (plus |C0| in accumulate mode).  For a block without
  cancellation this is exactly ||dC_b|| / ||C_ref,b||; with cancellation the
  rounding error of a floating-point dot product is bounded by the magnitudes
  of its terms, sum_k |a_ik| |b_kj| (the standard forward error bound of
  summation, whatever the order), not by the magnitude of the result, so the
  ratio to ||C_ref,b|| alone is not a sound test for fp32.  A wrong block
  (a dropped or foreign term, a wrong sign) scores O(1).  A block whose
  (|A| |B|)_b is all zero must come back exactly zero (or exactly C0).

Integer-valued inputs make every summation order exact, so those compare bit
for bit instead."""
import numpy as np

import oracle
from workloads.layout import view_addresses

TOL = {"f64": 1e-12, "f32": 1e-5, "bf16": 2e-2}


def torch():
    import torch as t
    return t


def have_gpu():
    try:
        import torch as t
        return t.cuda.is_available()
    except Exception:
        return False


def to_dev(x, dtype):
    t = torch()
    if dtype == "f64":
        return t.from_numpy(np.ascontiguousarray(x, np.float64)).cuda()
    if dtype == "f32":
        return t.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    # bf16 inputs: the generator's values are bf16-exact, so the conversion is exact
    return t.from_numpy(np.ascontiguousarray(x, np.float32)).cuda().to(t.bfloat16)


def c_dtype(dtype):
    return np.float64 if dtype == "f64" else np.float32


def block_addresses(con):
    """Per C block, the buffer addresses of its elements (a list of arrays)."""
    out = []
    for i in range(con.C.nblocks):
        r, c = int(con.C.row_key[i]), int(con.C.col_key[i])
        ri = 1 if con.m.inner is None else int(con.m.inner[r])
        ci = 1 if con.n.inner is None else int(con.n.inner[c])
        out.append(view_addresses(con.C.offset[i], con.C.row_stride[i], con.C.col_stride[i],
                                  int(con.m.dim[r]), int(con.n.dim[c]), ri, ci).ravel())
    return out


def c_addresses(con):
    """Addresses of every element of every C block (concatenated) and a mask."""
    parts = block_addresses(con)
    addr = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    mask = np.zeros(con.C.buffer_elems, bool)
    mask[addr] = True
    return addr, mask


def run_engine(plan, a, b, c_init, dtype, repeats=1):
    t = torch()
    A, B = to_dev(a, dtype), to_dev(b, dtype)
    C = t.from_numpy(np.ascontiguousarray(c_init, c_dtype(dtype))).cuda()
    for _ in range(repeats):
        plan.contract(A, B, C)
    t.cuda.synchronize()
    return C.cpu().numpy()


def rel_frobenius(got, ref, addr):
    g = got[addr].astype(np.float64)
    r = ref[addr].astype(np.float64)
    nr = np.linalg.norm(r)
    if nr == 0:
        return 0.0 if np.all(g == 0) else np.inf
    return float(np.linalg.norm(g - r) / nr)


def magnitude_scale(con, a, b, c0=None, accumulate=False):
    """(|A| |B|) (+ |C0| in accumulate mode) through C's views, float64."""
    c_abs = None if c0 is None else np.abs(np.nan_to_num(np.asarray(c0, np.float64)))
    return oracle.contract(con, np.abs(np.asarray(a, np.float64)), np.abs(np.asarray(b, np.float64)),
                           c_abs if accumulate else None, accumulate=accumulate, check=False)


def block_errors(con, got, ref, scale):
    """Per C block: ||got_b - ref_b||_F / ||scale_b||_F (float64).  A block whose
    scale is all zero scores 0 if got equals ref there bit for bit, else inf."""
    errs = np.zeros(con.C.nblocks)
    for i, ad in enumerate(block_addresses(con)):
        g = got[ad].astype(np.float64)
        r = ref[ad].astype(np.float64)
        s = np.linalg.norm(scale[ad])
        if s == 0:
            errs[i] = 0.0 if np.array_equal(g, r) else np.inf
        else:
            errs[i] = np.linalg.norm(g - r) / s
    return errs


def check_blocks(con, got, ref, a, b, tol, c0=None, accumulate=False, label=""):
    """Assert the per-block error (see the module docstring) is within tol."""
    if con.C.nblocks == 0:
        return 0.0
    errs = block_errors(con, got, ref, magnitude_scale(con, a, b, c0, accumulate))
    worst = int(np.argmax(errs))
    assert errs[worst] <= tol, (label, "worst C block", worst, (int(con.C.row_key[worst]), int(con.C.col_key[worst])),
                                float(errs[worst]))
    return float(errs[worst])


def canary(con, dtype):
    c = np.full(con.C.buffer_elems, np.nan, dtype=c_dtype(dtype))
    return c


def check_canary(got, mask):
    """Elements outside every C view still hold the NaN canary; views are finite."""
    assert np.all(np.isnan(got[~mask])), "a write landed outside the C views"
    assert np.all(np.isfinite(got[mask])), "a C view element was not written"


def int_chain_bound(ch):
    """Largest sum_k |a||b| over every stage of an integer-valued chain: while
    it stays below 2^24 every partial sum is an exact fp32 integer."""
    bufs = {k: np.abs(np.asarray(v, np.float64)) for k, v in ch.buffers.items()}
    worst = 0.0
    for st in ch.stages:
        out = oracle.contract(st.con, bufs[st.a_buf], bufs[st.b_buf], np.zeros(ch.sizes[st.c_buf]), check=False)
        bufs[st.c_buf] = out
        worst = max(worst, float(out.max(initial=0.0)))
    return worst


def check_float(con, got, ref, a, b, tol, c0=None, accumulate=False, label=""):
    """Both float checks: the global relative Frobenius error over the union of
    C blocks and the per-block error (see the module docstring)."""
    addr, _ = c_addresses(con)
    err = rel_frobenius(got, ref, addr)
    assert err <= tol, (label, "global", err)
    check_blocks(con, got, ref, a, b, tol, c0=c0, accumulate=accumulate, label=label)
    return err
