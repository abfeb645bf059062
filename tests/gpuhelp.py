"""Helpers for the GPU parity tests: move seeded inputs to the device, run the
engine through the C-ABI binding, and compare with the oracle over the union of
C blocks (relative Frobenius error in float64)."""
import numpy as np

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


def c_addresses(con):
    """Addresses of every element of every C block (concatenated) and a mask."""
    parts = []
    for i in range(con.C.nblocks):
        r, c = int(con.C.row_key[i]), int(con.C.col_key[i])
        ri = 1 if con.m.inner is None else int(con.m.inner[r])
        ci = 1 if con.n.inner is None else int(con.n.inner[c])
        parts.append(view_addresses(con.C.offset[i], con.C.row_stride[i], con.C.col_stride[i],
                                    int(con.m.dim[r]), int(con.n.dim[c]), ri, ci).ravel())
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


def canary(con, dtype):
    c = np.full(con.C.buffer_elems, np.nan, dtype=c_dtype(dtype))
    return c


def check_canary(got, mask):
    """Elements outside every C view still hold the NaN canary; views are finite."""
    assert np.all(np.isnan(got[~mask])), "a write landed outside the C views"
    assert np.all(np.isfinite(got[mask])), "a C view element was not written"
