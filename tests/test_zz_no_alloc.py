"""bsc_contract_noalloc: the contraction with its device region (work list,
pack workspace, K-split partials and counters) in the library's fixed per-GPU
scratch array instead of a bound region.  Same kernels and arithmetic order as
bsc_contract, so results must agree bit for bit; two calls in a row (the
second on a smaller plan) check that each call replaces what the last one left
in the shared array, and a repeat checks the K-split counters start at zero."""
import numpy as np
import pytest

from workloads import configs as C

from gpuhelp import have_gpu, to_dev, torch

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:
    bst = None


def _pair(plan_kw, con, a, b, dtype, bound_plan=None):
    """(bsc_contract result, bsc_contract_noalloc result) on fresh NaN-filled C."""
    t = torch()
    A, B = to_dev(a, dtype), to_dev(b, dtype)
    cdt = t.float64 if dtype == "f64" else t.float32
    ref_plan = bound_plan or bst.Plan(con, **plan_kw).bind()
    c_ref = t.full((con.C.buffer_elems,), float("nan"), dtype=cdt, device="cuda")
    ref_plan.contract(A, B, c_ref)
    free_plan = bst.Plan(con, **plan_kw)          # never bound
    c_free = t.full((con.C.buffer_elems,), float("nan"), dtype=cdt, device="cuda")
    free_plan.contract_noalloc(A, B, c_free)
    t.cuda.synchronize()
    return c_ref.cpu().numpy(), c_free.cpu().numpy(), free_plan, (A, B, c_free)


def _same_bits(x, y):
    return np.array_equal(x.view(np.uint64 if x.dtype == np.float64 else np.uint32),
                          y.view(np.uint64 if y.dtype == np.float64 else np.uint32))


def test_noalloc_matches_bound_two_calls():
    # call 1: the gather-heavy W stage of the U(1)xU(1) update (pack workspace in scratch)
    ch = C.rabc_u1u1()
    st = ch.stages[1]
    t = torch()
    bufs = {k: to_dev(v, ch.dtype) for k, v in ch.buffers.items()}
    for name, n in ch.sizes.items():
        if name not in bufs:
            bufs[name] = t.zeros(n, dtype=t.float32, device="cuda")
    p1 = bst.Plan(ch.stages[0].con).bind()
    p1.contract(bufs["E"], bufs["A"], bufs["T1"])     # the stage's input T1
    t.cuda.synchronize()
    t1 = bufs["T1"].cpu().numpy()
    plan_kw = dict(layout="force_pack")
    big = bst.Plan(st.con, **plan_kw)
    assert big.stats()["pack_bytes"] > 0
    print(f"[noalloc] call 1: W stage, device bytes {big.device_bytes()}", flush=True)
    r1, f1, _, _ = _pair(plan_kw, st.con, t1, ch.buffers["W"], "f32")
    assert _same_bits(r1, f1)
    # call 2: a smaller bf16 plan with K-split tiles (partials and counters in scratch)
    from test_gpu_split import _single
    con, a, b = _single(520, 1000, 260, True, seed=5)
    kw = dict(split_k=8)
    small = bst.Plan(con, **kw)
    assert small.stats()["split_tiles"] > 0 and small.device_bytes() < big.device_bytes()
    print(f"[noalloc] call 2: split bf16 tile, device bytes {small.device_bytes()}", flush=True)
    r2, f2, fp, (A, B, Cf) = _pair(kw, con, a, b, "bf16")
    assert _same_bits(r2, f2)
    # call 3: the same plan again (counters must have been reset by the upload)
    print("[noalloc] call 3: repeat", flush=True)
    Cf.fill_(float("nan"))
    fp.contract_noalloc(A, B, Cf)
    t.cuda.synchronize()
    assert _same_bits(r2, Cf.cpu().numpy())


def test_noalloc_too_large_is_refused():
    """A plan whose device region exceeds the scratch array is refused before
    anything is enqueued."""
    from test_gpu_split import _single
    con, a, b = _single(2048, 30000, 1024, True, seed=3)
    p = bst.Plan(con, split_k=1)                       # slices of 32: many 128 KB partial tiles
    assert p.device_bytes() > 64 << 20
    t = torch()
    A, B = to_dev(a, "bf16"), to_dev(b, "bf16")
    Cd = t.zeros(con.C.buffer_elems, dtype=t.float32, device="cuda")
    with pytest.raises(bst.BscError) as e:
        p.contract_noalloc(A, B, Cd)
    assert e.value.status == -9
