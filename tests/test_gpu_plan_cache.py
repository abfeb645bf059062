"""Plans handed out by the plan cache run on the GPU exactly like freshly
planned ones: a sweep over the small environment-update chain, replanned
through one cache at every visit, gives bit-identical results to the fresh
plans and matches the oracle."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import check_float, have_gpu, to_dev, torch

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:
    bst = None


def _run(plans, ch):
    t = torch()
    cdt = {"f64": t.float64, "f32": t.float32}[ch.dtype]
    bufs = {k: to_dev(v, ch.dtype) for k, v in ch.buffers.items()}
    for name, n in ch.sizes.items():
        if name not in bufs:
            bufs[name] = t.zeros(n, dtype=cdt, device="cuda")
    for p, st in zip(plans, ch.stages):
        p.contract(bufs[st.a_buf], bufs[st.b_buf], bufs[st.c_buf])
    t.cuda.synchronize()
    return {st.c_buf: bufs[st.c_buf].cpu().numpy() for st in ch.stages}


@pytest.mark.parametrize("layout", ["natural", "coop"])
def test_cached_plans_run_like_fresh(layout):
    ch = C.small_chain(seed=5, layout=layout)
    ref = oracle.run_chain(ch)
    fresh = _run([bst.Plan(st.con).bind() for st in ch.stages], ch)
    cache = bst.PlanCache(8)
    for visit in range(3):   # three visits of the same site
        print(f"[cache] small chain layout={layout} visit {visit}", flush=True)
        plans = [bst.Plan(st.con, cache=cache).bind() for st in ch.stages]
        assert all(p.cache_hit for p in plans) == (visit > 0)
        got = _run(plans, ch)
        for st in ch.stages:
            assert np.array_equal(got[st.c_buf], fresh[st.c_buf]), (visit, st.label)
            check_float(st.con, got[st.c_buf], ref[st.c_buf], ref[st.a_buf], ref[st.b_buf], 1e-12, label=st.label)
    assert cache.stats() == {"hits": 2 * len(ch.stages), "misses": len(ch.stages), "entries": len(ch.stages)}
