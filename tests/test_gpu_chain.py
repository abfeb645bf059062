"""Captured chains: a sequence of contractions recorded once into a HIP graph
and replayed with one launch (bsc_chain_*).  Every replay must equal the same
sequence run launch by launch, bit for bit (same kernels, same order), also
with eager GPU work and host synchronisation between replays, with gathers,
K-split tiles (whose counters the kernels reset) and accumulation."""
import numpy as np
import pytest

import oracle
from workloads import configs as C

from gpuhelp import c_addresses, check_float, have_gpu, rel_frobenius, to_dev, torch

pytestmark = pytest.mark.gpu

if have_gpu():
    import block_sparse_tensor_amd as bst
else:
    bst = None


def _chain_buffers(ch):
    t = torch()
    cdt = {"f64": t.float64, "f32": t.float32}[ch.dtype]
    bufs = {k: to_dev(v, ch.dtype) for k, v in ch.buffers.items()}
    for name, n in ch.sizes.items():
        if name not in bufs:
            bufs[name] = t.zeros(n, dtype=cdt, device="cuda")
    return bufs


@pytest.mark.parametrize("layout", ["auto", "force_pack"])
def test_chain_replays_match_eager(layout):
    """The small environment-update chain: eager run, then a captured chain over
    copies of the same buffers replayed three times with eager work between."""
    t = torch()
    ch = C.small_chain(seed=3, layout="natural")
    ref = oracle.run_chain(ch)
    plans = [bst.Plan(st.con, layout=layout).bind() for st in ch.stages]
    eager = _chain_buffers(ch)
    for p, st in zip(plans, ch.stages):
        p.contract(eager[st.a_buf], eager[st.b_buf], eager[st.c_buf])
    t.cuda.synchronize()
    for st in ch.stages:
        check_float(st.con, eager[st.c_buf].cpu().numpy(), ref[st.c_buf], ref[st.a_buf], ref[st.b_buf], 1e-12,
                    label=st.label)
    g = _chain_buffers(ch)
    chain = bst.Chain([(p, g[st.a_buf], g[st.b_buf], g[st.c_buf]) for p, st in zip(plans, ch.stages)])
    for r in range(3):
        print(f"[chain] small chain layout={layout} replay {r}", flush=True)
        for st in ch.stages:                      # outputs cleared by eager work between replays
            g[st.c_buf].zero_()
        x = t.randn(1 << 16, device="cuda")
        (x * 2.0).sum().item()                    # eager work and a host synchronisation
        chain.launch()
        t.cuda.synchronize()
        for st in ch.stages:
            assert t.equal(g[st.c_buf], eager[st.c_buf]), (r, st.label)


def test_chain_rabc_u1_full_size():
    """The full U(1) environment update (three stages, gathers) as one graph."""
    t = torch()
    ch = C.rabc_u1()
    plans = [bst.Plan(st.con).bind() for st in ch.stages]
    eager = _chain_buffers(ch)
    for p, st in zip(plans, ch.stages):
        p.contract(eager[st.a_buf], eager[st.b_buf], eager[st.c_buf])
    g = _chain_buffers(ch)
    chain = bst.Chain([(p, g[st.a_buf], g[st.b_buf], g[st.c_buf]) for p, st in zip(plans, ch.stages)])
    for r in range(2):
        print(f"[chain] rabc_u1 replay {r}", flush=True)
        chain.launch()
        t.cuda.synchronize()
        for st in ch.stages:
            assert t.equal(g[st.c_buf], eager[st.c_buf]), (r, st.label)


def test_chain_split_k_and_accumulate():
    """bf16 block-diagonal workload with every long tile split along K, in
    accumulate mode: n replays add n products, bit-identical to n eager calls."""
    t = torch()
    prob = C.blockdiag_bf16(ld_align=8, align=8)
    con = prob.con
    plan = bst.Plan(con, split_k=8, accumulate=True).bind()
    assert plan.stats()["split_tiles"] > 0
    A, B = to_dev(prob.a, "bf16"), to_dev(prob.b, "bf16")
    ce = t.zeros(con.C.buffer_elems, dtype=t.float32, device="cuda")
    cg = t.zeros_like(ce)
    chain = bst.Chain([(plan, A, B, cg)])
    for r in range(3):
        print(f"[chain] blockdiag_bf16 split accumulate replay {r}", flush=True)
        plan.contract(A, B, ce)
        t.cuda.synchronize()
        chain.launch()
        t.cuda.synchronize()
        assert t.equal(cg, ce), r
    addr, _ = c_addresses(con)
    ref = oracle.contract(con, prob.a, prob.b, np.zeros(con.C.buffer_elems), check=False)
    assert rel_frobenius(cg.cpu().numpy() / 3.0, ref, addr) <= 2e-2


def test_chain_errors():
    ch = C.small_chain(seed=3, layout="natural")
    st = ch.stages[0]
    p = bst.Plan(st.con)                          # not bound
    g = _chain_buffers(ch)
    with pytest.raises(bst.BscError) as e:
        bst.Chain([(p, g[st.a_buf], g[st.b_buf], g[st.c_buf])])
    assert e.value.status == -8
    with pytest.raises(bst.BscError):
        bst.Chain([])


def test_chain_checks_tensors_and_guards_rebind():
    """A chain rejects operand tensors that contract() would reject (the graph
    would replay their addresses unchecked), and a captured plan refuses to be
    rebound until the chain is released."""
    t = torch()
    ch = C.small_chain(seed=3, layout="natural")
    st = ch.stages[0]
    p = bst.Plan(st.con).bind()
    g = _chain_buffers(ch)
    small = t.zeros(max(1, p.c_elems // 2), dtype=g[st.c_buf].dtype, device="cuda")
    with pytest.raises(ValueError):
        bst.Chain([(p, g[st.a_buf], g[st.b_buf], small)])
    with pytest.raises(TypeError):
        bst.Chain([(p, g[st.a_buf].float(), g[st.b_buf], g[st.c_buf])])
    assert p._captured == 0
    chain = bst.Chain([(p, g[st.a_buf], g[st.b_buf], g[st.c_buf])])
    with pytest.raises(bst.BscError):
        p.bind()
    print("[chain] replay before release", flush=True)
    chain.launch()
    t.cuda.synchronize()
    chain.release()
    p.bind()                                      # allowed again
    p.contract(g[st.a_buf], g[st.b_buf], g[st.c_buf])
    t.cuda.synchronize()


def test_probe_mfma_measures_a_rate():
    """bsc_probe_mfma: a launch of known flops whose measured rate is positive
    and below the published peak of its instruction."""
    t = torch()
    sink = t.zeros(1, dtype=t.float32, device="cuda")
    spec = {"bf16": 2516.6e12, "f32": 157.3e12, "f64": 78.6e12}
    for dt, iters in (("bf16", 200), ("f32", 100), ("f64", 50)):
        bst.probe_mfma(dt, iters, sink)
        t.cuda.synchronize()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record()
        flops = bst.probe_mfma(dt, iters, sink)
        e1.record()
        t.cuda.synchronize()
        rate = flops / (e0.elapsed_time(e1) * 1e-3)
        assert flops > 0 and 0.05 * spec[dt] < rate < 1.05 * spec[dt], (dt, rate)
        assert sink.item() == 0.0   # never written
