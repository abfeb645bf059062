#!/usr/bin/env python3
"""Benchmark: useful GFLOP/s per block-sparse contraction on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload blockdiag_bf16]

A step is one whole contraction (every stage of the workload) over inputs
already resident in HBM.  Useful flops = sum over sector GEMMs of 2*M*N*K (the
work the block structure needs, not a dense equivalent).  Prints ONE JSON line.

Alongside the engine (grouped launches) the same run times:
  * the same contraction from cold caches: each one after a 512 MiB write that
    evicts the chiplet L2s and the 256 MB Infinity Cache;
  * the uncoalesced GPU path: the same kernels, one launch per sector GEMM;
  * (context, vendor library) a per-sector torch.mm loop over contiguous copies
    of the sector blocks, for workloads whose keys are single legs;
  * the CPU oracle (float64 sector loop) on the host cores, on a bounded sample.
"""
import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "useful GFLOP/s per block-sparse contraction (% MFMA peak); launches/contraction"
# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s)
MFMA_PEAK = {"bf16": 2516.6, "f32": 157.3, "f64": 78.6}
HBM_PEAK = 8000.0
MALL_BYTES = 256 << 20   # Infinity Cache

WORKLOADS = {
    "blockdiag_bf16": "block-diagonal bf16 GEMM, 64 U(1) sectors (45 lognormal dims rescaled to a 16384 dense equivalent + "
            "19 tail dims 1-4), fp32 accumulate",
    "ragged_batch": "4000 ragged fp32 sector GEMMs, geometric(0.35) dims capped at 64, stacked 8 per group",
    "rabc_u1": "U(1) R/A/B/C environment update, fp64, bond 1024 on 41 sectors, d=4, w=5 (3 chained stages)",
    "rabc_u1u1": "U(1)xU(1) R/A/B/C environment update, fp32, bond 4096 on 177 sectors, d=4, w=6, natural layout",
    "tiny_u1": "tiny U(1) block GEMM, fp64, 5 sectors per index",
}


# sources of the fused two-stage launch and the matrix-core probe: neither
# takes part in the grouped launch, so their edits leave its counters valid
NOT_GROUPED = ("fused.cpp", "fused.hip", "fused_internal.h", "kernels_fused.h", "probe.hip",
               "runtime_host_stub.cpp")


def _code_only(text):
    """C++ source without its comments and blank lines: what the counters
    depend on is the compiled code, so a comment edit keeps a record valid."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_source_hash():
    """Hash of the code that makes up the grouped launch: its kernels and
    launch code and the host planner that writes its work list (comments
    excluded)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_tensor_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h", ".cpp")) and f not in NOT_GROUPED:
            h.update(_code_only(open(os.path.join(csrc, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_contract_traffic.md")


def measured_traffic(workload, ld_align, stage):
    """HBM bytes per launch of the grouped kernel from committed counter runs
    (lines starting with TRAFFIC in profiles/grouped_contract_traffic.md), used
    only while the kernel sources still hash to the value they were taken with."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    src = kernel_source_hash()
    for ln in lines:
        if not ln.startswith("TRAFFIC "):
            continue
        rec = json.loads(ln[len("TRAFFIC "):])
        if rec.get("workload") == workload and rec.get("ld_align") == ld_align and rec.get("stage", 0) == stage \
                and rec.get("kernel_source") == src:
            return rec["hbm_bytes"]
    return None


def vendor_per_sector(torch, plan, con, a_buf, b_buf, dtype, steps, flops):
    """One torch.mm (hipBLASLt / rocBLAS) per sector GEMM over contiguous copies of
    the blocks, results not written back: a vendor-library context figure for the
    launch-per-sector approach.  Only for single-leg keys (plain 2-D blocks)."""
    import numpy as np
    for idx in (con.m, con.k, con.n):
        if idx.inner is not None and np.any(idx.inner != 1):
            return None

    def blocks(op, rows, cols, buf):
        d = {}
        for i in range(op.nblocks):
            r, c = int(op.row_key[i]), int(op.col_key[i])
            v = torch.as_strided(buf, (int(rows.dim[r]), int(cols.dim[c])),
                                 (int(op.row_stride[i, 0]), int(op.col_stride[i, 0])), int(op.offset[i]))
            d[(r, c)] = v.contiguous()
        return d

    A = blocks(con.A, con.m, con.k, a_buf)
    B = blocks(con.B, con.k, con.n, b_buf)
    triples = [tuple(int(x) for x in t) for t in plan.export()[0]]
    pairs = [(A[(m, k)], B[(k, n)]) for m, k, n in triples]

    def run(**kw):
        for a, b in pairs:
            torch.mm(a, b, **kw)

    def time_it(**kw):
        for _ in range(2):
            run(**kw)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run(**kw)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    vms = time_it()
    res = {"value": round(flops / (vms * 1e-3) / 1e9, 3), "unit": "GFLOP/s", "ms_per_step": round(vms, 6),
           "launches_per_contraction": len(pairs), "steps": steps, "kind": "vendor (torch.mm per sector)",
           "output_dtype": "bf16" if dtype == "bf16" else dtype}
    if dtype == "bf16":
        # the engine's output type (fp32) through the library's out_dtype route, where torch offers it
        try:
            fms = time_it(out_dtype=torch.float32)
            res["f32_output"] = {"value": round(flops / (fms * 1e-3) / 1e9, 3), "ms_per_step": round(fms, 6)}
        except Exception as e:  # not offered by this torch build
            res["f32_output"] = f"unavailable: {type(e).__name__}"
    return res


def dense_gemm_rate(torch, dtype, n=8192, reps=10):
    """torch.mm on one n x n x n dense GEMM of the workload's input dtype: the rate
    the vendor library reaches on this chip when nothing is block-sparse (a
    measured counterpart of the published peak)."""
    tdt = {"bf16": torch.bfloat16, "f32": torch.float32, "f64": torch.float64}[dtype]
    n = n if dtype == "bf16" else n // 2
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn(n, n, device="cuda", generator=g).to(tdt)
    b = torch.randn(n, n, device="cuda", generator=g).to(tdt)
    for _ in range(3):
        torch.mm(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(a, b)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps
    del a, b
    return {"tflops": round(2.0 * n ** 3 / (t * 1e-3) / 1e12, 2), "shape": [n, n, n], "ms": round(t, 4),
            "kind": "vendor (torch.mm, dense)"}


TOL = {"f64": 1e-12, "f32": 1e-5, "bf16": 2e-2}


def parity_vs_oracle(stages, bufs, ref, dtype):
    """Relative Frobenius error, over the union of each stage's C blocks, of the
    engine's buffers against the oracle's (float64), worst stage reported."""
    import numpy as np
    from workloads.layout import view_addresses
    worst = 0.0
    for con, _, _, c, _ in stages:
        parts = []
        for i in range(con.C.nblocks):
            r, cc = int(con.C.row_key[i]), int(con.C.col_key[i])
            ri = 1 if con.m.inner is None else int(con.m.inner[r])
            ci = 1 if con.n.inner is None else int(con.n.inner[cc])
            parts.append(view_addresses(con.C.offset[i], con.C.row_stride[i], con.C.col_stride[i],
                                        int(con.m.dim[r]), int(con.n.dim[cc]), ri, ci).ravel())
        if not parts:
            continue
        addr = np.concatenate(parts)
        got = bufs[c].cpu().numpy().astype(np.float64)[addr]
        want = np.asarray(ref[c], np.float64)[addr]
        nr = np.linalg.norm(want)
        err = float(np.linalg.norm(got - want) / nr) if nr > 0 else (0.0 if not np.any(got) else float("inf"))
        worst = max(worst, err)
    return {"rel_frobenius": worst, "tol": TOL[dtype], "pass": bool(worst <= TOL[dtype])}


def _view_mask(con):
    """Buffer elements that belong to some C block of `con`."""
    import numpy as np
    from workloads.layout import view_addresses
    mask = np.zeros(con.C.buffer_elems, bool)
    for i in range(con.C.nblocks):
        r, c = int(con.C.row_key[i]), int(con.C.col_key[i])
        ri = 1 if con.m.inner is None else int(con.m.inner[r])
        ci = 1 if con.n.inner is None else int(con.n.inner[c])
        mask[view_addresses(con.C.offset[i], con.C.row_stride[i], con.C.col_stride[i], int(con.m.dim[r]),
                            int(con.n.dim[c]), ri, ci).ravel()] = True
    return mask


def kernel_times(torch, fn, reps=10):
    """Device time per call (us) and launches per call of every kernel that fn
    enqueues, from torch.profiler's device activity (HIP kernel records)."""
    from torch.profiler import ProfilerActivity, profile
    fn()
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
    out = {}
    for ev in prof.key_averages():
        t = getattr(ev, "device_time_total", 0)
        if t > 0 and ev.device_type.name == "CUDA":
            out[ev.key] = {"us": round(t / reps, 3), "launches": ev.count / reps}
    return out


def calibrate_pack(torch, bst, np, reps=20):
    """Measure the pack-cost model's constants on this GPU (uni20 "block
    coalescing": the crossover uses calibrated constants).  For every stage of
    the two environment-update chains with operands to gather: the grouped
    kernel's time without gathers (NEVER_PACK), with every gatherable operand
    gathered (FORCE_PACK) and as the model decides at the library's constants
    (AUTO), each gather kernel's time, and the model's terms.  Fits
      pack_gbps   and the gather's fixed time t0: least squares of gather
                    kernel time = t0 + 2 x bytes / pack_gbps over every gather;
      t_launch_us = t0 plus the mean gap a plan's extra launch leaves
                    (contraction time - grouped kernel - gather kernel);
      t_seg_us    = (measured grouped-kernel saving - modelled padding saving)
                    / (piece set-ups saved, in units of t_seg_us) on the stage
                    where the piece term is largest;
    then re-plans every stage with the fitted constants and reports whether
    AUTO picks the faster of NEVER_PACK and FORCE_PACK.  The bf16 block-
    diagonal workload in its unpadded layout (rows off 16-byte boundaries,
    where gathers align rows for the direct-to-LDS tile) is timed and checked
    the same way."""
    cur_seg = 0.05   # t_seg_us the model's gain terms are computed with here
    rows = []
    for wl in ("rabc_u1", "rabc_u1u1", "blockdiag_bf16"):
        stages, inputs, sizes, dtype = load_workload(wl)
        cdt = torch.float64 if dtype == "f64" else torch.float32
        idt = torch.bfloat16 if dtype == "bf16" else cdt
        bufs = {k: torch.from_numpy(np.ascontiguousarray(v, np.float64)).to(idt).cuda() for k, v in inputs.items()}
        for k, n in sizes.items():
            if k not in bufs:
                bufs[k] = torch.zeros(n, dtype=cdt, device="cuda")
        for si, (con, a, b, c, ax) in enumerate(stages):
            r = {"workload": wl, "stage": si}
            for lay in ("never_pack", "force_pack", "auto"):
                # AUTO at the library's constants; the others record the model's terms at cur_seg
                p = bst.Plan(con, axis=ax, layout=lay, **({} if lay == "auto" else {"t_seg_us": cur_seg})).bind()
                st = p.stats()
                call = lambda: p.contract(bufs[a], bufs[b], bufs[c])
                for _ in range(5):
                    call()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    call()
                e1.record()
                torch.cuda.synchronize()
                kt = kernel_times(torch, call)
                r[lay] = {"us": round(e0.elapsed_time(e1) / reps * 1e3, 3), "pack_bytes": st["pack_bytes"],
                          "gather_us": sum(v["us"] for k, v in kt.items() if "pack_gather" in k),
                          "grouped_us": sum(v["us"] for k, v in kt.items() if "grouped_contract" in k),
                          "gain_seg_us": st["pack_gain_seg_us"], "gain_pad_us": st["pack_gain_pad_us"],
                          "cost_us": st["pack_cost_us"], "predicted_us": round(st["predicted_us"], 3)}
                del p
            if r["force_pack"]["pack_bytes"] > 0:
                rows.append(r)
    gathers = [r[lay] for r in rows for lay in ("force_pack", "auto") if r[lay]["pack_bytes"] > 0]
    x = np.array([2.0 * g["pack_bytes"] for g in gathers])
    y = np.array([g["gather_us"] for g in gathers])
    slope, t0 = np.polyfit(x, y, 1)            # us per byte moved, fixed us
    pack_gbps = 1.0 / (slope * 1e3)
    gap = float(np.mean([g["us"] - g["grouped_us"] - g["gather_us"] for g in gathers]))
    t_launch = t0 + max(0.0, gap)
    seg = max(rows, key=lambda r: r["force_pack"]["gain_seg_us"])
    saving = seg["never_pack"]["grouped_us"] - seg["force_pack"]["grouped_us"] - seg["force_pack"]["gain_pad_us"]
    t_seg = max(0.0, saving / (seg["force_pack"]["gain_seg_us"] / cur_seg))
    fitted = {"pack_gbps": round(pack_gbps, 1), "t_launch_us": round(t_launch, 3), "t_seg_us": round(t_seg, 6),
              "gather_fixed_us": round(float(t0), 3), "launch_gap_us": round(gap, 3)}
    # AUTO with the fitted constants against the measured faster arrangement
    checks = []
    for r in rows:
        stages, _, _, _ = load_workload(r["workload"])
        con, _, _, _, ax = stages[r["stage"]]
        st = bst.Plan(con, axis=ax, layout="auto", t_launch_us=t_launch, t_seg_us=t_seg, pack_gbps=pack_gbps).stats()
        picks_pack = st["pack_bytes"] > 0
        faster_pack = r["force_pack"]["us"] < r["never_pack"]["us"]
        checks.append({"workload": r["workload"], "stage": r["stage"], "auto_gathers": picks_pack,
                       "gathering_is_faster": faster_pack, "agrees": picks_pack == faster_pack})
    return {"stages": rows, "fitted": fitted, "auto_with_fitted": checks}


def measured_mfma_peaks(torch, bst):
    """Matrix-core rates measured on this GPU (bsc_probe_mfma), TFLOP/s, for
    the instruction each dtype's tiles use: the mean of 5 timed launches of
    about a millisecond each after one warm-up."""
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    out = {}
    for dt, iters in (("bf16", 2000), ("f32", 1000), ("f64", 500)):
        bst.probe_mfma(dt, iters, sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = sum(bst.probe_mfma(dt, iters, sink) for _ in range(5))
        e1.record()
        torch.cuda.synchronize()
        out[dt] = round(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12, 2)
    return out


def measured_memory_peaks(torch):
    """Memory rates and launch cost measured on this GPU, beside the published
    HBM figure: a device-to-device copy (torch copy_, the runtime's copy
    kernel) of 2 x 2 GiB buffers, far larger than the 256 MB Infinity Cache
    (HBM), and of 2 x 32 MiB buffers copied back to back, which stay in the
    Infinity Cache (MALL); bytes counted as read + write.  Launch cost: the
    interval between back-to-back launches of a one-element kernel."""
    def rate(nbytes, reps):
        n = nbytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        gbps = 2.0 * n * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst
        return round(gbps, 1)
    hbm = rate(2 << 30, 5)
    mall = rate(32 << 20, 200)
    x = torch.zeros(1, dtype=torch.float32, device="cuda")
    x.add_(1.0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(500):
        x.add_(1.0)
    e1.record()
    torch.cuda.synchronize()
    launch_us = e0.elapsed_time(e1) * 1e3 / 500
    torch.cuda.empty_cache()
    return {"hbm_copy_gbps": hbm, "mall_copy_gbps": mall, "hbm_spec_gbps": HBM_PEAK,
            "hbm_frac_of_spec": round(hbm / HBM_PEAK, 4), "launch_interval_us": round(launch_us, 3),
            "kind": "torch copy_ of 2 x 2 GiB (HBM) and 2 x 32 MiB (Infinity Cache), read + write bytes; "
                    "back-to-back one-element kernels"}


def load_workload(name, ld_align=1, relayout=False):
    from workloads import configs as C
    if name == "blockdiag_bf16":
        p = C.blockdiag_bf16(ld_align=ld_align, align=max(1, ld_align))
        stages = [(p.con, "a", "b", "c", "auto")]
        return stages, {"a": p.a, "b": p.b}, {"c": p.con.C.buffer_elems}, "bf16"
    if name == "tiny_u1":
        p = C.tiny_u1()
        return [(p.con, "a", "b", "c", "auto")], {"a": p.a, "b": p.b}, {"c": p.con.C.buffer_elems}, "f64"
    if name == "ragged_batch":
        p = C.ragged_batch()
        return [(p.con, "a", "b", "c", "auto")], {"a": p.a, "b": p.b}, {"c": p.con.C.buffer_elems}, "f32"
    if name in ("rabc_u1", "rabc_u1u1"):
        ch = C.rabc_u1() if name == "rabc_u1" else C.rabc_u1u1()
        stages = [(st.con, st.a_buf, st.b_buf, st.c_buf, "auto") for st in ch.stages]
        if not relayout:
            return stages, dict(ch.buffers), dict(ch.sizes), ch.dtype
        # every intermediate laid out for the stage that writes it, every input for a stage that reads it
        # (bsc_plan_layout), inputs moved to match
        from block_sparse_tensor_amd.layouts import move_blocks, relayout_chain
        new, sizes, _ = relayout_chain([s[:4] for s in stages], axes=[s[4] for s in stages])
        inputs = {}
        for buf, v in ch.buffers.items():
            i, which = next((i, w) for i, s in enumerate(stages) for w, b in zip("AB", s[1:3]) if b == buf)
            inputs[buf] = move_blocks(v, stages[i][0], which, new[i])
        return [(c,) + s[1:] for c, s in zip(new, stages)], inputs, sizes, ch.dtype
    raise SystemExit(f"unknown workload {name}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="blockdiag_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--baseline-steps", type=int, default=20)
    ap.add_argument("--no-baseline", action="store_true", help="skip the per-sector GPU baseline")
    ap.add_argument("--ld-align", type=int, default=8,
                    help="blockdiag_bf16: pad each block's leading dimension (and start) to a multiple of this many "
                         "elements; 8 = 16-byte aligned rows (default), 1 = unpadded contiguous blocks")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes (counter calibration) and exit")
    ap.add_argument("--calibrate-pack", action="store_true",
                    help="only measure the pack-cost model's constants on the chains' stages and exit")
    ap.add_argument("--layout", default="auto", choices=["auto", "never_pack", "force_pack"],
                    help="operand arrangement policy of the grouped plans (auto = the planner's pack-cost model)")
    ap.add_argument("--relayout", action="store_true",
                    help="chains: lay out every buffer for the stage that writes it, inputs for a stage that reads "
                         "them (cross-stage layout planning)")
    ap.add_argument("--tile-cols", type=int, default=0, choices=[0, 128, 256],
                    help="bf16 direct-to-LDS tile width: 0 = the engine's choice, 128 = 256x128 tiles two per CU, "
                         "256 = the wide tile, one workgroup per CU")
    ap.add_argument("--split-k", type=int, default=0, help="K split policy of the bf16 tiles (plan option)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="contractions timed one by one after a cache-evicting write (0 = skip)")
    ap.add_argument("--no-vendor", action="store_true", help="skip the per-sector torch.mm context baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this engine runs on one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is a design note only)", file=sys.stderr)
        raise SystemExit(2)

    import numpy as np
    import torch

    import block_sparse_tensor_amd as bst

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    if args.copy_calibration:
        # a plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it calibrates the counters
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 5}), flush=True)
        return
    if args.calibrate_pack:
        print(json.dumps(calibrate_pack(torch, bst, np)), flush=True)
        return
    stages, inputs, sizes, dtype = load_workload(args.workload, args.ld_align, args.relayout)

    # inputs resident in HBM before timing
    def dev(x):
        t = torch.from_numpy(np.ascontiguousarray(x, np.float64 if dtype == "f64" else np.float32)).cuda()
        return t.to(torch.bfloat16) if dtype == "bf16" else t

    cdt = torch.float64 if dtype == "f64" else torch.float32
    bufs = {k: dev(v) for k, v in inputs.items()}
    for k, n in sizes.items():
        if k not in bufs:
            bufs[k] = torch.zeros(n, dtype=cdt, device="cuda")

    def plans_for(mode):
        layout = args.layout if mode == "grouped" else "never_pack"
        return [bst.Plan(con, axis=ax, launch_mode=mode, layout=layout, tile_cols=args.tile_cols,
                         split_k=args.split_k).bind() for con, _, _, _, ax in stages]

    def step(plans):
        for p, (_, a, b, c, _) in zip(plans, stages):
            p.contract(bufs[a], bufs[b], bufs[c])

    grouped = plans_for("grouped")
    st = [p.stats() for p in grouped]
    flops = sum(s["useful_flops"] for s in st)
    alg_bytes = sum(s["alg_bytes"] for s in st)
    launches = sum(s["launches_per_contract"] for s in st)
    launches_ps = sum(s["launches_per_sector"] for s in st)

    def timed(plans, K, W):
        for _ in range(W):
            step(plans)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            step(plans)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    # --- engine: timed region ----------------------------------------------------------
    # K steps between two events on torch's current stream (the stream the engine
    # launches on).  A one-launch step needs nothing more: the average launch
    # duration is the region over K.  For a step of several launches a second
    # pass of K steps records an event after every launch, so each stage's
    # launches are timed on their own (kept out of the first pass, whose step
    # time they would lengthen).
    for _ in range(args.warmup):
        step(grouped)
    torch.cuda.synchronize()
    multi = len(stages) > 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        step(grouped)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    if multi:
        marks = []
        m0 = torch.cuda.Event(enable_timing=True)
        m0.record()
        for _ in range(args.steps):
            for p, (_, a, b, c, _) in zip(grouped, stages):
                p.contract(bufs[a], bufs[b], bufs[c])
                ev = torch.cuda.Event(enable_timing=True)
                ev.record()
                marks.append(ev)
        torch.cuda.synchronize()
        bounds = [m0] + marks
        stage_ms = [statistics.fmean(bounds[j].elapsed_time(bounds[j + 1])
                                     for j in range(i, len(marks), len(stages))) for i in range(len(stages))]
    else:
        stage_ms = [ms]
    dom = max(range(len(stages)), key=lambda i: stage_ms[i])
    dom_flops = st[dom]["useful_flops"]
    dom_bytes = st[dom]["alg_bytes"]
    achieved_tflops = dom_flops / (stage_ms[dom] * 1e-3) / 1e12
    achieved_gbps = dom_bytes / (stage_ms[dom] * 1e-3) / 1e9
    peak = MFMA_PEAK[dtype]
    # Which roofline bounds the dominant stage.  Below the ridge point (peak
    # flops over HBM bandwidth) a stage streamed from HBM is bandwidth-bound.
    # The timed runs are back to back, so a stage whose operands fit in the
    # 256 MB Infinity Cache is served from there, not from HBM: such a stage is
    # rated against HBM only when it is far below the ridge (under a tenth of
    # it: the W stage of the chains, 0.4 flop/B), otherwise against the matrix
    # cores.  Both fractions and the fraction of the attainable roofline
    # min(peak, AI x HBM) are reported either way.
    ridge = peak * 1e12 / (HBM_PEAK * 1e9)
    ai = dom_flops / max(1, dom_bytes)
    mall_resident = dom_bytes <= MALL_BYTES
    hbm_bound = ai < 0.1 * ridge or (ai < ridge and not mall_resident)
    traffic = measured_traffic(args.workload, args.ld_align, dom)

    # --- the same stages captured once into a HIP graph, one graph launch per step ----
    graph = None
    if multi:
        chain = bst.Chain([(p, bufs[a], bufs[b], bufs[c]) for p, (_, a, b, c, _) in zip(grouped, stages)])
        for _ in range(args.warmup):
            chain.launch()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            chain.launch()
        g1.record()
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / args.steps
        graph = {"ms_per_step": round(gms, 6), "value": round(flops / (gms * 1e-3) / 1e9, 3), "unit": "GFLOP/s",
                 "launches_per_step": 1}

    # --- stages 1 and 2 as one fused launch (bsc_fused): the intermediate never written ---
    fused = None
    if multi and dtype in ("f64", "f32"):
        try:
            fplan = bst.FusedPlan(stages[0][0], stages[1][0]).bind()
        except bst.BscError as e:
            fused = {"skipped": str(e)}
        else:
            fbuf = {k: v for k, v in bufs.items()}
            fbuf[stages[1][3]] = torch.zeros_like(bufs[stages[1][3]])

            def fstep(marks=None):
                fplan.contract(fbuf[stages[0][1]], fbuf[stages[0][2]], fbuf[stages[1][2]], fbuf[stages[1][3]])
                if marks is not None:
                    ev = torch.cuda.Event(enable_timing=True)
                    ev.record()
                    marks.append(ev)
                for p, (_, a, b, c, _) in zip(grouped[2:], stages[2:]):
                    p.contract(fbuf[a], fbuf[b], fbuf[c])
                    if marks is not None:
                        ev = torch.cuda.Event(enable_timing=True)
                        ev.record()
                        marks.append(ev)
            for _ in range(args.warmup):
                fstep()
            torch.cuda.synchronize()
            f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            f0.record()
            for _ in range(args.steps):
                fstep()
            f1.record()
            torch.cuda.synchronize()
            fms = f0.elapsed_time(f1) / args.steps
            fm = [torch.cuda.Event(enable_timing=True)]
            fm[0].record()
            for _ in range(args.steps):
                fstep(fm)
            torch.cuda.synchronize()
            nl = len(stages) - 1
            fstage = [statistics.fmean(fm[j].elapsed_time(fm[j + 1]) for j in range(i, len(fm) - 1, nl))
                      for i in range(nl)]
            fs = fplan.stats()
            # parity of the fused intermediate-free path against the two-stage engine result
            step(grouped)
            fstep()
            torch.cuda.synchronize()
            ad = torch.from_numpy(np.nonzero(_view_mask(stages[1][0]))[0]).cuda()
            ref_t2 = bufs[stages[1][3]].index_select(0, ad).double()
            got_t2 = fbuf[stages[1][3]].index_select(0, ad).double()
            rel = float((got_t2 - ref_t2).norm() / ref_t2.norm().clamp_min(1e-300))
            fused = {"ms_per_step": round(fms, 6), "value": round(flops / (fms * 1e-3) / 1e9, 3), "unit": "GFLOP/s",
                     "stage_kernel_ms": [round(x, 6) for x in fstage],
                     "fused_kernel_ms_vs_stages_1_2": [round(fstage[0], 6), round(stage_ms[0] + stage_ms[1], 6)],
                     "fused_flops": fs["useful_flops"], "fused_alg_bytes": fs["alg_bytes"],
                     "fused_tflops": round(fs["useful_flops"] / (fstage[0] * 1e-3) / 1e12, 4),
                     "items": fs["items"], "products": fs["channels"], "terms": fs["terms"],
                     "t2_rel_diff_vs_two_stage": rel, "launches_per_step": len(stages) - 1}
            # the same with the later stages on the plan the library prefers for them
            # (best_plan: the register stream where bsc_stream_plan reports it preferred)
            tail = []
            for p, (con, _, _, _, ax) in zip(grouped[2:], stages[2:]):
                bp = bst.best_plan(con, dtype=dtype)
                tail.append(("stream", bp.bind()) if isinstance(bp, bst.StreamPlan) else ("grouped", p))
            sbuf = {k: v for k, v in fbuf.items()}
            for _, a, b, c, _ in stages[2:]:
                sbuf[c] = torch.zeros_like(fbuf[c])

            def sstep(marks=None):
                fplan.contract(sbuf[stages[0][1]], sbuf[stages[0][2]], sbuf[stages[1][2]], sbuf[stages[1][3]])
                if marks is not None:
                    ev = torch.cuda.Event(enable_timing=True)
                    ev.record()
                    marks.append(ev)
                for (_, p), (_, a, b, c, _) in zip(tail, stages[2:]):
                    p.contract(sbuf[a], sbuf[b], sbuf[c])
                    if marks is not None:
                        ev = torch.cuda.Event(enable_timing=True)
                        ev.record()
                        marks.append(ev)
            for _ in range(args.warmup):
                sstep()
            torch.cuda.synchronize()
            f0.record()
            for _ in range(args.steps):
                sstep()
            f1.record()
            torch.cuda.synchronize()
            sms = f0.elapsed_time(f1) / args.steps
            sm = [torch.cuda.Event(enable_timing=True)]
            sm[0].record()
            for _ in range(args.steps):
                sstep(sm)
            torch.cuda.synchronize()
            sstage = [statistics.fmean(sm[j].elapsed_time(sm[j + 1]) for j in range(i, len(sm) - 1, nl))
                      for i in range(nl)]
            # parity of the last stage's output against the all-grouped step
            last = stages[-1][3]
            adl = torch.from_numpy(np.nonzero(_view_mask(stages[-1][0]))[0]).cuda()
            ref_l = bufs[last].index_select(0, adl).double()
            got_l = sbuf[last].index_select(0, adl).double()
            srel = float((got_l - ref_l).norm() / ref_l.norm().clamp_min(1e-300))
            tail_flops = [bp.stats()["useful_flops"] for _, bp in tail]
            fused["stream_tail"] = {"ms_per_step": round(sms, 6), "value": round(flops / (sms * 1e-3) / 1e9, 3),
                                    "unit": "GFLOP/s", "stage_kernel_ms": [round(x, 6) for x in sstage],
                                    "tail_plans": [k for k, _ in tail],
                                    # each launch's useful rate against the matrix-core peak of the dtype
                                    "frac_mfma": [round(fs["useful_flops"] / (sstage[0] * 1e-3) / 1e12 / peak, 5)] +
                                                 [round(fl / (t * 1e-3) / 1e12 / peak, 5)
                                                  for fl, t in zip(tail_flops, sstage[1:])],
                                    "last_output_rel_diff_vs_grouped": srel}

    # --- the gather (pack) phase against the HBM roofline: every gatherable operand of each
    # stage gathered (FORCE_PACK), the gather kernel's own time from the profiler ---
    pack_phase = []
    if multi:
        for si, (con, a, b, c, ax) in enumerate(stages):
            fpl = bst.Plan(con, axis=ax, layout="force_pack").bind()
            pb = fpl.stats()["pack_bytes"]
            if pb == 0:
                continue
            kt = kernel_times(torch, lambda: fpl.contract(bufs[a], bufs[b], bufs[c]))
            gus = sum(v["us"] for k, v in kt.items() if "pack_gather" in k)
            if gus > 0:
                pack_phase.append({"stage": si, "bytes_gathered": pb, "gather_kernel_us": round(gus, 3),
                                   "gbps": round(2 * pb / (gus * 1e3), 1),
                                   "frac_hbm": round(2 * pb / (gus * 1e3) / HBM_PEAK, 4),
                                   "auto_gathers": st[si]["pack_bytes"] > 0})
            del fpl
        step(grouped)   # the timed plans' results back in C for the parity check below

    # --- host planning of every stage: fresh, and a plan-cache hit (a site revisited in a sweep) ---
    def plan_all(cache=None):
        t0 = time.perf_counter()
        for con, _, _, _, ax in stages:
            bst.Plan(con, axis=ax, layout=args.layout, cache=cache)
        return (time.perf_counter() - t0) * 1e3
    pcache = bst.PlanCache(max(4, len(stages)))
    plan_all(pcache)
    planning = {"fresh_ms": round(min(plan_all() for _ in range(3)), 4),
                "cached_ms": round(min(plan_all(pcache) for _ in range(3)), 4)}

    # --- uncoalesced GPU baseline: one launch per sector GEMM -----------------------
    if not args.no_baseline:
        per_sector = plans_for("per_sector")
        ms_ps = timed(per_sector, args.baseline_steps, 2)

    # --- cold caches: every contraction after a 512 MiB write (twice the Infinity Cache) ---
    cold = None
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        ev = []
        for _ in range(args.cold_steps):
            flush.fill_(1)
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            step(grouped)
            c1.record()
            ev.append((c0, c1))
        torch.cuda.synchronize()
        cms = [a.elapsed_time(b) for a, b in ev]
        del flush
        cmed = statistics.median(cms)
        cold = {"ms_per_step_median": round(cmed, 6), "ms_per_step_min": round(min(cms), 6),
                "value": round(flops / (cmed * 1e-3) / 1e9, 3), "unit": "GFLOP/s",
                "pct_mfma_peak": round(100.0 * flops / (cmed * 1e-3) / 1e12 / peak, 3),
                # cold ceiling: every algorithmic byte from HBM at its peak, flops at the MFMA peak
                "hbm_ceiling_pct_mfma_peak": round(100.0 * min(1.0, HBM_PEAK * 1e9 * (flops / alg_bytes)
                                                               / (peak * 1e12)), 2),
                "steps": args.cold_steps, "flush_bytes": 512 << 20}

    # --- the bf16 workload in its unpadded, as-generated layout (rows not 16-byte aligned) ---
    unpadded = None
    if args.workload == "blockdiag_bf16" and args.ld_align != 1:
        ustages, uinputs, usizes, _ = load_workload(args.workload, 1)
        ubufs = {k: dev(v) for k, v in uinputs.items()}
        for k, n in usizes.items():
            ubufs[k] = torch.zeros(n, dtype=cdt, device="cuda")
        uplans = [bst.Plan(con, axis=ax, layout=args.layout, tile_cols=args.tile_cols, split_k=args.split_k).bind()
                  for con, _, _, _, ax in ustages]

        def ustep():
            for p, (_, a, b, c, _) in zip(uplans, ustages):
                p.contract(ubufs[a], ubufs[b], ubufs[c])
        for _ in range(args.warmup):
            ustep()
        torch.cuda.synchronize()
        u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        u0.record()
        for _ in range(args.steps):
            ustep()
        u1.record()
        torch.cuda.synchronize()
        ums = u0.elapsed_time(u1) / args.steps
        us = uplans[0].stats()
        unpadded = {"ld_align": 1, "ms_per_step": round(ums, 6), "value": round(flops / (ums * 1e-3) / 1e9, 3),
                    "unit": "GFLOP/s", "pct_mfma_peak": round(100.0 * flops / (ums * 1e-3) / 1e12 / peak, 3),
                    "items_by_class": us["items_by_class"], "launches_per_contraction": us["launches_per_contract"]}
        del ubufs, uplans

    # --- context: per-sector vendor GEMMs (torch.mm) on contiguous copies of the blocks ---
    vendor = None
    if not args.no_vendor and len(stages) == 1:
        vendor = vendor_per_sector(torch, grouped[0], stages[0][0], bufs[stages[0][1]], bufs[stages[0][2]],
                                   dtype, args.baseline_steps, flops)

    # --- context: what the vendor library reaches on one large dense GEMM of the dtype ---
    dense_ref = None
    if not args.no_vendor:
        dense_ref = dense_gemm_rate(torch, dtype)

    value = flops / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {WORKLOADS[args.workload]}", "stages": len(stages),
                   "ld_align": args.ld_align, "layout": args.layout, "relayout": args.relayout,
                   "tile_cols": args.tile_cols, "split_k": args.split_k,
                   "pack_bytes": sum(s["pack_bytes"] for s in st),
                   "sector_gemms": sum(s["triples"] for s in st), "useful_flops": flops,
                   "alg_bytes": alg_bytes, "parallelism": "single GPU"},
        "pct_mfma_peak": round(100.0 * value / (peak * 1e3), 3),
        "launches_per_contraction": launches,
        "launches_per_sector_baseline": launches_ps,
        "launch_reduction": round(launches_ps / max(1, launches), 2),
        "roofline": {
            "bound": "hbm" if hbm_bound else "mfma",
            "kernel": "grouped_contract",
            "achieved": round(achieved_gbps if hbm_bound else achieved_tflops, 4),
            "peak": HBM_PEAK if hbm_bound else peak,
            "unit": "GB/s" if hbm_bound else "TFLOP/s",
            "frac": round(achieved_gbps / HBM_PEAK if hbm_bound else achieved_tflops / peak, 5),
            "traffic": traffic,
            "kernel_ms": round(stage_ms[dom], 6),
            "flops_per_launch": dom_flops,
            "alg_bytes_per_launch": dom_bytes,
            "hbm_gbps_on_alg_bytes": round(dom_bytes / (stage_ms[dom] * 1e-3) / 1e9, 2),
            "arithmetic_intensity": round(ai, 3),
            "ridge_flop_per_byte": round(ridge, 2),
            "frac_mfma": round(achieved_tflops / peak, 5),
            "frac_hbm": round(achieved_gbps / HBM_PEAK, 5),
            "frac_attainable": round(achieved_tflops / min(peak, ai * HBM_PEAK * 1e-3), 5),
            "operands_fit_infinity_cache": mall_resident,
            "kernel_source": kernel_source_hash(),
        },
        "gpu_per_sector_baseline": None if args.no_baseline else {
            "value": round(flops / (ms_ps * 1e-3) / 1e9, 3), "unit": "GFLOP/s", "ms_per_step": round(ms_ps, 6),
            "launches_per_contraction": launches_ps, "steps": args.baseline_steps,
        },
        "cold_caches": cold,
        "unpadded_layout": unpadded,
        "vendor_per_sector_context": vendor,
        "vendor_dense_gemm_context": dense_ref if dense_ref is None else dict(
            dense_ref, engine_pct_of_it=round(100.0 * value / 1e3 / dense_ref["tflops"], 3)),
        "stage_kernel_ms": [round(x, 6) for x in stage_ms],
        "host_planning": planning,
        # the pack-cost model's estimate of one step next to the measured time
        "cost_model": {"predicted_us": round(sum(x["predicted_us"] for x in st), 3),
                       "measured_us": round(ms * 1e3, 3),
                       "per_stage": [{"predicted_us": round(x["predicted_us"], 3), "measured_us": round(t * 1e3, 3),
                                      "pack_bytes": x["pack_bytes"]} for x, t in zip(st, stage_ms)]},
    }
    mpk = measured_mfma_peaks(torch, bst)
    out["mfma_peak_measured"] = dict(mpk, unit="TFLOP/s", spec=MFMA_PEAK, kernel="bsc_probe_mfma")
    mem = measured_memory_peaks(torch)
    out["memory_peak_measured"] = mem
    if not hbm_bound:
        out["roofline"]["frac_of_measured_peak"] = round(achieved_tflops / mpk[dtype], 5)
    else:
        out["roofline"]["frac_of_measured_peak"] = round(achieved_gbps / mem["hbm_copy_gbps"], 5)
    if pack_phase:
        out["pack_phase"] = pack_phase
    if graph is not None:
        # the stages as one captured graph (bsc_chain): no host gaps between launches
        out["graph_chain"] = graph
    if fused is not None:
        out["fused_stage_1_2"] = fused

    # --- CPU oracle baseline on the host cores ----------------------------------------
    if not args.no_cpu:
        import oracle
        blas = {}
        try:
            from threadpoolctl import threadpool_info, threadpool_limits
            info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
            threads = max([i.get("num_threads", 1) for i in info] or [1])
            if info:
                blas = {"library": info[0].get("internal_api"), "version": info[0].get("version")}
        except Exception:
            threadpool_limits = None
            threads = os.cpu_count() or 1
        cpu_model = None
        try:
            cpu_model = next(ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name"))
        except Exception:
            pass
        host = {k: np.asarray(v, np.float64) for k, v in inputs.items()}

        def oracle_times(budget_s):
            times = []
            t_start = time.perf_counter()
            while True:
                hb = dict(host)
                t0 = time.perf_counter()
                for con, a, b, c, _ in stages:
                    hb[c] = oracle.contract(con, hb[a], hb[b], np.zeros(sizes[c]), check=False)
                times.append(time.perf_counter() - t0)
                if time.perf_counter() - t_start >= budget_s or len(times) >= 1000:
                    return times, hb

        times, hb = oracle_times(args.cpu_seconds)
        med = statistics.median(times)
        out["cpu_baseline"] = {
            "value": round(flops / med / 1e9, 4), "unit": "GFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(times)} full contractions of the same workload (median {med:.4f} s), float64 numpy "
                      f"sector loop, {len(os.sched_getaffinity(0))} host cores visible",
            "cpu_model": cpu_model, "blas": blas,
        }
        # parity of the timed path: one more grouped step (the per-sector baseline
        # and the vendor leg wrote C since the timed region), then every stage's
        # C views against the oracle's result for the same inputs
        step(grouped)
        torch.cuda.synchronize()
        out["cpu_baseline"]["parity"] = parity_vs_oracle(stages, bufs, hb, dtype)
        if threadpool_limits is not None:
            # the same oracle on one BLAS thread, over a third of the time budget
            with threadpool_limits(limits=1, user_api="blas"):
                t1, _ = oracle_times(args.cpu_seconds / 3)
            m1 = statistics.median(t1)
            out["cpu_baseline"]["one_thread"] = {"value": round(flops / m1 / 1e9, 4), "unit": "GFLOP/s",
                                                 "contractions": len(t1), "median_s": round(m1, 5)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
