"""Python binding over the C-ABI (argument marshalling only).

Every step of a contraction runs in libbsc.so: planning in its host planner,
the contraction in its HIP kernels.  PyTorch supplies device memory and the
stream; no torch operator touches operand data here.
"""
from __future__ import annotations

import ctypes
from ctypes import byref, c_int32, c_size_t, c_void_p

import numpy as np

from . import _capi

AXES = {"none": 0, "free_m": 1, "free_n": 2, "contract": 3, "auto": 4}
AXIS_NAMES = {v: k for k, v in AXES.items()}
DTYPES = {"f64": 0, "f32": 1, "bf16": 2}
LAUNCH = {"grouped": 0, "per_sector": 1}
LAYOUT = {"auto": 0, "never_pack": 1, "force_pack": 2}
MODES = {0: "view", 1: "pack", 2: "segments"}


class BscError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = _capi.STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


def _check(st: int):
    if st != 0:
        raise BscError(st, _capi.lib().bsc_last_error().decode())


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class _Keep:
    """Holds the numpy arrays a ctypes struct points into."""

    def __init__(self):
        self.arrays = []

    def arr(self, x, dt):
        a = np.ascontiguousarray(x, dtype=dt)
        self.arrays.append(a)
        return a


def _index(idx, keep):
    s = _capi.BscIndex()
    ch = keep.arr(idx.charge, np.int32)
    dim = keep.arr(idx.dim, np.int64)
    s.nkeys = int(dim.shape[0])
    s.nq = int(ch.shape[1]) if ch.ndim == 2 else 1
    s.charge = _ptr(ch, ctypes.c_int32)
    s.dim = _ptr(dim, ctypes.c_int64)
    s.inner = None if idx.inner is None else _ptr(keep.arr(idx.inner, np.int64), ctypes.c_int64)
    return s


def _operand(op, keep):
    s = _capi.BscOperand()
    s.nblocks = int(len(op.row_key))
    s.row_key = _ptr(keep.arr(op.row_key, np.int32), ctypes.c_int32)
    s.col_key = _ptr(keep.arr(op.col_key, np.int32), ctypes.c_int32)
    s.offset = _ptr(keep.arr(op.offset, np.int64), ctypes.c_int64)
    s.row_stride = _ptr(keep.arr(np.reshape(op.row_stride, (-1, 2)), np.int64), ctypes.c_int64)
    s.col_stride = _ptr(keep.arr(np.reshape(op.col_stride, (-1, 2)), np.int64), ctypes.c_int64)
    s.flux = _ptr(keep.arr(op.flux, np.int32), ctypes.c_int32)
    s.buffer_elems = int(op.buffer_elems)
    return s


def _torch():
    import torch  # only for device memory and streams
    return torch


_raw_stream = None


def _current_stream_raw():
    """Raw handle of torch's current stream on the current device.  torch's
    raw-stream query (the one its own extensions use) takes about 0.3 us;
    building a Stream object through current_stream() about 2.8 us, which
    is a third of a whole small contraction's time, so the former is used
    where this torch has it."""
    global _raw_stream
    torch = _torch()
    if _raw_stream is None:
        _raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if _raw_stream:
        return _raw_stream(torch.cuda.current_device())
    return torch.cuda.current_stream().cuda_stream


def _stream_handle(stream):
    if stream is None:
        return c_void_p(_current_stream_raw())
    if isinstance(stream, int):
        return c_void_p(stream)
    return c_void_p(stream.cuda_stream)


def _plan_args(con, dtype, axis, keep, launch_mode="grouped", layout="auto", accumulate=False, grid_limit=0,
               t_launch_us=0.0, t_seg_us=0.0, pack_gbps=0.0, tile_gflops=0.0, split_k=0, tile_rows=0, tile_cols=0):
    """bsc_plan's arguments (without the output handle) as ctypes values."""
    L = _capi.lib()
    m, k, n = _index(con.m, keep), _index(con.k, keep), _index(con.n, keep)
    A, B, C = _operand(con.A, keep), _operand(con.B, keep), _operand(con.C, keep)
    opt = _capi.BscOptions()
    L.bsc_options_default(byref(opt))
    opt.launch_mode = LAUNCH[launch_mode]
    opt.layout_policy = LAYOUT[layout]
    opt.accumulate = int(bool(accumulate))
    opt.grid_limit = int(grid_limit)
    opt.t_launch_us, opt.t_seg_us, opt.pack_gbps, opt.tile_gflops = t_launch_us, t_seg_us, pack_gbps, tile_gflops
    opt.split_k = int(split_k)
    opt.tile_rows = int(tile_rows)
    opt.tile_cols = int(tile_cols)
    keep.arrays.extend([m, k, n, A, B, C, opt])
    return (byref(m), byref(k), byref(n), byref(A), byref(B), byref(C), DTYPES[dtype], AXES[axis], byref(opt))


def plan_layout(con, which: str, align: int = 1, dtype: str = None, axis: str = "auto", **options):
    """Layout of operand `which` ("A", "B" or "C") that lets the contraction
    `con` address its groups' members of that operand as single strided views
    (bsc_plan_layout).  The operand's own offsets and strides are ignored.
    Returns (offset [nb], row_stride [nb, 2], col_stride [nb, 2], buffer_elems)."""
    op = {"A": con.A, "B": con.B, "C": con.C}[which]
    nb = len(op.row_key)
    keep = _Keep()
    args = _plan_args(con, dtype or con.dtype, axis, keep, **options)
    off = np.zeros(max(nb, 1), np.int64)
    rs = np.zeros((max(nb, 1), 2), np.int64)
    cs = np.zeros((max(nb, 1), 2), np.int64)
    total = ctypes.c_int64()
    _check(_capi.lib().bsc_plan_layout(*args, "ABC".index(which), int(align), _ptr(off, ctypes.c_int64),
                                       _ptr(rs, ctypes.c_int64), _ptr(cs, ctypes.c_int64), byref(total)))
    return off[:nb], rs[:nb], cs[:nb], int(total.value)


class Plan:
    """A planned block-sparse contraction C[m,n] = sum_k A[m,k] B[k,n].

    `con` is any object with attributes m, k, n (indices: charge, dim, inner)
    and A, B, C (operands: row_key, col_key, offset, row_stride, col_stride,
    flux, buffer_elems), e.g. workloads.Contraction.  With `cache` (a
    PlanCache) the plan is copied from the cache when every input matches a
    cached one (bsc_plan_cached); `cache_hit` tells which happened."""

    def __init__(self, con, dtype: str = None, axis: str = "auto", launch_mode: str = "grouped",
                 layout: str = "auto", accumulate: bool = False, grid_limit: int = 0,
                 t_launch_us: float = 0.0, t_seg_us: float = 0.0, pack_gbps: float = 0.0, tile_gflops: float = 0.0,
                 split_k: int = 0, tile_rows: int = 0, tile_cols: int = 0, cache: "PlanCache" = None):
        L = _capi.lib()
        self.dtype = dtype or con.dtype
        keep = _Keep()
        args = _plan_args(con, self.dtype, axis, keep, launch_mode=launch_mode, layout=layout, accumulate=accumulate,
                          grid_limit=grid_limit, t_launch_us=t_launch_us, t_seg_us=t_seg_us, pack_gbps=pack_gbps,
                          tile_gflops=tile_gflops, split_k=split_k, tile_rows=tile_rows, tile_cols=tile_cols)
        h = c_void_p()
        if cache is None:
            _check(L.bsc_plan(*args, byref(h)))
            self.cache_hit = False
        else:
            hit = c_int32()
            _check(L.bsc_plan_cached(cache._h, *args, byref(h), byref(hit)))
            self.cache_hit = bool(hit.value)
        self._h = h
        self.a_elems, self.b_elems, self.c_elems = int(con.A.buffer_elems), int(con.B.buffer_elems), int(con.C.buffer_elems)
        self._dev = None
        self._captured = 0   # live Chains whose graph holds this plan's device region

    # -- host-side queries -------------------------------------------------------
    def device_bytes(self) -> int:
        n = c_size_t()
        _check(_capi.lib().bsc_plan_device_bytes(self._h, byref(n)))
        return int(n.value)

    def stats(self) -> dict:
        s = _capi.BscStats()
        _check(_capi.lib().bsc_plan_stats(self._h, byref(s)))
        out = {}
        for name, _ in s._fields_:
            v = getattr(s, name)
            if name == "mode_count":
                v = {op: {MODES[j]: int(v[i][j]) for j in range(3)} for i, op in enumerate("ABC")}
            elif name == "items_by_class":
                v = dict(zip(("generic", "mfma", "tail", "zero", "mfma_fast", "skinny"), (int(x) for x in v)))
            out[name] = v
        out["axis_name"] = AXIS_NAMES[out["axis"]]
        return out

    def export(self):
        """(triples [T,3] (m,k,n), group_of_triple [T], group_mode [G,3])."""
        s = self.stats()
        T, G = s["triples"], s["groups"]
        t = np.zeros((T, 3), np.int32)
        g = np.zeros(T, np.int32)
        md = np.zeros((G, 3), np.int32)
        _check(_capi.lib().bsc_plan_export(self._h, _ptr(t, ctypes.c_int32), _ptr(g, ctypes.c_int32),
                                           _ptr(md, ctypes.c_int32)))
        return t, g, md

    def worklist(self):
        """(info dict, bytes) of the device work-list image, for inspection."""
        info = _capi.BscWorklistInfo()
        _check(_capi.lib().bsc_plan_worklist(self._h, byref(info), None, 0))
        buf = ctypes.create_string_buffer(int(info.bytes))
        _check(_capi.lib().bsc_plan_worklist(self._h, byref(info), ctypes.cast(buf, c_void_p), int(info.bytes)))
        return {n: int(getattr(info, n)) for n, _ in info._fields_}, bytes(buf.raw)

    # -- device ------------------------------------------------------------------
    def bind(self, device=None, stream=None):
        """Allocate the plan's device region (torch memory) and upload the work list.

        Refused while a live Chain has captured this plan: its graph holds the
        current device region (work list, counters, workspace)."""
        if self._captured:
            raise BscError(-1, "plan is captured by a live Chain; rebinding would free the region its graph uses")
        torch = _torch()
        nbytes = self.device_bytes()
        dev = torch.empty(nbytes + 256, dtype=torch.uint8, device=device or "cuda")
        ptr = dev.data_ptr()
        pad = (-ptr) % 256
        _check(_capi.lib().bsc_plan_bind(self._h, c_void_p(ptr + pad), c_size_t(nbytes), _stream_handle(stream)))
        self._dev = dev
        return self

    @staticmethod
    def _check_tensor(torch, t, name, need, dtypes):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA/HIP torch tensor")
        if t.dtype not in dtypes:
            raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
        if not t.is_contiguous() or t.numel() < need:
            raise ValueError(f"{name} must be contiguous with at least {need} elements")

    def _operand_dtypes(self):
        """Accepted torch dtypes of (A and B, C)."""
        torch = _torch()
        if self.dtype == "f64":
            return (torch.float64,), (torch.float64,)
        if self.dtype == "f32":
            return (torch.float32,), (torch.float32,)
        return (torch.bfloat16, torch.int16, torch.uint16), (torch.float32,)

    def check_operands(self, A, B, C):
        """Device, dtype, contiguity and size of A, B, C (raises on a mismatch).
        Runs on every contraction, so the accepted dtypes are looked up once."""
        torch = _torch()
        dts = getattr(self, "_dtypes", None)
        if dts is None:
            dts = self._dtypes = self._operand_dtypes()
        ab, cd = dts
        self._check_tensor(torch, A, "A", self.a_elems, ab)
        self._check_tensor(torch, B, "B", self.b_elems, ab)
        self._check_tensor(torch, C, "C", self.c_elems, cd)

    def contract(self, A, B, C, stream=None):
        """Enqueue C (+)= A B on `stream` (default: torch's current stream)."""
        if self._dev is None:
            raise BscError(-8, "plan is not bound (call bind())")
        self.check_operands(A, B, C)
        _check(_capi.lib().bsc_contract(self._h, c_void_p(A.data_ptr()), c_void_p(B.data_ptr()),
                                        c_void_p(C.data_ptr()), _stream_handle(stream)))
        return C

    def contract_noalloc(self, A, B, C, stream=None):
        """Enqueue C (+)= A B without a bound device region (bsc_contract_noalloc):
        the plan's work list, workspace and partials go to the library's fixed
        per-GPU scratch array (64 MiB), so nothing is allocated.  Calls that
        overlap on one GPU race; the plan need not be bound."""
        self.check_operands(A, B, C)
        _check(_capi.lib().bsc_contract_noalloc(self._h, c_void_p(A.data_ptr()), c_void_p(B.data_ptr()),
                                                c_void_p(C.data_ptr()), _stream_handle(stream)))
        return C

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _capi.lib().bsc_plan_destroy(h)
            except Exception:
                pass
            self._h = None


def probe_mfma(dtype: str, iters: int, sink, stream=None) -> float:
    """Enqueue the matrix-core issue-rate probe (bsc_probe_mfma) on `stream`
    and return its flops; the caller times the launch.  `sink` is a device
    float32 tensor the kernel never writes."""
    f = ctypes.c_double()
    _check(_capi.lib().bsc_probe_mfma(DTYPES[dtype], int(iters), c_void_p(sink.data_ptr()), _stream_handle(stream),
                                      byref(f)))
    return f.value


class FusedPlan:
    """Two contractions planned as one launch (bsc_fused_plan): stage 1
    C1 = A1 B1 (`con1`), then stage 2 C2 (+)= C1 B2 (`con2`), where stage 2's
    A operand is C1's blocks with their rows and columns fused into one row
    index and B2 holds 1 x 1 blocks.  C1 is never formed: contract() reads
    A1, B1, B2 and writes C2 only."""

    def __init__(self, con1, con2, dtype: str = None, accumulate: bool = False, split: int = 0,
                 tile_cols: int = 0):
        L = _capi.lib()
        self.dtype = dtype or con1.dtype
        if self.dtype not in ("f64", "f32"):
            raise BscError(-7, "fused plans take f64 or f32")
        keep = _Keep()
        a1 = _plan_args(con1, self.dtype, "auto", keep)
        a2 = _plan_args(con2, self.dtype, "auto", keep)
        opt = _capi.BscOptions()
        L.bsc_options_default(byref(opt))
        opt.accumulate = int(bool(accumulate))
        opt.split_k = int(split)   # waves per output tile: 0 automatic (up to 4), 1 never split
        opt.tile_cols = int(tile_cols)   # a wave's output tile edge: 0 automatic, 16, 32 (fp32, <= 4 outputs)
        keep.arrays.append(opt)
        h = c_void_p()
        _check(L.bsc_fused_plan(*a1[:6], *a2[:6], DTYPES[self.dtype], byref(opt), byref(h)))
        self._h = h
        self.elems = {"A1": int(con1.A.buffer_elems), "B1": int(con1.B.buffer_elems),
                      "B2": int(con2.B.buffer_elems), "C2": int(con2.C.buffer_elems)}
        self._dev = None

    def device_bytes(self) -> int:
        n = c_size_t()
        _check(_capi.lib().bsc_fused_device_bytes(self._h, byref(n)))
        return int(n.value)

    def stats(self) -> dict:
        s = _capi.BscFusedStats()
        _check(_capi.lib().bsc_fused_stats(self._h, byref(s)))
        return {name: int(getattr(s, name)) for name, _ in s._fields_}

    def worklist(self):
        """(stats dict, bytes) of the device image, for host replay."""
        s = self.stats()
        buf = ctypes.create_string_buffer(max(1, s["device_bytes"]))
        _check(_capi.lib().bsc_fused_worklist(self._h, ctypes.cast(buf, c_void_p), c_size_t(s["device_bytes"])))
        return s, bytes(buf.raw[:s["device_bytes"]])

    def bind(self, device=None, stream=None):
        """Allocate the work-list region (torch memory) and upload it."""
        torch = _torch()
        nbytes = self.device_bytes()
        dev = torch.empty(nbytes + 256, dtype=torch.uint8, device=device or "cuda")
        ptr = dev.data_ptr()
        pad = (-ptr) % 256
        _check(_capi.lib().bsc_fused_bind(self._h, c_void_p(ptr + pad), c_size_t(nbytes), _stream_handle(stream)))
        self._dev = dev
        return self

    def contract(self, A1, B1, B2, C2, stream=None):
        """Enqueue C2 (+)= (A1 B1) B2 on `stream` (default: torch's current stream)."""
        if self._dev is None:
            raise BscError(-8, "plan is not bound (call bind())")
        torch = _torch()
        dt = torch.float64 if self.dtype == "f64" else torch.float32
        for name, t in (("A1", A1), ("B1", B1), ("B2", B2), ("C2", C2)):
            if not isinstance(t, torch.Tensor) or not t.is_cuda:
                raise TypeError(f"{name} must be a CUDA/HIP torch tensor")
            if t.dtype != dt:
                raise TypeError(f"{name} has dtype {t.dtype}, expected {dt}")
            if not t.is_contiguous() or t.numel() < self.elems[name]:
                raise ValueError(f"{name} must be contiguous with at least {self.elems[name]} elements")
        _check(_capi.lib().bsc_fused_contract(self._h, c_void_p(A1.data_ptr()), c_void_p(B1.data_ptr()),
                                              c_void_p(B2.data_ptr()), c_void_p(C2.data_ptr()),
                                              _stream_handle(stream)))
        return C2

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _capi.lib().bsc_fused_destroy(h)
            except Exception:
                pass
            self._h = None


class StreamPlan(FusedPlan):
    """One contraction C (+)= A B (`con`) planned for the fused launch's
    register-stream kernel (bsc_stream_plan): every C block computed by waves
    of 16 x 16 (fp32: possibly 32 x 32) tiles that stream the block's products
    through registers and write it directly.  f64 and f32 only; bind, stats
    and worklist as for FusedPlan; contract(A, B, C)."""

    def __init__(self, con, dtype: str = None, accumulate: bool = False, tile_cols: int = 0):
        L = _capi.lib()
        self.dtype = dtype or con.dtype
        if self.dtype not in ("f64", "f32"):
            raise BscError(-7, "stream plans take f64 or f32")
        keep = _Keep()
        a = _plan_args(con, self.dtype, "auto", keep)
        opt = _capi.BscOptions()
        L.bsc_options_default(byref(opt))
        opt.accumulate = int(bool(accumulate))
        opt.tile_cols = int(tile_cols)
        keep.arrays.append(opt)
        h = c_void_p()
        _check(L.bsc_stream_plan(*a[:6], DTYPES[self.dtype], byref(opt), byref(h)))
        self._h = h
        self.elems = {"A": int(con.A.buffer_elems), "B": int(con.B.buffer_elems), "C": int(con.C.buffer_elems)}
        self._dev = None

    def contract(self, A, B, C, stream=None):
        """Enqueue C (+)= A B on `stream` (default: torch's current stream)."""
        if self._dev is None:
            raise BscError(-8, "plan is not bound (call bind())")
        torch = _torch()
        dt = torch.float64 if self.dtype == "f64" else torch.float32
        for name, t in (("A", A), ("B", B), ("C", C)):
            if not isinstance(t, torch.Tensor) or not t.is_cuda:
                raise TypeError(f"{name} must be a CUDA/HIP torch tensor")
            if t.dtype != dt:
                raise TypeError(f"{name} has dtype {t.dtype}, expected {dt}")
            if not t.is_contiguous() or t.numel() < self.elems[name]:
                raise ValueError(f"{name} must be contiguous with at least {self.elems[name]} elements")
        _check(_capi.lib().bsc_fused_contract(self._h, c_void_p(A.data_ptr()), c_void_p(B.data_ptr()), None,
                                              c_void_p(C.data_ptr()), _stream_handle(stream)))
        return C


def best_plan(con, dtype: str = None, accumulate: bool = False, **plan_kw):
    """The plan the library expects to run `con` fastest: a StreamPlan where
    bsc_stream_plan accepts the contraction and reports it preferred
    (stream_preferred), else a grouped Plan (bsc_plan).  Both are unbound."""
    dt = dtype or con.dtype
    if dt in ("f64", "f32"):
        try:
            sp = StreamPlan(con, dtype=dt, accumulate=accumulate)
        except BscError:
            sp = None
        if sp is not None and sp.stats()["stream_preferred"]:
            return sp
    return Plan(con, dtype=dt, accumulate=accumulate, **plan_kw)


class Chain:
    """A fixed sequence of contractions [(plan, A, B, C), ...] captured once
    into a HIP graph and replayed with one launch (bsc_chain_*).  The plans
    must be bound and every tensor must pass the checks Plan.contract applies
    (device, dtype, contiguity, size), since the graph replays the addresses
    without looking again.  The chain keeps references to the plans, their
    device regions and the tensors, whose addresses the graph holds, and a
    captured plan refuses bind() until the chain is released."""

    def __init__(self, steps):
        self._h = None
        self._plans = []
        steps = list(steps)
        if not steps:
            raise BscError(-1, "empty chain")
        for p, A, B, C in steps:
            if p._dev is None:
                raise BscError(-8, "plan is not bound (call bind())")
            p.check_operands(A, B, C)
        n = len(steps)
        arr = lambda xs: (c_void_p * n)(*xs)
        plans = arr([p._h.value for p, _, _, _ in steps])
        a = arr([A.data_ptr() for _, A, _, _ in steps])
        b = arr([B.data_ptr() for _, _, B, _ in steps])
        c = arr([C.data_ptr() for _, _, _, C in steps])
        h = c_void_p()
        _check(_capi.lib().bsc_chain_create(plans, a, b, c, n, byref(h)))
        self._h = h
        # plans, their device regions and the tensors must outlive the graph
        self._keep = [(p, p._dev, A, B, C) for p, A, B, C in steps]
        self._plans = [p for p, _, _, _ in steps]
        for p in self._plans:
            p._captured += 1

    def launch(self, stream=None):
        """Enqueue one replay on `stream` (default: torch's current stream)."""
        if self._h is None:
            raise BscError(-1, "chain was released")
        _check(_capi.lib().bsc_chain_launch(self._h, _stream_handle(stream)))

    def release(self):
        """Destroy the graph; the plans may be rebound afterwards.  The caller
        must have synchronised any replay still in flight."""
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _capi.lib().bsc_chain_destroy(h)
            except Exception:
                pass
        self._h = None
        for p in getattr(self, "_plans", []):
            p._captured -= 1
        self._plans = []
        self._keep = []

    def __del__(self):
        self.release()


class PlanCache:
    """Host-side cache of plans keyed by their complete inputs (bsc_plan_cache_*).
    Pass it to Plan(..., cache=...); every Plan it yields is a separate,
    unbound copy."""

    def __init__(self, capacity: int = 64):
        h = c_void_p()
        _check(_capi.lib().bsc_plan_cache_create(int(capacity), byref(h)))
        self._h = h

    def stats(self) -> dict:
        hits, misses, entries = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(_capi.lib().bsc_plan_cache_stats(self._h, byref(hits), byref(misses), byref(entries)))
        return {"hits": hits.value, "misses": misses.value, "entries": entries.value}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            try:
                _capi.lib().bsc_plan_cache_destroy(h)
            except Exception:
                pass
            self._h = None
