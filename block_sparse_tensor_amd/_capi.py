"""ctypes declarations mirroring include/bsc.h."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_int32, c_int64, c_size_t, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
# BSC_LIBRARY may name another build of the same interface (the host-only
# planner library of a sanitizer run, whose device entry points return
# BSC_ERR_UNSUPPORTED); by default the in-tree HIP library is loaded.
LIB_PATH = os.environ.get("BSC_LIBRARY") or os.path.join(_HERE, "libbsc.so")

STATUS = {
    0: "BSC_OK", -1: "BSC_ERR_ARG", -2: "BSC_ERR_CHARGE", -3: "BSC_ERR_SHAPE", -4: "BSC_ERR_BOUNDS",
    -5: "BSC_ERR_OVERLAP", -6: "BSC_ERR_MISSING_OUTPUT", -7: "BSC_ERR_UNSUPPORTED", -8: "BSC_ERR_NOT_BOUND",
    -9: "BSC_ERR_DEVICE_BYTES", -10: "BSC_ERR_HIP",
}

EXPORTED = ["bsc_options_default", "bsc_plan", "bsc_plan_device_bytes", "bsc_plan_bind", "bsc_contract",
            "bsc_plan_stats", "bsc_plan_export", "bsc_plan_worklist", "bsc_plan_destroy", "bsc_status_string",
            "bsc_last_error", "bsc_chain_create", "bsc_chain_launch", "bsc_chain_destroy", "bsc_plan_cache_create",
            "bsc_plan_cached", "bsc_plan_cache_stats", "bsc_plan_cache_destroy", "bsc_plan_layout",
            "bsc_contract_noalloc", "bsc_fused_plan", "bsc_fused_device_bytes", "bsc_fused_bind",
            "bsc_fused_contract", "bsc_fused_stats", "bsc_fused_worklist", "bsc_fused_destroy", "bsc_probe_mfma",
            "bsc_stream_plan"]


class BscIndex(ctypes.Structure):
    _fields_ = [("nkeys", c_int32), ("nq", c_int32), ("charge", POINTER(c_int32)),
                ("dim", POINTER(c_int64)), ("inner", POINTER(c_int64))]


class BscOperand(ctypes.Structure):
    _fields_ = [("nblocks", c_int64), ("row_key", POINTER(c_int32)), ("col_key", POINTER(c_int32)),
                ("offset", POINTER(c_int64)), ("row_stride", POINTER(c_int64)), ("col_stride", POINTER(c_int64)),
                ("flux", POINTER(c_int32)), ("buffer_elems", c_int64)]


class BscOptions(ctypes.Structure):
    _fields_ = [("launch_mode", c_int32), ("layout_policy", c_int32), ("accumulate", c_int32),
                ("grid_limit", c_int32), ("t_launch_us", c_double), ("t_seg_us", c_double),
                ("pack_gbps", c_double), ("tile_gflops", c_double), ("split_k", c_int32), ("tile_rows", c_int32),
                ("tile_cols", c_int32)]


class BscStats(ctypes.Structure):
    _fields_ = [("triples", c_int64), ("c_blocks", c_int64), ("zero_blocks", c_int64), ("groups", c_int64),
                ("zero_groups", c_int64), ("axis", c_int32), ("dtype", c_int32),
                ("mode_count", (c_int64 * 3) * 3), ("runs", c_int64), ("items", c_int64),
                ("items_by_class", c_int64 * 6), ("launches_per_contract", c_int64),
                ("launches_per_sector", c_int64), ("useful_flops", c_int64), ("alg_bytes", c_int64),
                ("pack_bytes", c_int64), ("device_bytes", c_int64), ("tail_triples", c_int64),
                ("launches_issued", c_int64), ("grid", c_int32), ("split_tiles", c_int32),
                ("predicted_us", c_double), ("pack_gain_seg_us", c_double), ("pack_gain_pad_us", c_double),
                ("pack_cost_us", c_double), ("pack_gain_align_us", c_double),
                ("wide_only", c_int64)]


class BscWorklistInfo(ctypes.Structure):
    _fields_ = [(n, c_int64) for n in ("n_groups", "n_runs", "n_apieces", "n_bpieces", "n_cpieces", "n_tasks",
                                        "n_dense", "off_groups", "off_runs", "off_apieces", "off_bpieces",
                                        "off_cpieces", "off_tasks", "off_dense", "n_packs", "n_pack_tasks",
                                        "off_packs", "off_pack_tasks", "off_workspace", "workspace_elems",
                                        "bytes", "n_launches", "n_counters", "off_counters",
                                        "off_partials", "partial_elems", "n_tail", "off_tail")]


class BscFusedStats(ctypes.Structure):
    _fields_ = [(n, c_int64) for n in ("groups", "channels", "outputs", "terms", "items", "launches_per_contract",
                                        "useful_flops", "stage1_flops", "alg_bytes", "device_bytes",
                                        "launches_issued", "off_groups", "off_chans", "off_outs", "off_widx",
                                        "off_tasks", "outs_per_task", "off_parts", "n_parts", "off_pchans",
                                        "n_pchans", "tile_blocks", "stream", "off_ones", "longest_chunks",
                                        "stream_preferred")]


_lib = None


def lib():
    """Load libbsc.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m block_sparse_tensor_amd.build`")
        # torch (which supplies device memory and streams) ships its own HIP
        # runtime under the same sonames as the system one the library links;
        # whichever is loaded first serves the whole process.  Importing torch
        # first makes the library bind to torch's runtime, so both see the
        # same devices, streams and allocations (loaded the other way round,
        # the library's calls found no device).
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.bsc_options_default.argtypes = [POINTER(BscOptions)]
        L.bsc_options_default.restype = None
        L.bsc_plan.argtypes = [POINTER(BscIndex)] * 3 + [POINTER(BscOperand)] * 3 + [c_int32, c_int32,
                                                                                   POINTER(BscOptions), POINTER(c_void_p)]
        L.bsc_plan.restype = c_int32
        L.bsc_plan_device_bytes.argtypes = [c_void_p, POINTER(c_size_t)]
        L.bsc_plan_device_bytes.restype = c_int32
        L.bsc_plan_bind.argtypes = [c_void_p, c_void_p, c_size_t, c_void_p]
        L.bsc_plan_bind.restype = c_int32
        L.bsc_contract.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.bsc_contract.restype = c_int32
        L.bsc_contract_noalloc.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.bsc_contract_noalloc.restype = c_int32
        L.bsc_plan_stats.argtypes = [c_void_p, POINTER(BscStats)]
        L.bsc_plan_stats.restype = c_int32
        L.bsc_plan_export.argtypes = [c_void_p, POINTER(c_int32), POINTER(c_int32), POINTER(c_int32)]
        L.bsc_plan_export.restype = c_int32
        L.bsc_plan_worklist.argtypes = [c_void_p, POINTER(BscWorklistInfo), c_void_p, c_size_t]
        L.bsc_plan_worklist.restype = c_int32
        L.bsc_plan_destroy.argtypes = [c_void_p]
        L.bsc_plan_destroy.restype = None
        L.bsc_status_string.argtypes = [c_int32]
        L.bsc_status_string.restype = c_char_p
        L.bsc_last_error.argtypes = []
        L.bsc_last_error.restype = c_char_p
        L.bsc_chain_create.argtypes = [POINTER(c_void_p), POINTER(c_void_p), POINTER(c_void_p), POINTER(c_void_p),
                                       c_int32, POINTER(c_void_p)]
        L.bsc_chain_create.restype = c_int32
        L.bsc_chain_launch.argtypes = [c_void_p, c_void_p]
        L.bsc_chain_launch.restype = c_int32
        L.bsc_chain_destroy.argtypes = [c_void_p]
        L.bsc_chain_destroy.restype = None
        L.bsc_plan_cache_create.argtypes = [c_int32, POINTER(c_void_p)]
        L.bsc_plan_cache_create.restype = c_int32
        L.bsc_plan_cached.argtypes = [c_void_p] + L.bsc_plan.argtypes + [POINTER(c_int32)]
        L.bsc_plan_cached.restype = c_int32
        L.bsc_plan_cache_stats.argtypes = [c_void_p, POINTER(c_int64), POINTER(c_int64), POINTER(c_int64)]
        L.bsc_plan_cache_stats.restype = c_int32
        L.bsc_plan_cache_destroy.argtypes = [c_void_p]
        L.bsc_plan_cache_destroy.restype = None
        L.bsc_plan_layout.argtypes = L.bsc_plan.argtypes[:-1] + [c_int32, c_int64, POINTER(c_int64), POINTER(c_int64),
                                                                POINTER(c_int64), POINTER(c_int64)]
        L.bsc_plan_layout.restype = c_int32
        L.bsc_fused_plan.argtypes = ([POINTER(BscIndex)] * 3 + [POINTER(BscOperand)] * 3) * 2 + [
            c_int32, POINTER(BscOptions), POINTER(c_void_p)]
        L.bsc_fused_plan.restype = c_int32
        L.bsc_stream_plan.argtypes = [POINTER(BscIndex)] * 3 + [POINTER(BscOperand)] * 3 + [
            c_int32, POINTER(BscOptions), POINTER(c_void_p)]
        L.bsc_stream_plan.restype = c_int32
        L.bsc_fused_device_bytes.argtypes = [c_void_p, POINTER(c_size_t)]
        L.bsc_fused_device_bytes.restype = c_int32
        L.bsc_fused_bind.argtypes = [c_void_p, c_void_p, c_size_t, c_void_p]
        L.bsc_fused_bind.restype = c_int32
        L.bsc_fused_contract.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.bsc_fused_contract.restype = c_int32
        L.bsc_fused_stats.argtypes = [c_void_p, POINTER(BscFusedStats)]
        L.bsc_fused_stats.restype = c_int32
        L.bsc_fused_worklist.argtypes = [c_void_p, c_void_p, c_size_t]
        L.bsc_fused_worklist.restype = c_int32
        L.bsc_probe_mfma.argtypes = [c_int32, c_int32, c_void_p, c_void_p, POINTER(c_double)]
        L.bsc_probe_mfma.restype = c_int32
        L.bsc_fused_destroy.argtypes = [c_void_p]
        L.bsc_fused_destroy.restype = None
        _lib = L
    return _lib
