"""Block-sparse contraction engine for AMD Instinct MI355X (gfx950).

C[m,n] = sum_k A[m,k] B[k,n] over symmetry sectors, planned once on the host
(single-axis coalescing into strided views) and run as one grouped HIP launch.
The compute lives in libbsc.so (include/bsc.h); this package only marshals
arguments and uses PyTorch for device memory and streams.
"""
from .engine import (AXES, DTYPES, BscError, Chain, FusedPlan, Plan, PlanCache, StreamPlan,  # noqa: F401
                     best_plan, plan_layout, probe_mfma)
from ._capi import LIB_PATH  # noqa: F401
from . import layouts  # noqa: F401,E402
