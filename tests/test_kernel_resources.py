"""Register and scratch use of every device kernel, as the compiler reported
it for the last build (kernel-resource-usage remarks recorded by
block_sparse_tensor_amd.build).  A kernel that spills to scratch memory pays
a private-memory round trip in its inner loop, so no kernel may use scratch
beyond the two known cases: the four-wave wide bf16 tile (an option, 256 x 256
output per workgroup with all accumulators in registers; its eight-wave form
has none) and the fp32 general-tile
instance compiled for four waves per SIMD (12 bytes per lane; compiled for
three it was measured slower)."""
import json
import os
import subprocess

import pytest

from block_sparse_tensor_amd import build as B

ALLOWED_SCRATCH = {
    "grouped_contract_wide<": 112,
    "grouped_contract_narrow<float, float, float, 1>": 12,
}


def _load():
    if not os.path.exists(B.RESOURCES):
        pytest.skip("no build record: run python -m block_sparse_tensor_amd.build")
    with open(B.RESOURCES) as f:
        rec = json.load(f)
    if rec.get("sources") != B.source_hash():
        pytest.skip("the build record is from other sources: rebuild first")
    names = list(rec["kernels"])
    dem = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True).stdout.splitlines()
    if len(dem) != len(names):
        dem = names
    return {d: rec["kernels"][n] for n, d in zip(names, dem)}


def test_every_kernel_reported():
    k = _load()
    for name in ("pack_gather<unsigned short>", "fused_contract<float, 4, 2>", "fused_contract<double, 16, 1>",
                 "grouped_contract<unsigned short, float, float, 2>", "grouped_contract<double, double, double, 1>",
                 "grouped_contract_narrow<float, float, float, 0>", "probe_bf16", "grouped_contract_wide8"):
        assert any(name in d for d in k), name
    assert len(k) >= 27


def test_no_unexpected_scratch():
    k = _load()
    for d, r in k.items():
        limit = next((v for key, v in ALLOWED_SCRATCH.items() if key in d), 0)
        assert r.get("scratch", 0) <= limit, (d, r)
        assert r.get("vgpr_spill", 0) == 0 or limit > 0, (d, r)


def test_bench_kernel_keeps_two_waves_per_simd():
    """The bf16 direct-to-LDS tile needs two workgroups per CU (two waves per
    SIMD) to overlap one wave's copies with the other's matrix-core work."""
    k = _load()
    for d, r in k.items():
        if "grouped_contract<unsigned short, float, float," in d or "grouped_contract_wide8" in d:
            assert r["occupancy"] >= 2, (d, r)
