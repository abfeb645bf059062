"""bench.py's host-side contract, checked without a GPU: it refuses more than
one GPU, refuses to run without one (no CPU fallback), and the committed
counter record it reads for roofline.traffic belongs to the current sources of
the grouped launch."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.skipif(os.environ.get("HIP_VISIBLE_DEVICES") is None and os.path.exists("/dev/kfd"),
                    reason="a GPU may be present")
def test_no_gpu_no_fallback():
    r = _run("--steps", "1", "--warmup", "0", "--no-cpu")
    assert r.returncode != 0
    assert "needs a GPU" in (r.stderr + r.stdout)


def test_traffic_record_matches_sources():
    """profiles/grouped_contract_traffic.md holds the FETCH_SIZE / WRITE_SIZE
    bytes of the bench launch taken at the current grouped-launch sources."""
    b = bench.measured_traffic("blockdiag_bf16", 8, 0)
    assert b is not None, "counter record is from other sources: retake the profiles"
    assert 65_000_000 <= b <= 200_000_000


def test_record_hash_ignores_comments():
    a = "int a; // one\n// two\n/* three\nfour */ int b;\n"
    b = "int a; // changed\n\n/* x */ int b;\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only("int a = 1;") != bench._code_only("int a = 2;")
