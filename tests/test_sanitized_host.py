"""The host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds the host-only planner library (the planner, plan cache and layout
sources with a device-runtime stub whose entry points return
BSC_ERR_UNSUPPORTED) with -fsanitize=address,undefined, then runs the host
tests of the C-ABI against it in a child process (the sanitizer runtime
preloaded, leak detection off for the interpreter's own allocations).  Any
sanitizer report, or any failing test, fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST_TESTS = ["tests/test_capi_host.py", "tests/test_worklist_emulation.py", "tests/test_plan_cache.py",
              "tests/test_layouts.py", "tests/test_fused_host.py"]


def _runtime(name):
    r = subprocess.run(["gcc", f"-print-file-name={name}"], stdout=subprocess.PIPE, text=True)
    path = r.stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.slow
def test_host_planner_sanitized():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("gcc's AddressSanitizer runtime is not installed")
    sys.path.insert(0, ROOT)
    from block_sparse_tensor_amd import build
    out = os.path.join(build.BUILD, "libbsc_host_asan_ubsan.so")
    build.build_host(["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                      "-fno-sanitize-recover=undefined"], out=out)
    # the C++ runtime preloaded too, so the sanitizer's exception interceptor finds it
    stdcxx = _runtime("libstdc++.so")
    env = dict(os.environ, BSC_LIBRARY=out, LD_PRELOAD=" ".join(x for x in (asan, stdcxx) if x),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        *HOST_TESTS], cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       text=True, timeout=900)
    tail = r.stdout[-4000:]
    assert "AddressSanitizer" not in r.stdout and "runtime error:" not in r.stdout, tail
    assert r.returncode == 0, tail
    assert " passed" in tail, tail
