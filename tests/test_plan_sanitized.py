"""ra_ring_plan under AddressSanitizer and UndefinedBehaviorSanitizer.

The planner is plain host C++, so tests/sanitize/plan_sweep.cpp builds it
with g++ (host code only) and sweeps every layout, order, rank and P,
including invalid ones, with exact-size and one-short item buffers.  Any
out-of-bounds write or undefined behaviour aborts the sweep.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_sweep_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_sweep"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "sanitize", "plan_sweep.cpp"),
           os.path.join(ROOT, "ring_blockwise_softmax_amd", "csrc", "ra_plan.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.startswith("ok")
