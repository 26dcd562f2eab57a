"""The host planner built on its own with AddressSanitizer and
UndefinedBehaviorSanitizer, running its coverage and bookkeeping checks
(tests/sanitize/plan_check.cpp) on fixed and seeded random metadata. The
planner is plain C++ with no HIP, so g++ builds it for the host alone."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gqa_attention_agentic_amd", "csrc")


def test_planner_under_asan_and_ubsan(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path / "plan_check")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "sanitize", "plan_check.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "plan_check ok" in r.stdout
