"""The launch planner and the argument checks of the C ABI (csrc/cf_plan.h)
on the CPU: tests/host_plan_check.cpp against fake devices, built with g++
under AddressSanitizer and UndefinedBehaviorSanitizer (host code only; no HIP
header, no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host_plan_check.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "b2bgemm_stage_stream_amd", "csrc"), SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "planner ok" in r.stdout
