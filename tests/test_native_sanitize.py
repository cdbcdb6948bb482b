"""Host sanitizer run of the planners: tests/native/plan_fuzz.cpp and the
library's plan.cpp built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer (any report aborts), then driven with random and
hostile arguments -- huge and overflowing sizes, bad indices, short output
arrays -- checking layout invariants on every plan made (CPU only)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "plan_fuzz")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "sharded_bucket_plan_amd", "csrc"),
           "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "native", "plan_fuzz.cpp"),
           os.path.join(ROOT, "sharded_bucket_plan_amd", "csrc", "plan.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "8000"], capture_output=True, text=True, timeout=240, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "plans made" in r.stdout
