"""Host sanitizer runs of the library's host code, built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts), CPU only:

- tests/native/plan_fuzz.cpp drives the planners and plan queries with random
  and hostile arguments (huge and overflowing sizes, bad indices, short output
  arrays) and checks layout invariants on every plan made;
- tests/native/layout_fuzz.cpp executes the copy-segment lists of pack,
  unpack, shard_of and gather on host buffers with guard bands (the GPU copy
  kernel runs these lists as they are), and checks the run tables."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


CSRC = os.path.join(ROOT, "sharded_bucket_plan_amd", "csrc")


def _build_and_run(tmp_path, driver, sources, iters, expect):
    exe = str(tmp_path / driver)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", "/opt/rocm/include",
           os.path.join(ROOT, "tests", "native", driver + ".cpp")]
    cmd += [os.path.join(CSRC, s) for s in sources] + ["-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, str(iters)], capture_output=True, text=True, timeout=240, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert expect in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_under_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, "plan_fuzz", ["plan.cpp"], 8000, "plans made")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_layout_segments_under_asan_ubsan(tmp_path):
    _build_and_run(tmp_path, "layout_fuzz", ["layout_host.cpp", "plan.cpp"], 12000, "ok")
