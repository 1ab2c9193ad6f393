"""Workspace planning and argument validation (csrc/plan.cpp) built on the host
with g++ under AddressSanitizer and UndefinedBehaviorSanitizer, driven by
tests/host/plan_check.cpp: region layout and split-K coverage over a grid of
shapes up to the largest accepted dimensions, and a table of argument errors.
No GPU and no HIP are involved."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "orthonormal_optimizer_update_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_plan_and_validation_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", CSRC, os.path.join(HERE, "host", "plan_check.cpp"), os.path.join(CSRC, "plan.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout
