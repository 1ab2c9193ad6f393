"""The symmetric product kernel's workgroup -> tile map (csrc/gemm_sym.h,
symk::sym_tile), built with hipcc as host code by tests/host/sym_map_check.hip:
a bijection onto the diagonal tiles and the halves above the diagonal for every
T x T grid up to T = 64, and the XCD block partition's row-block bound.  No GPU
is involved."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "orthonormal_optimizer_update_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_sym_tile_map(tmp_path):
    exe = tmp_path / "sym_map_check"
    cmd = [HIPCC, "-O1", "-std=c++17", "--offload-arch=gfx950", "-I", CSRC,
           os.path.join(HERE, "host", "sym_map_check.hip"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "0 failures" in run.stdout
