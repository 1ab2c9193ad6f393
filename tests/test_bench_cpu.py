"""bench.py's command-line contract, on the host: more than one GPU is refused
with a message, before anything touches a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_bench_models():
    sys.path.insert(0, ROOT)
    import bench
    # 26 bytes per element of the 4096^2 matrix plus 16 (m + n) r of factors
    nbytes, flops = bench.dion_model(4096, 4096, 256)
    assert nbytes == 26 * 4096 * 4096 + 16 * 8192 * 256
    assert flops == 8 * 4096 * 4096 * 256 + 2 * 4096 * 256 ** 2 + 3 * 4096 * 256
    # Newton-Schulz on the wide orientation: 4 m^2 n + 2 m^3 per iteration
    _, f = bench.ns_model(8192, 2048, iters=1)
    assert f == 4 * 2048 ** 2 * 8192 + 2 * 2048 ** 3
