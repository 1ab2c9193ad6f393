"""Dion parity at large ranks on dense inputs (no block structure), at sizes the
fp64 oracle finishes in seconds, and the plain dion_step entry point.

* 8192 x 8192 at r = 2048 (rank fraction 1/4) with the planted rank-32
  gradient of the 4096 x 4096 workload's recipe, two steps, each side carrying
  its own state.
* r = 4096 on 4096 x 12288 (r equal to the row count: P~ = B Q is square) and
  12288 x 4096 (r equal to the column count: Q is square).
Every entry of the Gram matrix, of its Cholesky factor and of every trailing
update is dense here, unlike the block-structured full-size cases."""

import numpy as np
import pytest
import torch

import oracle
from orthonormal_optimizer_update_amd import api, synth

from parity_util import TOL, note, rel, run_dion_parity, to_dev, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()
    torch.cuda.set_device(0)


def test_dion_dense_square_8192_r2048_planted():
    wl = synth.WORKLOADS[2]
    m = n = 8192
    r = 2048
    X = synth.weight(20, m, n, "bf16")
    Q0 = synth.right_factor0(20, n, r)
    S = synth.planted(20, m, n, 32, wl["planted_ratio"])
    Gs = [synth.gradient(20, m, n, t, "bf16", planted_part=S) for t in (1, 2)]
    del S
    worst, recs = run_dion_parity(X, Gs, Q0, wl["mu"], wl["lr"], "bf16", label="dense r2048")
    print(worst, recs)
    assert max(worst.values()) <= TOL["bf16"], recs


@pytest.mark.parametrize("m,n,steps", [(4096, 12288, 2), (12288, 4096, 1)])
def test_dion_dense_r4096(m, n, steps):
    r = 4096
    X = synth.weight(21, m, n, "bf16")
    Q0 = synth.right_factor0(21, n, r)
    S = synth.planted(21, m, n, 32, 10.0)
    Gs = [synth.gradient(21, m, n, t, "bf16", planted_part=S) for t in range(1, steps + 1)]
    del S
    worst, recs = run_dion_parity(X, Gs, Q0, 0.95, 0.01, "bf16", label="dense r4096")
    print(m, n, worst, recs)
    assert max(worst.values()) <= TOL["bf16"], recs


@pytest.mark.parametrize("m,n,r,dtype", [(300, 200, 37, "f32"), (1024, 1024, 512, "bf16"),
                                         (2048, 1024, 256, "bf16")])
def test_plain_dion_step_entry_point(m, n, r, dtype):
    """dion_step (no scale, no optional outputs) gives the bits of dion_step_ex
    with scale 1, and matches the oracle."""
    X, G, Q0 = synth.small_case(50 + r, m, n, r, dtype, planted_rank=4)
    res = {}
    for entry in ("plain", "ex"):
        tX, tG = to_dev(X, dtype), to_dev(G, dtype)
        tM = torch.zeros(m, n, device="cuda")
        tQ = to_dev(Q0, "f32")
        ws = api.workspace(api.dion_workspace_size(m, n, r), "cuda")
        note(f"dion {entry} entry {m}x{n} r={r} {dtype}")
        if entry == "plain":
            st = api.lib().dion_step(api.mat(tX), api.mat(tG), api.mat(tM), api.mat(tQ), r, 0.95,
                                     0.01, api._ptr(ws), ws.numel(), api._stream_ptr(tX.device))
        else:
            st = api.lib().dion_step_ex(api.mat(tX), api.mat(tG), api.mat(tM), api.mat(tQ), r,
                                        0.95, 0.01, 1.0, None, None, None, api._ptr(ws),
                                        ws.numel(), api._stream_ptr(tX.device))
        assert st == 0, api.status_str(st)
        torch.cuda.synchronize()
        res[entry] = (to_host(tX), to_host(tM), to_host(tQ))
    for a, b in zip(res["plain"], res["ex"]):
        assert np.array_equal(a, b)
    ref = oracle.dion_step(X, G, np.zeros((m, n)), Q0, 0.95, 0.01, x_dtype=dtype)
    Xg, Mg, Qg = res["plain"]
    errs = dict(X=rel(Xg, ref["X_exact"]), M=rel(Mg, ref["M"]), Q=rel(Qg, ref["Q"]))
    print(errs)
    assert max(errs.values()) <= TOL[dtype], errs
