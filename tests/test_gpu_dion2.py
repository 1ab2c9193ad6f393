"""Dion2 through the C-ABI against the fp64 oracle.

The selection is an integer decision taken on fp32 row norms on the GPU and on
fp64 ones in the oracle, so it is checked for validity (every selected row's
norm at least every other row's, to fp32 accuracy, in descending order), and the
oracle then runs on the GPU's selection; outputs are compared element by element
at the dtype's tolerance.  Rows that are not selected must come out exactly:
X untouched and M' = fl32(M + G)."""

import numpy as np
import pytest
import torch

import oracle
from orthonormal_optimizer_update_amd import api, synth

from parity_util import TOL, note, rel, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()
    torch.cuda.set_device(0)


def gpu_dion2(X, G, M, k, mu, lr, dtype, scale=1.0, steps=5, abc=None):
    """One HIP Dion2 step on host arrays; dX comes from a twin call with X = 0
    (with bf16 weights, X's own rounding would otherwise swamp the update)."""
    out = {}
    for twin in (False, True):
        tX = to_dev(np.zeros_like(X) if twin else X, dtype)
        tG, tM = to_dev(G, dtype), to_dev(M, "f32")
        sel = torch.full((k,), -1, dtype=torch.int32, device="cuda")
        api.dion2_step(tX, tG, tM, k, mu, lr, scale, steps=steps, abc=abc, selected=sel)
        torch.cuda.synchronize()
        res = dict(X=to_host(tX), M=to_host(tM), S=sel.cpu().numpy().astype(np.int64))
        if twin:
            assert np.array_equal(res["S"], out["S"]) and np.array_equal(res["M"], out["M"])
            out["dX"] = res["X"]
        else:
            out.update(res)
    return out


def check_selection(B, S, k):
    """S: k distinct rows, norms non-increasing, and no other row larger (fp32)."""
    assert len(S) == k and len(set(S.tolist())) == k
    assert S.min() >= 0 and S.max() < B.shape[0]
    sq = np.einsum("ij,ij->i", B, B)
    tol = 1e-5 * sq.max()
    assert np.all(np.diff(sq[S]) <= tol)
    rest = np.setdiff1d(np.arange(B.shape[0]), S)
    if rest.size:
        assert sq[rest].max() <= sq[S].min() + tol


def run_dion2_parity(X, Gs, M0, k, mu, lr, dtype, scale=1.0, label=""):
    """Each side carries its own state; the oracle follows the GPU's selection."""
    Xg, Mg = X.astype(np.float64), M0.astype(np.float64)
    Xo, Mo = Xg.copy(), Mg.copy()
    worst = {}
    for t, G in enumerate(Gs):
        m, n = X.shape
        note(f"dion2 {label} {m}x{n} k={k} {dtype} step {t + 1}")
        gpu = gpu_dion2(Xg, G, Mg, k, mu, lr, dtype, scale)
        B = Mg + G.astype(np.float64)
        check_selection(B, gpu["S"], k)
        ref = oracle.dion2_step(Xo, G, Mo, k, mu, lr, scale, x_dtype=dtype, selected=gpu["S"])
        rest = np.setdiff1d(np.arange(m), gpu["S"])
        # untouched rows: X as it was, M' = M + G rounded to fp32
        assert np.array_equal(gpu["X"][rest], Xg[rest])
        want = (Mg[rest].astype(np.float32) + G[rest].astype(np.float32)).astype(np.float64)
        assert np.array_equal(gpu["M"][rest], want)
        assert np.all(gpu["dX"][rest] == 0)
        errs = dict(X=rel(gpu["X"], ref["X_exact"]), M=rel(gpu["M"], ref["M"]),
                    dX=rel(gpu["dX"], ref["dX"]))
        for key, v in errs.items():
            worst[key] = max(worst.get(key, 0.0), v)
        Xg, Mg = gpu["X"], gpu["M"]
        Xo, Mo = ref["X"], ref["M"]
    return worst


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("m,n,k", [(96, 160, 24), (300, 100, 75), (64, 333, 64), (200, 96, 1),
                                   (512, 768, 128)])
def test_dion2_small(m, n, k, dtype):
    X, G1, _ = synth.small_case(200 + k, m, n, 1, dtype, planted_rank=4)
    Gs = [G1] + [synth.gradient(1200 + k, m, n, t, dtype) for t in (2, 3)]
    worst = run_dion2_parity(X, Gs, np.zeros((m, n)), k, 0.95, 0.02, dtype, scale=1.3, label="small")
    print(m, n, k, dtype, worst)
    # the update rows carry the Newton-Schulz precision of their dtype
    assert worst["dX"] <= TOL[dtype] and worst["X"] <= TOL[dtype]
    assert worst["M"] <= TOL["f32"]


def test_dion2_square_4096_planted():
    """The 4096 x 4096 bf16 workload, k = 1024 rows (fraction 1/4), two steps."""
    wl = synth.WORKLOADS[2]
    X = synth.weight(2, 4096, 4096, "bf16")
    S = synth.planted(2, 4096, 4096, 32, wl["planted_ratio"])
    Gs = [synth.gradient(2, 4096, 4096, t, "bf16", planted_part=S) for t in (1, 2)]
    worst = run_dion2_parity(X, Gs, np.zeros((4096, 4096)), 1024, wl["mu"], wl["lr"], "bf16",
                             label="cfg2")
    print(worst)
    assert worst["dX"] <= TOL["bf16"] and worst["X"] <= TOL["bf16"]
    assert worst["M"] <= TOL["f32"]


def test_dion2_special_cases():
    m, n = 128, 256
    X, G, _ = synth.small_case(210, m, n, 1, "f32")
    M0 = synth.gradient(211, m, n, 1, "f32")
    note("dion2 mu=1, lr=0")
    gpu = gpu_dion2(X, G, M0, 32, 1.0, 0.0, "f32")
    assert np.array_equal(gpu["X"], X.astype(np.float64))
    assert np.array_equal(gpu["M"], (M0.astype(np.float32) + G.astype(np.float32)).astype(np.float64))
    note("dion2 mu=0, k=m")
    gpu = gpu_dion2(X, G, M0, m, 0.0, 0.05, "f32")
    assert sorted(gpu["S"].tolist()) == list(range(m))
    assert np.all(gpu["M"] == 0)
    ref = oracle.dion2_step(X, G, M0, m, 0.0, 0.05, x_dtype="f32", selected=gpu["S"])
    assert rel(gpu["dX"], ref["dX"]) <= TOL["f32"]
    note("dion2 equal row norms")
    Xe = np.zeros((8, 64), np.float32)
    Ge = np.zeros((8, 64), np.float32)
    Ge[:, 0] = [1, 2, 2, 0, 2, 1, 0, 3]
    gpu = gpu_dion2(Xe, Ge, np.zeros((8, 64)), 4, 0.5, 0.1, "f32")
    assert gpu["S"].tolist() == [7, 1, 2, 4]
