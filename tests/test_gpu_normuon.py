"""Parity of the NorMuon step (momentum buffer, Newton-Schulz of it, neuron-wise
row normalisation, SGD-form update) through the C-ABI with the fp64 oracle.
Each side carries its own state (X, M) through the steps.  Tolerances as for
Muon: 1e-4 for the fp32 momentum buffer, 2e-2 for the update and the new weight
(the Newton-Schulz products use bf16 matrix cores for either input dtype; the
row factors are fp32 sums of squares)."""

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


def gpu_normuon(X, G, M, mu, lr, dtype, scale=1.0, ws=None):
    """One step on host arrays: returns X', M' and dX (from a twin call with X = 0)."""
    out = {}
    for twin in (False, True):
        tX = to_dev(np.zeros_like(X) if twin else X, dtype)
        tG = to_dev(G, dtype)
        tM = to_dev(M, "f32")
        api.normuon_step(tX, tG, tM, mu, lr, scale, ws=ws)
        torch.cuda.synchronize()
        if twin:
            out["dX"] = to_host(tX)
            out["twin_M"] = to_host(tM)
        else:
            out["X"], out["M"] = to_host(tX), to_host(tM)
    return out


def run_normuon_parity(X, Gs, mu, lr, dtype, label, scale=1.0):
    m, n = X.shape
    ws = api.workspace(api.normuon_workspace_size(m, n), "cuda")
    Xg, Mg = X.astype(np.float64), np.zeros((m, n))
    Xo, Mo = Xg.copy(), Mg.copy()
    worst = {}
    for t, G in enumerate(Gs):
        note(f"normuon {label} {m}x{n} {dtype} step {t + 1}")
        gpu = gpu_normuon(Xg, G, Mg, mu, lr, dtype, scale=scale, ws=ws)
        ref = oracle.normuon_step(Xo, G, Mo, mu, lr, scale=scale, x_dtype=dtype)
        for k in ("X", "M", "dX"):
            assert np.all(np.isfinite(gpu[k])), k
        assert np.array_equal(gpu["twin_M"], gpu["M"])
        errs = dict(M=rel(gpu["M"], ref["M"]), dX=rel(gpu["dX"], ref["dX"]),
                    X=rel(gpu["X"], ref["X_exact"]))
        # every row of the update carries the same norm
        rn = np.linalg.norm(gpu["dX"], axis=1)
        errs["rows"] = float(np.abs(rn - rn.mean()).max() / rn.mean())
        for k, v in errs.items():
            worst[k] = max(worst.get(k, 0.0), v)
        Xg, Mg = gpu["X"], gpu["M"]
        Xo, Mo = ref["X"], ref["M"]
    return worst


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", [(96, 160), (300, 100), (257, 513), (1, 50), (640, 200)])
def test_normuon_small(shape, dtype):
    m, n = shape
    X, G1, _ = synth.small_case(90 + m, m, n, 1, dtype, planted_rank=min(4, m, n))
    Gs = [G1] + [synth.gradient(1090 + m, m, n, t, dtype) for t in (2, 3)]
    worst = run_normuon_parity(X, Gs, mu=0.95, lr=0.02, dtype=dtype, label="small", scale=1.3)
    print(shape, dtype, worst)
    assert worst["M"] <= TOL["f32"]
    assert worst["dX"] <= TOL[dtype] and worst["X"] <= TOL[dtype]
    # dX is stored in X's dtype: bf16 rounding moves each row norm slightly
    assert worst["rows"] <= TOL[dtype]


def test_normuon_square_4096_planted():
    """The 4096 x 4096 bf16 workload (planted rank-32 gradient), two steps."""
    wl = synth.WORKLOADS[2]
    X = synth.weight(2, 4096, 4096, "bf16")
    S = synth.planted(2, 4096, 4096, 32, wl["planted_ratio"])
    Gs = [synth.gradient(2, 4096, 4096, t, "bf16", planted_part=S) for t in (1, 2)]
    worst = run_normuon_parity(X, Gs, mu=0.95, lr=0.02, dtype="bf16", label="cfg2")
    print(worst)
    assert worst["M"] <= TOL["f32"]
    assert worst["dX"] <= TOL["bf16"] and worst["X"] <= TOL["bf16"]
    assert worst["rows"] <= TOL["bf16"]


def test_normuon_zero_row_stays_zero():
    """A row that is zero in both the buffer and the gradient has a zero
    orthogonalised row; its factor is 0, so its update is exactly zero, and the
    other rows match the oracle."""
    m, n = 64, 96
    X, G, _ = synth.small_case(95, m, n, 1, "f32")
    G = G.copy()
    G[5] = 0.0
    note("normuon zero row")
    gpu = gpu_normuon(X, G, np.zeros((m, n)), 0.9, 0.05, "f32")
    ref = oracle.normuon_step(X, G, np.zeros((m, n)), 0.9, 0.05, x_dtype="f32")
    assert np.all(gpu["dX"][5] == 0.0)
    assert rel(gpu["dX"], ref["dX"]) <= TOL["f32"]


def test_normuon_batched_equals_single():
    """A group through normuon_step_batched gives the bits of one call per member."""
    m, n, b = 256, 384, 3
    Xs = [synth.weight(82, m, n, "bf16", index=i) for i in range(b)]
    Gs = [synth.gradient(82, m, n, 1 + i, "bf16") for i in range(b)]
    single = []
    note("normuon batched vs single")
    for X, G in zip(Xs, Gs):
        tX, tG, tM = to_dev(X, "bf16"), to_dev(G, "bf16"), torch.zeros(m, n, device="cuda")
        api.normuon_step(tX, tG, tM, 0.9, 0.03)
        single.append((tX, tM))
    tXs = [to_dev(X, "bf16") for X in Xs]
    tGs = [to_dev(G, "bf16") for G in Gs]
    tMs = [torch.zeros(m, n, device="cuda") for _ in range(b)]
    api.normuon_step_batched(tXs, tGs, tMs, 0.9, 0.03)
    torch.cuda.synchronize()
    for (sx, sm), bx, bm in zip(single, tXs, tMs):
        assert torch.equal(sx, bx) and torch.equal(sm, bm)


def test_normuon_batched_ragged_chunks_per_head():
    """35 members of 128 x 4096 (the per-head block shape): a launch chunk of
    32 and a ragged one of 3, every member against the oracle.  The Gram of a
    128-row side is split over k by a count chosen from the members in the
    launch (8 slices for 32 members, 16 for 3 or for one), so only the ragged
    chunk's members share their single calls' summation order, and bits."""
    m, n, b = 128, 4096, 35
    Gh = [synth.gradient(83, m, n, 1, "bf16", index=i) for i in range(b)]
    Xh = [synth.weight(83, m, n, "bf16", index=i) for i in range(b)]
    note("normuon batched 35 members of 128x4096")
    Xs = [to_dev(x, "bf16") for x in Xh]
    Gs = [to_dev(g, "bf16") for g in Gh]
    Ms = [torch.zeros(m, n, device="cuda") for _ in range(b)]
    api.normuon_step_batched(Xs, Gs, Ms, 0.9, 0.03)
    # twin call with X = 0: the stored result is the update itself
    dXs = [torch.zeros(m, n, device="cuda", dtype=torch.bfloat16) for _ in range(b)]
    api.normuon_step_batched(dXs, Gs, [torch.zeros(m, n, device="cuda") for _ in range(b)],
                             0.9, 0.03)
    torch.cuda.synchronize()
    for i in range(b):
        ref = oracle.normuon_step(Xh[i], Gh[i], np.zeros((m, n)), 0.9, 0.03, x_dtype="bf16")
        assert rel(to_host(dXs[i]), ref["dX"]) <= TOL["bf16"], i
        assert rel(to_host(Xs[i]), ref["X_exact"]) <= TOL["bf16"], i
        assert rel(to_host(Ms[i]), ref["M"]) <= TOL["f32"], i
    for i in range(32, b):
        x, mm = to_dev(Xh[i], "bf16"), torch.zeros(m, n, device="cuda")
        api.normuon_step(x, Gs[i], mm, 0.9, 0.03)
        torch.cuda.synchronize()
        assert torch.equal(x, Xs[i]) and torch.equal(mm, Ms[i]), i
