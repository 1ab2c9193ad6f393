"""Helpers for the GPU parity tests: run the HIP path through the C-ABI binding
and the fp64 oracle on the same seeded inputs, and compare."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from orthonormal_optimizer_update_amd import api

# Relative Frobenius tolerances.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def note(msg: str):
    """Name the case before a GPU step, flushed, so a crash still says what ran."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b)
    num = np.linalg.norm(a - b)
    if den == 0:
        return float(num)
    return float(num / den)


def tdtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a, dtype: str):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda").to(tdtype(dtype))


def to_host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def gpu_dion_step(X, G, M, Q, mu, lr, dtype, scale=1.0, ws=None):
    """One HIP Dion step on host arrays; returns dict of host fp64 results,
    including dX taken from a twin call with X = 0."""
    m, n = X.shape
    r = Q.shape[1]
    if ws is None:
        ws = api.workspace(api.dion_workspace_size(m, n, r), "cuda")
    out = {}
    for twin in (False, True):
        tX = to_dev(np.zeros_like(X) if twin else X, dtype)
        tG = to_dev(G, dtype)
        tM = to_dev(M, "f32")
        tQ = to_dev(Q, "f32")
        P = torch.empty(m, r, dtype=torch.float32, device="cuda")
        R = torch.empty(n, r, dtype=torch.float32, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        api.dion_step(tX, tG, tM, tQ, mu, lr, scale, ws=ws, P_out=P, R_out=R, dev_status=status)
        torch.cuda.synchronize()
        res = dict(X=to_host(tX), M=to_host(tM), Q=to_host(tQ), P=to_host(P), R=to_host(R),
                   status=int(status.item()))
        if twin:
            out["dX"] = res["X"]
            out["twin_M"], out["twin_Q"] = res["M"], res["Q"]
        else:
            out.update(res)
    return out


def compare_dion(gpu: dict, ref: dict) -> dict:
    return dict(M=rel(gpu["M"], ref["M"]), Q=rel(gpu["Q"], ref["Q"]), P=rel(gpu["P"], ref["P"]),
                R=rel(gpu["R"], ref["R"]), dX=rel(gpu["dX"], ref["dX"]), X=rel(gpu["X"], ref["X_exact"]))


def run_dion_parity(X, Gs, Q0, mu, lr, dtype, scale=1.0, label=""):
    """Carry each side's own state through len(Gs) steps; return the worst
    relative error per output and the per-step records."""
    m, n = X.shape
    ws = api.workspace(api.dion_workspace_size(m, n, Q0.shape[1]), "cuda")
    Xg, Mg, Qg = X.astype(np.float64), np.zeros((m, n)), Q0.astype(np.float64)
    Xo, Mo, Qo = Xg.copy(), Mg.copy(), Qg.copy()
    worst, records = {}, []
    for t, G in enumerate(Gs):
        note(f"dion {label} {m}x{n} r={Q0.shape[1]} {dtype} step {t + 1}")
        gpu = gpu_dion_step(Xg, G, Mg, Qg, mu, lr, dtype, scale, ws)
        ref = oracle.dion_step(Xo, G, Mo, Qo, mu, lr, scale, x_dtype=dtype)
        for k in ("M", "Q", "P", "R", "X", "dX"):
            assert np.all(np.isfinite(gpu[k])), f"non-finite {k} at step {t + 1}"
        assert np.array_equal(gpu["twin_M"], gpu["M"]) and np.array_equal(gpu["twin_Q"], gpu["Q"])
        errs = compare_dion(gpu, ref)
        records.append(errs)
        for k, v in errs.items():
            worst[k] = max(worst.get(k, 0.0), v)
        Xg, Mg, Qg = gpu["X"], gpu["M"], gpu["Q"]
        Xo, Mo, Qo = ref["X"], ref["M"], ref["Q"]
    return worst, records


def gpu_ns(G, dtype, steps=5, abc=None):
    g = to_dev(G, dtype)
    out = api.newton_schulz(g, steps=steps, abc=abc)
    torch.cuda.synchronize()
    return to_host(out)
