"""Seeded synthetic inputs for the optimizer-step workloads.

This module only draws random numbers and rounds them to the storage dtype; it
holds none of the update's arithmetic.  Both the GPU tests and the fp64 oracle
receive exactly these values.

Recipe (one generator per (workload, role, step, matrix index)):
    numpy.random.default_rng([workload_id, role, step, index])
    role 0 = weight X, 1 = initial right factor Q0, 2 = planted low-rank part,
    3 = gradient noise E_t.
Values are drawn in fp64, rounded to fp32 (IEEE round to nearest even) and, for
bf16 tensors, rounded again to bfloat16 (nearest even).  Returned arrays are
float32 whose values are exactly representable in the storage dtype.

Workloads (the talk's square-matrix sweep, a GPT-style parameter set, per-head
attention blocks, and Llama-3-405B-shaped matrices; MSR talk "Dion: The
distributed orthonormal update revolution is here", microbenchmark passage):
"""

from __future__ import annotations

import numpy as np

ROLE_X, ROLE_Q0, ROLE_PLANT, ROLE_NOISE, ROLE_LAYOUT = 0, 1, 2, 3, 4

WORKLOADS = {
    1: dict(name="single-256x256-f32", dtype="f32",
            groups=[(1, 256, 256)], ranks=[64], mu=0.95, lr=0.01, steps=10,
            planted_rank=0, ns=None),
    2: dict(name="square-4096x4096-bf16", dtype="bf16",
            groups=[(1, 4096, 4096)], ranks=[1024, 256], mu=0.95, lr=0.01, steps=3,
            planted_rank=32, planted_ratio=10.0, ns=dict(steps=5, blocks=1)),
    3: dict(name="gpt12-d2048-grouped-bf16", dtype="bf16",
            groups=[(48, 2048, 2048), (12, 2048, 8192), (12, 8192, 2048)],
            ranks=[512], mu=0.95, lr=0.01, steps=3, planted_rank=0, ns=None),
    4: dict(name="per-head-4096x4096-bf16", dtype="bf16",
            groups=[(1, 4096, 4096)], ranks=[256], mu=0.95, lr=0.01, steps=3,
            planted_rank=0, ns=dict(steps=5, blocks=32)),
    5: dict(name="llama405b-shaped-bf16", dtype="bf16",
            groups=[(1, 16384, 16384), (1, 16384, 53248)], ranks=[1024, 4096],
            mu=0.95, lr=0.01, steps=1, planted_rank=0, ns=dict(steps=5, blocks=1)),
}


def _rng(workload: int, role: int, step: int = 0, index: int = 0):
    return np.random.default_rng([workload, role, step, index])


def to_bf16_values(x) -> np.ndarray:
    """fp64/fp32 -> fp32 (nearest even) -> bfloat16 (nearest even), as float32.

    The bfloat16 step keeps the upper 16 bits of the fp32 pattern after adding
    0x7FFF plus the lowest kept bit (ties go to the even pattern).  NaN is not
    produced by these generators.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def to_storage(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return to_bf16_values(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    raise ValueError(dtype)


def weight(workload: int, m: int, n: int, dtype: str, index: int = 0) -> np.ndarray:
    """X ~ N(0, 0.02^2) (0.02 is the standard deviation)."""
    return to_storage(0.02 * _rng(workload, ROLE_X, 0, index).standard_normal((m, n)), dtype)


def right_factor0(workload: int, n: int, r: int, index: int = 0) -> np.ndarray:
    """Q0: Gaussian n x r with unit-norm columns, fp32."""
    q = _rng(workload, ROLE_Q0, 0, index).standard_normal((n, r))
    q /= np.linalg.norm(q, axis=0, keepdims=True)
    return q.astype(np.float32)


def noise(workload: int, m: int, n: int, step: int, index: int = 0) -> np.ndarray:
    """E_t ~ N(0,1) iid, fp64 (not yet rounded)."""
    return _rng(workload, ROLE_NOISE, step, index).standard_normal((m, n))


def _haar(rng, rows, k):
    q, r = np.linalg.qr(rng.standard_normal((rows, k)))
    s = np.sign(np.diag(r))
    s[s == 0] = 1
    return q * s


def planted(workload: int, m: int, n: int, rank: int, ratio: float, index: int = 0):
    """S = sigma * U V^T with Haar-orthonormal U (m x rank), V (n x rank), fixed
    across steps; sigma makes |S|_F = ratio * |E_1|_F."""
    rng = _rng(workload, ROLE_PLANT, 0, index)
    U = _haar(rng, m, rank)
    V = _haar(rng, n, rank)
    e1 = np.linalg.norm(noise(workload, m, n, 1, index))
    sigma = ratio * e1 / np.sqrt(rank)
    return sigma * (U @ V.T)


def gradient(workload: int, m: int, n: int, step: int, dtype: str, index: int = 0,
             planted_part=None) -> np.ndarray:
    """G_t = E_t (+ S), rounded to the storage dtype.  step counts from 1."""
    g = noise(workload, m, n, step, index)
    if planted_part is not None:
        g = g + planted_part
    return to_storage(g, dtype)


def small_case(seed: int, m: int, n: int, r: int, dtype: str, planted_rank: int = 0,
               planted_ratio: float = 10.0, x_scale: float = 0.02):
    """Inputs for ad-hoc parity cases (ragged shapes, edge cases): X, G, Q0, with
    workload id 1000 + seed so they never collide with the named workloads."""
    wid = 1000 + seed
    X = to_storage(x_scale * _rng(wid, ROLE_X).standard_normal((m, n)), dtype)
    Q0 = right_factor0(wid, n, r)
    S = planted(wid, m, n, planted_rank, planted_ratio) if planted_rank else None
    G = gradient(wid, m, n, 1, dtype, planted_part=S)
    return X, G, Q0


def block_layout(workload: int, m: int, n: int, r: int, blocks: int):
    """Scattered block-diagonal layout for full-size structural cases: block i
    owns rows perm_m[i*m/k : (i+1)*m/k] of an m x n matrix and columns
    perm_n[i*n/k : (i+1)*n/k].  Returns (perm_m, perm_n) as int64 arrays."""
    return block_layout_r(workload, m, n, r, blocks)[:2]


def block_layout_r(workload: int, m: int, n: int, r: int, blocks: int):
    """block_layout plus a permutation of the r factor columns: block i also
    owns columns sorted(perm_r[i*r/k : (i+1)*r/k]) of an n x r (or m x r)
    factor, so the blocks' factor columns interleave.  Returns (perm_m,
    perm_n, perm_r) as int64 arrays; the first two equal block_layout's."""
    if m % blocks or n % blocks or r % blocks:
        raise ValueError("block count must divide m, n and r")
    rng = _rng(workload, ROLE_LAYOUT, 0, m * 1000003 + n * 1009 + r)
    perm_m = rng.permutation(m).astype(np.int64)
    perm_n = rng.permutation(n).astype(np.int64)
    return perm_m, perm_n, rng.permutation(r).astype(np.int64)
