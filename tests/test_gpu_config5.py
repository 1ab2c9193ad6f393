"""Llama-405B-shaped matrices at full size: 16384 x 16384 and 16384 x 53248
bf16, Dion at rank fractions 1/16 and 1/4 of the smaller side (r = 1024,
4096) and Newton-Schulz (5 iterations) on 16384 x 16384, through the same
entry points and launch configuration as any other call.

The fp64 oracle cannot run these shapes whole in test time, so the inputs carry
an exact structure that reduces the full-size step to small independent
problems.  The gradient is block diagonal after row and column permutations
(16 blocks), and Q0 is block diagonal with the same column blocks and r/16
columns per block, those columns scattered over the r columns (each block's
in increasing order).  Then P~ = B Q, its Gram matrix, the Cholesky factor,
the QR factor, R = B^T P and the column norms all act block by block: a
column's Gram-Schmidt projections on other blocks' columns are exact zeros,
and the Cholesky factor's cross-block entries are exact zeros, while every
64 x 64 tile of the Gram and of the factor mixes columns of many blocks, so
the blocked factorisation runs on dense tiles.  The result is exact, not
approximate, so:
  * two blocks per case are compared with the oracle run on that block alone,
    at the bf16 tolerance;
  * everything off the blocks must come out bit for bit as the structure
    dictates: M' = 0, P = 0, Q' = 0 there, and X' = X.
Newton-Schulz is equivariant under the permutations and acts block by block
on a block-diagonal matrix, with every block scaled by the norm of the whole
matrix; off the blocks the output is exactly zero."""

import numpy as np
import pytest
import torch

import oracle
from oracle import dion_ref
from orthonormal_optimizer_update_amd import api, synth

from parity_util import TOL, note, rel, to_host

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

K = 16          # blocks
CHECK = (0, K - 1)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    api.lib()
    torch.cuda.set_device(0)


def _idx(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _put(dst, rows, cols, block, dtype):
    dst[_idx(rows)[:, None], _idx(cols)[None, :]] = torch.from_numpy(block).to("cuda").to(dtype)


def _take(src, rows, cols):
    return to_host(src[_idx(rows)[:, None], _idx(cols)[None, :]])


def _clear(t, rows, cols):
    t[_idx(rows)[:, None], _idx(cols)[None, :]] = 0


@pytest.mark.parametrize("m,n,r", [(16384, 16384, 1024), (16384, 16384, 4096),
                                   (16384, 53248, 1024), (16384, 53248, 4096)])
def test_config5_dion_block_structured(m, n, r):
    wl = synth.WORKLOADS[5]
    mu, lr = wl["mu"], wl["lr"]
    mb, nb, rb = m // K, n // K, r // K
    perm_m, perm_n, perm_r = synth.block_layout_r(5, m, n, r, K)
    rows = [perm_m[i * mb:(i + 1) * mb] for i in range(K)]
    cols = [perm_n[i * nb:(i + 1) * nb] for i in range(K)]
    rcols = [np.sort(perm_r[i * rb:(i + 1) * rb]) for i in range(K)]

    note(f"config5 dion {m}x{n} r={r}: building inputs")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5_000_000 + m + n + r)
    X = (0.02 * torch.randn(m, n, device="cuda", generator=gen)).to(torch.bfloat16)
    G = torch.zeros(m, n, device="cuda", dtype=torch.bfloat16)
    M = torch.zeros(m, n, device="cuda", dtype=torch.float32)
    Q = torch.zeros(n, r, device="cuda", dtype=torch.float32)
    blocks = {}
    for i in range(K):
        Xb = synth.weight(5, mb, nb, "bf16", index=i)
        Gb = synth.gradient(5, mb, nb, 1, "bf16", index=i)
        Qb = synth.right_factor0(5, nb, rb, index=i)
        _put(X, rows[i], cols[i], Xb, torch.bfloat16)
        _put(G, rows[i], cols[i], Gb, torch.bfloat16)
        _put(Q, cols[i], rcols[i], Qb, torch.float32)
        if i in CHECK:
            blocks[i] = (Xb, Gb, Qb)
    X0 = X.clone()
    P = torch.empty(m, r, device="cuda", dtype=torch.float32)
    R = torch.empty(n, r, device="cuda", dtype=torch.float32)
    status = torch.zeros(1, device="cuda", dtype=torch.int32)
    ws = api.workspace(api.dion_workspace_size(m, n, r), "cuda")
    note(f"config5 dion {m}x{n} r={r}: step")
    api.dion_step(X, G, M, Q, mu, lr, ws=ws, P_out=P, R_out=R, dev_status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0

    for i in CHECK:
        Xb, Gb, Qb = blocks[i]
        ref = oracle.dion_step(Xb, Gb, np.zeros((mb, nb)), Qb, mu, lr, x_dtype="bf16")
        errs = dict(M=rel(_take(M, rows[i], cols[i]), ref["M"]),
                    Q=rel(_take(Q, cols[i], rcols[i]), ref["Q"]),
                    P=rel(_take(P, rows[i], rcols[i]), ref["P"]),
                    R=rel(_take(R, cols[i], rcols[i]), ref["R"]),
                    X=rel(_take(X, rows[i], cols[i]), ref["X_exact"]))
        print(m, n, r, "block", i, errs)
        assert max(errs.values()) <= TOL["bf16"], (i, errs)

    note(f"config5 dion {m}x{n} r={r}: off-block exactness")
    D = X.float() - X0.float()
    for i in range(K):
        _clear(M, rows[i], cols[i])
        _clear(D, rows[i], cols[i])
        _clear(P, rows[i], rcols[i])
        _clear(Q, cols[i], rcols[i])
    assert torch.count_nonzero(M).item() == 0
    assert torch.count_nonzero(D).item() == 0
    assert torch.count_nonzero(P).item() == 0
    assert torch.count_nonzero(Q).item() == 0


def test_config5_newton_schulz_block_structured():
    m = n = 16384
    mb = m // K
    perm_m, perm_n = synth.block_layout(5, m, n, K, K)
    rows = [perm_m[i * mb:(i + 1) * mb] for i in range(K)]
    cols = [perm_n[i * mb:(i + 1) * mb] for i in range(K)]
    note("config5 NS 16384x16384: building input")
    G = torch.zeros(m, n, device="cuda", dtype=torch.bfloat16)
    sq = 0.0
    blocks = {}
    for i in range(K):
        Gb = synth.gradient(5, mb, mb, 1, "bf16", index=100 + i)
        sq += float(np.sum(Gb.astype(np.float64) ** 2))
        _put(G, rows[i], cols[i], Gb, torch.bfloat16)
        if i in CHECK:
            blocks[i] = Gb
    note("config5 NS 16384x16384: 5 iterations")
    out = api.newton_schulz(G, steps=5)
    torch.cuda.synchronize()
    a, b, c = dion_ref.MUON_ABC
    scale = 1.0 / (np.sqrt(sq) + dion_ref.NS_EPS)
    for i in CHECK:
        Xk = blocks[i].astype(np.float64) * scale
        for _ in range(5):
            Xk = dion_ref._ns_step(Xk, a, b, c)
        e = rel(_take(out, rows[i], cols[i]), Xk)
        print("NS block", i, e)
        assert e <= TOL["bf16"], (i, e)
    note("config5 NS 16384x16384: off-block exactness")
    for i in range(K):
        _clear(out, rows[i], cols[i])
    assert torch.count_nonzero(out).item() == 0
