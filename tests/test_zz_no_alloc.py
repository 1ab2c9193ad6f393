"""dion_step_noalloc, whose workspace is the library's static device array,
against dion_step with a caller workspace: the same bits on two calls in a row
(the second on a smaller problem, so it runs on what the first left in the
array), both within the parity tolerance of the oracle; a problem beyond the
array's size is refused before anything runs."""

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


CASES = [  # (m, n, r, dtype, seed): the 4096 x 4096 r = 256 step, then a smaller fp32 one
    (4096, 4096, 256, "bf16", 61),
    (300, 200, 37, "f32", 62),
]


def _state(m, n, r, dtype, seed):
    X, G, Q0 = synth.small_case(seed, m, n, r, dtype, planted_rank=4)
    return X, G, Q0


def _run(entry, X, G, Q0, dtype):
    m, n = X.shape
    tX, tG = to_dev(X, dtype), to_dev(G, dtype)
    tM = torch.zeros(m, n, device="cuda")
    tQ = to_dev(Q0, "f32")
    if entry == "noalloc":
        api.dion_step_noalloc(tX, tG, tM, tQ, 0.95, 0.01)
    else:
        api.dion_step(tX, tG, tM, tQ, 0.95, 0.01)
    torch.cuda.synchronize()
    return to_host(tX), to_host(tM), to_host(tQ)


def test_noalloc_matches_dion_step_on_two_calls():
    assert api.dion_workspace_size(4096, 4096, 256) <= api.NOALLOC_SCRATCH_BYTES
    for m, n, r, dtype, seed in CASES:
        X, G, Q0 = _state(m, n, r, dtype, seed)
        note(f"dion_step_noalloc {m}x{n} r={r} {dtype}")
        got = _run("noalloc", X, G, Q0, dtype)
        note(f"dion_step {m}x{n} r={r} {dtype}")
        want = _run("ws", X, G, Q0, dtype)
        for a, b in zip(got, want):
            assert np.array_equal(a, b)
        ref = oracle.dion_step(X, G, np.zeros((m, n)), Q0, 0.95, 0.01, x_dtype=dtype)
        errs = dict(X=rel(got[0], ref["X_exact"]), M=rel(got[1], ref["M"]), Q=rel(got[2], ref["Q"]))
        print(m, n, r, dtype, errs)
        assert max(errs.values()) <= TOL[dtype], errs


def test_noalloc_refuses_problems_beyond_its_scratch():
    m = n = 4096
    r = 1024
    assert api.dion_workspace_size(m, n, r) > api.NOALLOC_SCRATCH_BYTES
    tX = torch.zeros(m, n, device="cuda", dtype=torch.bfloat16)
    tM = torch.zeros(m, n, device="cuda")
    tQ = torch.zeros(n, r, device="cuda")
    note("dion_step_noalloc beyond the scratch size")
    st = api.lib().dion_step_noalloc(api.mat(tX), api.mat(tX), api.mat(tM), api.mat(tQ), r, 0.95,
                                     0.01, api._stream_ptr(tX.device))
    assert st == api.ORTHO_E_SCRATCH
    torch.cuda.synchronize()
    assert torch.count_nonzero(tM).item() == 0
