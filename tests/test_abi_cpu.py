"""C-ABI checks that need no GPU: the library loads, exports every function that
include/ortho.h declares, sizes workspaces, and rejects bad arguments with the
documented status codes before touching the device."""

import ctypes
import os
import re

import pytest

from orthonormal_optimizer_update_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000   # never dereferenced: validation fails first


def header_functions():
    text = open(os.path.join(ROOT, "include", "ortho.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


def test_header_declares_expected_entry_points():
    names = header_functions()
    for n in ["dion_step", "dion_step_ex", "dion_step_batched", "newton_schulz",
              "newton_schulz_batched", "ortho_dion_workspace_size", "ortho_ns_workspace_size",
              "muon_step", "muon_step_batched", "ortho_muon_workspace_size",
              "normuon_step", "normuon_step_batched", "ortho_normuon_workspace_size",
              "dion2_step", "ortho_dion2_workspace_size",
              "ortho_status_str", "ortho_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = api.lib()
    for name in header_functions():
        assert hasattr(L, name), name
    assert set(header_functions()) <= set(api.EXPORTED)
    assert L.ortho_abi_version() == 1


def test_status_strings():
    for s in range(9):
        assert api.status_str(s)
    assert api.status_str(99) == "unknown status"


def test_workspace_sizes():
    small = api.dion_workspace_size(256, 256, 64)
    assert small > 0 and small % 256 == 0
    assert api.dion_workspace_size(4096, 4096, 1024) > api.dion_workspace_size(4096, 4096, 256)
    # a group needs one slot per member up to the per-launch cap, then reuses them
    # (split-K factors, hence slot sizes, depend on how many members share a launch)
    full = api.dion_workspace_size(2048, 2048, 512, 32)
    assert full > api.dion_workspace_size(2048, 2048, 512, 1)
    assert api.dion_workspace_size(2048, 2048, 512, 48) == full
    # invalid sizes give 0
    assert api.dion_workspace_size(10, 5, 6) == 0
    assert api.dion_workspace_size(0, 5, 1) == 0
    assert api.ns_workspace_size(4096, 4096) >= 4096 * 4096 * (4 + 2 * 4)
    # 32 members share a launch at most; larger groups reuse the slots
    assert api.ns_workspace_size(128, 4096, 64) == api.ns_workspace_size(128, 4096, 32)
    assert api.ns_workspace_size(128, 4096, 32) > 16 * api.ns_workspace_size(128, 4096, 1)
    assert api.ns_workspace_size(4096, 128) == api.ns_workspace_size(128, 4096)


def M(rows, cols, dtype, ld=None, data=FAKE):
    return api.OrthoMat(data, rows, cols, ld if ld is not None else cols, dtype)


def dion(X, G, Mo, Q, r, mu=0.9, lr=0.1, ws=FAKE, wsb=None, P=None, R=None):
    L = api.lib()
    if wsb is None:
        wsb = api.dion_workspace_size(X.rows, X.cols, max(r, 1)) or 1 << 30
    return L.dion_step_ex(X, G, Mo, Q, r, mu, lr, 1.0, P, R, None,
                          ctypes.c_void_p(ws) if ws else None, wsb, None)


BF, F = api.ORTHO_BF16, api.ORTHO_F32


def good():
    return M(64, 48, BF), M(64, 48, BF), M(64, 48, F), M(48, 8, F)


@pytest.mark.parametrize("case,want", [
    ("null_x", 1), ("null_ws", 6), ("small_ws", 6), ("misaligned_ws", 6),
    ("rank_big", 4), ("rank_zero", 4), ("rank_vs_q", 4),
    ("mu_neg", 7), ("mu_big", 7), ("lr_nan", 7),
    ("g_dtype", 3), ("m_bf16", 3), ("q_bf16", 3), ("bad_dtype", 3),
    ("g_shape", 2), ("m_shape", 2), ("q_rows", 2), ("zero_rows", 2),
    ("ld_small", 5), ("p_out_shape", 2), ("r_out_dtype", 3),
])
def test_dion_argument_errors(case, want):
    X, G, Mo, Q = good()
    r, kw = 8, {}
    if case == "null_x": X = M(64, 48, BF, data=None)
    elif case == "null_ws": kw = dict(ws=0)
    elif case == "small_ws": kw = dict(wsb=1024)
    elif case == "misaligned_ws": kw = dict(ws=FAKE + 8)
    elif case == "rank_big": r = 49; Q = M(48, 49, F)
    elif case == "rank_zero": r = 0
    elif case == "rank_vs_q": r = 7
    elif case == "mu_neg": kw = dict(mu=-0.1)
    elif case == "mu_big": kw = dict(mu=1.01)
    elif case == "lr_nan": kw = dict(lr=float("nan"))
    elif case == "g_dtype": G = M(64, 48, F)
    elif case == "m_bf16": Mo = M(64, 48, BF)
    elif case == "q_bf16": Q = M(48, 8, BF)
    elif case == "bad_dtype": X = M(64, 48, 5)
    elif case == "g_shape": G = M(64, 47, BF)
    elif case == "m_shape": Mo = M(63, 48, F)
    elif case == "q_rows": Q = M(47, 8, F)
    elif case == "zero_rows": X = M(0, 48, BF)
    elif case == "ld_small": Mo = M(64, 48, F, ld=40)
    elif case == "p_out_shape": kw = dict(P=ctypes.byref(M(64, 9, F)))
    elif case == "r_out_dtype": kw = dict(R=ctypes.byref(M(48, 8, BF)))
    assert dion(X, G, Mo, Q, r, **kw) == want


def test_dion_batched_errors():
    L = api.lib()
    arr = api.OrthoMat * 2
    X = arr(M(64, 48, BF), M(64, 48, BF))
    G = arr(M(64, 48, BF), M(64, 48, BF))
    Mo = arr(M(64, 48, F), M(64, 48, F))
    Q = arr(M(48, 8, F), M(48, 8, F))
    wsb = api.dion_workspace_size(64, 48, 8, 2)
    call = lambda b, x=X: L.dion_step_batched(b, x, G, Mo, Q, 8, 0.9, 0.1, 1.0, None,
                                              ctypes.c_void_p(FAKE), wsb, None)
    assert call(0) == 7
    assert call(2, arr(M(64, 48, BF), M(64, 40, BF))) == 2          # members differ in shape
    assert call(2, arr(M(64, 48, BF), M(64, 48, BF, ld=64))) == 5   # members differ in ld
    assert L.dion_step_batched(2, X, G, Mo, Q, 8, 0.9, 0.1, 1.0, None, ctypes.c_void_p(FAKE),
                               wsb - 256, None) == 6
    # a member whose right factor is narrower than r (same ld) is a rank error
    Qn = arr(M(48, 8, F), M(48, 4, F, ld=8))
    assert L.dion_step_batched(2, X, G, Mo, Qn, 8, 0.9, 0.1, 1.0, None, ctypes.c_void_p(FAKE),
                               wsb, None) == 4


def test_dion_noalloc_argument_errors():
    """Argument errors and the scratch limit come back before any device call."""
    L = api.lib()
    X, G, Mo, Q = M(64, 48, BF), M(64, 48, BF), M(64, 48, F), M(48, 8, F)
    assert L.dion_step_noalloc(X, G, Mo, Q, 8, 1.5, 0.1, None) == 7
    assert L.dion_step_noalloc(X, G, Mo, Q, 9, 0.9, 0.1, None) == 4
    assert L.dion_step_noalloc(M(64, 48, BF, data=None), G, Mo, Q, 8, 0.9, 0.1, None) == 1
    assert L.dion_step_noalloc(X, M(64, 48, F), Mo, Q, 8, 0.9, 0.1, None) == 3
    big = (M(4096, 4096, BF), M(4096, 4096, BF), M(4096, 4096, F), M(4096, 1024, F))
    assert api.dion_workspace_size(4096, 4096, 1024) > api.NOALLOC_SCRATCH_BYTES
    assert L.dion_step_noalloc(*big, 1024, 0.9, 0.1, None) == api.ORTHO_E_SCRATCH
    assert "scratch" in api.status_str(api.ORTHO_E_SCRATCH)


def test_dion2_argument_errors():
    L = api.lib()
    wsb = api.dion2_workspace_size(64, 48, 16)
    assert wsb > api.ns_workspace_size(16, 48)
    assert api.dion2_workspace_size(64, 48, 65) == 0
    ws = ctypes.c_void_p(FAKE)
    X, G, Mo = M(64, 48, BF), M(64, 48, BF), M(64, 48, F)
    call = lambda *a: L.dion2_step(*a, None, ws, wsb, None)
    assert call(X, G, Mo, 0, 5, None, 0.9, 0.1, 1.0) == 4
    assert call(X, G, Mo, 65, 5, None, 0.9, 0.1, 1.0) == 4
    assert call(X, G, Mo, 16, -1, None, 0.9, 0.1, 1.0) == 7
    assert call(X, G, Mo, 16, 5, None, 1.5, 0.1, 1.0) == 7
    assert call(X, M(64, 48, F), Mo, 16, 5, None, 0.9, 0.1, 1.0) == 3
    assert call(X, G, M(64, 48, BF), 16, 5, None, 0.9, 0.1, 1.0) == 3
    assert call(X, G, M(64, 40, F), 16, 5, None, 0.9, 0.1, 1.0) == 2
    assert call(M(64, 48, BF, data=None), G, Mo, 16, 5, None, 0.9, 0.1, 1.0) == 1
    assert L.dion2_step(X, G, Mo, 16, 5, None, 0.9, 0.1, 1.0, None, ws, wsb - 1, None) == 6
    big = M(70000, 8, BF)
    assert L.dion2_step(big, big, M(70000, 8, F), 4, 5, None, 0.9, 0.1, 1.0, None, ws, 1 << 40,
                        None) == 2


def test_ns_argument_errors():
    L = api.lib()
    wsb = api.ns_workspace_size(64, 48)
    ws = ctypes.c_void_p(FAKE)
    G, O = M(64, 48, BF), M(64, 48, BF)
    assert L.newton_schulz(G, O, -1, None, ws, wsb, None) == 7
    assert L.newton_schulz(G, M(64, 48, F), 5, None, ws, wsb, None) == 3
    assert L.newton_schulz(G, M(48, 64, BF), 5, None, ws, wsb, None) == 2
    assert L.newton_schulz(G, O, 5, None, None, wsb, None) == 6
    assert L.newton_schulz(G, O, 5, None, ws, wsb - 1, None) == 6
    bad = (ctypes.c_float * 3)(1.0, float("inf"), 0.0)
    assert L.newton_schulz(G, O, 5, bad, ws, wsb, None) == 7
    assert L.newton_schulz(M(64, 48, BF, data=None), O, 5, None, ws, wsb, None) == 1
    arr = api.OrthoMat * 2
    assert L.newton_schulz_batched(2, arr(G, M(64, 48, BF, ld=50)), arr(O, O), 5, None, ws,
                                   api.ns_workspace_size(64, 48, 2), None) == 5


def test_muon_argument_errors():
    L = api.lib()
    wsb = api.muon_workspace_size(64, 48)
    assert wsb >= api.ns_workspace_size(64, 48) + 64 * 48 * 4
    ws = ctypes.c_void_p(FAKE)
    X, G, Mo = M(64, 48, BF), M(64, 48, BF), M(64, 48, F)
    call = lambda x=X, g=G, m=Mo, steps=5, abc=None, mu=0.95, lr=0.02, w=ws, b=wsb: L.muon_step(
        x, g, m, steps, abc, mu, lr, 1.0, w, b, None)
    assert call(steps=-1) == 7
    assert call(mu=1.5) == 7
    assert call(lr=float("inf")) == 7
    assert call(abc=(ctypes.c_float * 3)(1.0, float("nan"), 0.0)) == 7
    assert call(g=M(64, 48, F)) == 3            # G must have X's dtype
    assert call(m=M(64, 48, BF)) == 3           # momentum is fp32
    assert call(m=M(64, 47, F)) == 2
    assert call(x=M(64, 48, BF, data=None)) == 1
    assert call(w=None) == 6
    assert call(b=wsb - 1) == 6
    arr = api.OrthoMat * 2
    assert L.muon_step_batched(2, arr(X, M(64, 48, BF, ld=56)), arr(G, G), arr(Mo, Mo), 5, None,
                               0.95, 0.02, 1.0, ws, api.muon_workspace_size(64, 48, 2), None) == 5
    assert L.muon_step_batched(0, arr(X, X), arr(G, G), arr(Mo, Mo), 5, None, 0.95, 0.02, 1.0, ws,
                               wsb, None) == 7


def test_normuon_argument_errors():
    """NorMuon validates as Muon does, against its own (larger) workspace: the
    Muon workspace plus one fp32 factor per row and member."""
    L = api.lib()
    wsb = api.normuon_workspace_size(64, 48)
    assert wsb >= api.muon_workspace_size(64, 48) + 64 * 4
    assert api.normuon_workspace_size(64, 48, 3) >= api.muon_workspace_size(64, 48, 3) + 3 * 64 * 4
    assert api.normuon_workspace_size(0, 48) == 0
    ws = ctypes.c_void_p(FAKE)
    X, G, Mo = M(64, 48, BF), M(64, 48, BF), M(64, 48, F)
    call = lambda x=X, g=G, m=Mo, steps=5, mu=0.95, lr=0.02, w=ws, b=wsb: L.normuon_step(
        x, g, m, steps, None, mu, lr, 1.0, w, b, None)
    assert call(steps=-1) == 7
    assert call(mu=-0.1) == 7
    assert call(lr=float("nan")) == 7
    assert call(g=M(64, 48, F)) == 3
    assert call(m=M(64, 48, BF)) == 3
    assert call(m=M(63, 48, F)) == 2
    assert call(w=None) == 6
    # a Muon-sized workspace is too small for NorMuon
    assert call(b=api.muon_workspace_size(64, 48)) == 6
    assert call(w=ctypes.c_void_p(FAKE + 64)) == 6   # not 256-byte aligned
    arr = api.OrthoMat * 2
    assert L.normuon_step_batched(2, arr(X, M(64, 40, BF)), arr(G, G), arr(Mo, Mo), 5, None, 0.95,
                                  0.02, 1.0, ws, api.normuon_workspace_size(64, 48, 2), None) == 2


def test_valid_call_without_gpu_reports_hip_error():
    """With no usable device the call gets past validation and reports the
    launch failure as ORTHO_E_HIP instead of crashing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    X, G, Mo, Q = good()
    assert dion(X, G, Mo, Q, 8) == 8
