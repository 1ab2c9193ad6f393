"""Python binding of libortho.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
only turns torch tensors into ``ortho_mat`` descriptors (device pointer, rows,
cols, leading dimension, dtype), sizes the workspace, and passes torch's
current HIP stream.  It raises if the library has not been built -- there is no
fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libortho.so")

ORTHO_F32, ORTHO_BF16 = 0, 1
ORTHO_E_SCRATCH = 9
NOALLOC_SCRATCH_BYTES = 64 << 20
DEV_CHOL_SHIFT, DEV_ZERO_COLUMN = 1, 2
MUON_ABC = (3.4445, -4.7750, 2.0315)


class OrthoMat(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64), ("dtype", ctypes.c_int32)]


class OrthoError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


_lib = None

_SIGS = {
    "ortho_dion_workspace_size": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]),
    "ortho_ns_workspace_size": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]),
    "dion_step": (ctypes.c_int, [OrthoMat, OrthoMat, OrthoMat, OrthoMat, ctypes.c_int32, ctypes.c_float,
                                 ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "dion_step_ex": (ctypes.c_int, [OrthoMat, OrthoMat, OrthoMat, OrthoMat, ctypes.c_int32, ctypes.c_float,
                                    ctypes.c_float, ctypes.c_float, ctypes.POINTER(OrthoMat),
                                    ctypes.POINTER(OrthoMat), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]),
    "dion_step_batched": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(OrthoMat), ctypes.POINTER(OrthoMat),
                                         ctypes.POINTER(OrthoMat), ctypes.POINTER(OrthoMat), ctypes.c_int32,
                                         ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "newton_schulz": (ctypes.c_int, [OrthoMat, OrthoMat, ctypes.c_int32, ctypes.POINTER(ctypes.c_float),
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "newton_schulz_batched": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(OrthoMat), ctypes.POINTER(OrthoMat),
                                             ctypes.c_int32, ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                             ctypes.c_size_t, ctypes.c_void_p]),
    "ortho_muon_workspace_size": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]),
    "muon_step": (ctypes.c_int, [OrthoMat, OrthoMat, OrthoMat, ctypes.c_int32, ctypes.POINTER(ctypes.c_float),
                                 ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                 ctypes.c_size_t, ctypes.c_void_p]),
    "muon_step_batched": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(OrthoMat), ctypes.POINTER(OrthoMat),
                                         ctypes.POINTER(OrthoMat), ctypes.c_int32,
                                         ctypes.POINTER(ctypes.c_float), ctypes.c_float, ctypes.c_float,
                                         ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "ortho_normuon_workspace_size": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]),
    "normuon_step": (ctypes.c_int, [OrthoMat, OrthoMat, OrthoMat, ctypes.c_int32, ctypes.POINTER(ctypes.c_float),
                                    ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]),
    "normuon_step_batched": (ctypes.c_int, [ctypes.c_int32, ctypes.POINTER(OrthoMat), ctypes.POINTER(OrthoMat),
                                            ctypes.POINTER(OrthoMat), ctypes.c_int32,
                                            ctypes.POINTER(ctypes.c_float), ctypes.c_float, ctypes.c_float,
                                            ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "dion_step_noalloc": (ctypes.c_int, [OrthoMat, OrthoMat, OrthoMat, OrthoMat, ctypes.c_int32,
                                         ctypes.c_float, ctypes.c_float, ctypes.c_void_p]),
    "ortho_dion2_workspace_size": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32]),
    "dion2_step": (ctypes.c_int, [OrthoMat, OrthoMat, OrthoMat, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.POINTER(ctypes.c_float), ctypes.c_float, ctypes.c_float,
                                  ctypes.c_float, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                  ctypes.c_void_p]),
    "ortho_status_str": (ctypes.c_char_p, [ctypes.c_int32]),
    "ortho_abi_version": (ctypes.c_int32, []),
}

EXPORTED = tuple(_SIGS)


def lib():
    """Load libortho.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m orthonormal_optimizer_update_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().ortho_status_str(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise OrthoError(fn, status, status_str(status))


def mat(t) -> OrthoMat:
    """Descriptor of a 2-D row-major torch tensor (unit column stride)."""
    import torch
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.size(1) > 1 and t.stride(1) != 1:
        raise ValueError("expected unit stride along columns")
    if t.dtype == torch.float32:
        dt = ORTHO_F32
    elif t.dtype == torch.bfloat16:
        dt = ORTHO_BF16
    else:
        raise ValueError(f"unsupported dtype {t.dtype}")
    ld = t.stride(0) if t.size(0) > 1 else t.size(1)
    return OrthoMat(t.data_ptr(), t.size(0), t.size(1), max(ld, t.size(1)), dt)


def _stream_ptr(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def dion_workspace_size(m: int, n: int, r: int, batch: int = 1) -> int:
    return int(lib().ortho_dion_workspace_size(m, n, r, batch))


def ns_workspace_size(m: int, n: int, batch: int = 1) -> int:
    return int(lib().ortho_ns_workspace_size(m, n, batch))


def workspace(nbytes: int, device):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def dion_step(X, G, M, Q, mu: float, lr: float, scale: float = 1.0, ws=None, P_out=None,
              R_out=None, dev_status=None):
    """One Dion step in place on (X, M, Q): ``dion_step`` of ortho.h, or
    ``dion_step_ex`` when a scale other than 1 or an optional output is given."""
    r = Q.size(1)
    if ws is None:
        ws = workspace(dion_workspace_size(X.size(0), X.size(1), r), X.device)
    if scale == 1.0 and P_out is None and R_out is None and dev_status is None:
        st = lib().dion_step(mat(X), mat(G), mat(M), mat(Q), r, mu, lr, _ptr(ws), ws.numel(),
                             _stream_ptr(X.device))
        _check("dion_step", st)
        return
    dion_step_ex(X, G, M, Q, mu, lr, scale, ws, P_out, R_out, dev_status)


def dion_step_ex(X, G, M, Q, mu: float, lr: float, scale: float = 1.0, ws=None, P_out=None,
                 R_out=None, dev_status=None):
    """``dion_step_ex`` of ortho.h: a Dion step with an update scale and the
    optional outputs P, R and the device status word."""
    r = Q.size(1)
    if ws is None:
        ws = workspace(dion_workspace_size(X.size(0), X.size(1), r), X.device)
    pm = ctypes.byref(mat(P_out)) if P_out is not None else None
    rm = ctypes.byref(mat(R_out)) if R_out is not None else None
    st = lib().dion_step_ex(mat(X), mat(G), mat(M), mat(Q), r, mu, lr, scale, pm, rm,
                            _ptr(dev_status), _ptr(ws), ws.numel(), _stream_ptr(X.device))
    _check("dion_step_ex", st)


def dion_step_noalloc(X, G, M, Q, mu: float, lr: float):
    """``dion_step_noalloc`` of ortho.h: a Dion step whose workspace is the
    library's static device array (no allocation by the library or here)."""
    st = lib().dion_step_noalloc(mat(X), mat(G), mat(M), mat(Q), Q.size(1), mu, lr,
                                 _stream_ptr(X.device))
    _check("dion_step_noalloc", st)


def dion_step_batched(Xs: Sequence, Gs: Sequence, Ms: Sequence, Qs: Sequence, mu: float, lr: float,
                      scale: float = 1.0, ws=None, dev_status=None):
    """Dion on a group of same-shape matrices in one call."""
    b = len(Xs)
    arr = OrthoMat * b
    X = arr(*[mat(t) for t in Xs])
    G = arr(*[mat(t) for t in Gs])
    M = arr(*[mat(t) for t in Ms])
    Q = arr(*[mat(t) for t in Qs])
    r = Qs[0].size(1)
    if ws is None:
        ws = workspace(dion_workspace_size(Xs[0].size(0), Xs[0].size(1), r, b), Xs[0].device)
    st = lib().dion_step_batched(b, X, G, M, Q, r, mu, lr, scale, _ptr(dev_status), _ptr(ws),
                                 ws.numel(), _stream_ptr(Xs[0].device))
    _check("dion_step_batched", st)


def _abc(abc):
    if abc is None:
        return None
    return (ctypes.c_float * 3)(*[float(v) for v in abc])


def newton_schulz(G, out=None, steps: int = 5, abc=None, ws=None):
    """Newton-Schulz of G into ``out`` (allocated like G when None); returns out."""
    import torch
    if out is None:
        out = torch.empty_like(G)
    if ws is None:
        ws = workspace(ns_workspace_size(G.size(0), G.size(1)), G.device)
    st = lib().newton_schulz(mat(G), mat(out), steps, _abc(abc), _ptr(ws), ws.numel(),
                             _stream_ptr(G.device))
    _check("newton_schulz", st)
    return out


def newton_schulz_batched(Gs: Sequence, outs: Optional[Sequence] = None, steps: int = 5, abc=None,
                          ws=None):
    import torch
    b = len(Gs)
    if outs is None:
        outs = [torch.empty_like(g) for g in Gs]
    arr = OrthoMat * b
    G = arr(*[mat(t) for t in Gs])
    O = arr(*[mat(t) for t in outs])
    if ws is None:
        ws = workspace(ns_workspace_size(Gs[0].size(0), Gs[0].size(1), b), Gs[0].device)
    st = lib().newton_schulz_batched(b, G, O, steps, _abc(abc), _ptr(ws), ws.numel(),
                                     _stream_ptr(Gs[0].device))
    _check("newton_schulz_batched", st)
    return outs


def muon_workspace_size(m: int, n: int, batch: int = 1) -> int:
    return int(lib().ortho_muon_workspace_size(m, n, batch))


def muon_step(X, G, M, mu: float, lr: float, scale: float = 1.0, steps: int = 5, abc=None, ws=None):
    """One Muon step in place on (X, M); see ``muon_step`` in ortho.h."""
    if ws is None:
        ws = workspace(muon_workspace_size(X.size(0), X.size(1)), X.device)
    st = lib().muon_step(mat(X), mat(G), mat(M), steps, _abc(abc), mu, lr, scale, _ptr(ws),
                         ws.numel(), _stream_ptr(X.device))
    _check("muon_step", st)


def muon_step_batched(Xs: Sequence, Gs: Sequence, Ms: Sequence, mu: float, lr: float,
                      scale: float = 1.0, steps: int = 5, abc=None, ws=None):
    """Muon on a group of same-shape matrices in one call."""
    b = len(Xs)
    arr = OrthoMat * b
    X = arr(*[mat(t) for t in Xs])
    G = arr(*[mat(t) for t in Gs])
    M = arr(*[mat(t) for t in Ms])
    if ws is None:
        ws = workspace(muon_workspace_size(Xs[0].size(0), Xs[0].size(1), b), Xs[0].device)
    st = lib().muon_step_batched(b, X, G, M, steps, _abc(abc), mu, lr, scale, _ptr(ws), ws.numel(),
                                 _stream_ptr(Xs[0].device))
    _check("muon_step_batched", st)


def normuon_workspace_size(m: int, n: int, batch: int = 1) -> int:
    return int(lib().ortho_normuon_workspace_size(m, n, batch))


def normuon_step(X, G, M, mu: float, lr: float, scale: float = 1.0, steps: int = 5, abc=None,
                 ws=None):
    """One NorMuon step in place on (X, M); see ``normuon_step`` in ortho.h."""
    if ws is None:
        ws = workspace(normuon_workspace_size(X.size(0), X.size(1)), X.device)
    st = lib().normuon_step(mat(X), mat(G), mat(M), steps, _abc(abc), mu, lr, scale, _ptr(ws),
                            ws.numel(), _stream_ptr(X.device))
    _check("normuon_step", st)


def normuon_step_batched(Xs: Sequence, Gs: Sequence, Ms: Sequence, mu: float, lr: float,
                         scale: float = 1.0, steps: int = 5, abc=None, ws=None):
    """NorMuon on a group of same-shape matrices in one call."""
    b = len(Xs)
    arr = OrthoMat * b
    X = arr(*[mat(t) for t in Xs])
    G = arr(*[mat(t) for t in Gs])
    M = arr(*[mat(t) for t in Ms])
    if ws is None:
        ws = workspace(normuon_workspace_size(Xs[0].size(0), Xs[0].size(1), b), Xs[0].device)
    st = lib().normuon_step_batched(b, X, G, M, steps, _abc(abc), mu, lr, scale, _ptr(ws),
                                    ws.numel(), _stream_ptr(Xs[0].device))
    _check("normuon_step_batched", st)


def dion2_workspace_size(m: int, n: int, k: int) -> int:
    return int(lib().ortho_dion2_workspace_size(m, n, k))


def dion2_step(X, G, M, k: int, mu: float, lr: float, scale: float = 1.0, steps: int = 5,
               abc=None, selected=None, ws=None):
    """One Dion2 step in place on (X, M); see ``dion2_step`` in ortho.h.
    ``selected`` (optional) is a device int32 tensor of k entries."""
    if ws is None:
        ws = workspace(dion2_workspace_size(X.size(0), X.size(1), k), X.device)
    st = lib().dion2_step(mat(X), mat(G), mat(M), k, steps, _abc(abc), mu, lr, scale,
                          _ptr(selected), _ptr(ws), ws.numel(), _stream_ptr(X.device))
    _check("dion2_step", st)
