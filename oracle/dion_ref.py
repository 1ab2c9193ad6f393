"""fp64 reference for the Dion step and for Newton-Schulz.  TEST INFRASTRUCTURE.

Inputs are numpy arrays holding the exact values the GPU receives (fp32 values,
or fp32 arrays whose values are bf16-representable).  Everything is widened to
fp64 and computed in fp64 with plain numpy routines; no blocking, fusion or
reordering beyond what the steps themselves state.

Each step is a small module-level function so that the pin tests can replace
one of them with a deliberately wrong variant and show that a pin catches it.
"""

from __future__ import annotations

import numpy as np

# Muon's published quintic Newton-Schulz coefficients (a, b, c).  The pages name
# Muon (hysenlabs "Microsoft Dion: orthonormal optimizers that assume DTensor
# parallelism", section "What an orthonormal optimizer changes about the update
# rule") but print no coefficients; this is the plain reading, and both sides
# take (a, b, c) as an explicit argument.
MUON_ABC = (3.4445, -4.7750, 2.0315)

# Added to the Frobenius norm before the Newton-Schulz normalisation, so that a
# zero gradient gives a zero output instead of 0/0.
NS_EPS = 1e-7


# ----------------------------------------------------------------------------
# Rounding to the storage dtype (round to nearest, ties to even)
# ----------------------------------------------------------------------------

_BF16_MANT_BITS = 8          # significant bits including the implicit one
_BF16_EMIN = -126            # smallest normal exponent (shared with fp32)
_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 value, ties to even.

    Written from the number format: a bfloat16 normal number is f * 2**e with
    8 significant bits, so its spacing in the binade [2**e, 2**(e+1)) is
    2**(e-7); below 2**-126 the spacing stays 2**-133 (subnormals).  Scaling by a
    power of two is exact in fp64 and ``np.rint`` rounds half to even.
    Returns fp64 values.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    xf = x[finite]
    _, e = np.frexp(xf)                      # xf = f * 2**e, 0.5 <= |f| < 1
    e = np.maximum(e - 1, _BF16_EMIN)        # exponent of the leading bit
    quantum = np.ldexp(1.0, e - (_BF16_MANT_BITS - 1))
    y = np.rint(xf / quantum) * quantum
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, y), y)
    out[finite] = y
    return out


def round_to_dtype(x, dtype: str) -> np.ndarray:
    """Round fp64 values to the storage dtype ('bf16' or 'f32'), returned as fp64."""
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# Dion: amortised power iteration with error feedback
# ----------------------------------------------------------------------------

def qr_positive(A: np.ndarray):
    """Thin QR factorisation A = P R with diag(R) >= 0.

    Householder QR from LAPACK, then the columns whose R-diagonal is negative
    are flipped, which makes the factor unique for full-column-rank A (it is
    then the Gram-Schmidt basis of A's columns, in order).
    """
    P, R = np.linalg.qr(_f64(A), mode="reduced")
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return P * s[None, :], R * s[:, None]


def _momentum_accumulate(M, G):
    # The gradient is added to the decoupled momentum buffer; mu is not applied
    # here (it acts as the error-feedback decay below).
    return M + G


def _power_left(B, Q):
    # One power-iteration product, warm-started from the previous right factor.
    return B @ Q


def _orthonormalize(P_tilde):
    return qr_positive(P_tilde)[0]


def _power_right(B, P):
    return B.T @ P


def _error_feedback(B, P, R, mu):
    # The rank-r part P R^T is what the step applies; the buffer keeps all of the
    # rest and a fraction mu of the applied part.
    return B - (1.0 - mu) * (P @ R.T)


def _column_normalize(R):
    norms = np.linalg.norm(R, axis=0)
    safe = np.where(norms > 0, norms, 1.0)
    Qn = R / safe[None, :]
    Qn[:, norms == 0] = 0.0
    return Qn, norms


def _weight_update(X, P, Q_new, lr, scale):
    # SGD form: step along minus the orthonormalised direction, scaled by lr.
    dX = -lr * scale * (P @ Q_new.T)
    return X + dX, dX


def dion_step(X, G, M, Q, mu: float, lr: float, scale: float = 1.0,
              x_dtype: str = "bf16") -> dict:
    """One Dion step on one matrix, in fp64.

    X (m x n) weight, G (m x n) gradient, M (m x n) momentum, Q (n x r) right
    factor.  Returns a dict with the new state and the intermediates:
    ``X`` (rounded to ``x_dtype``), ``X_exact`` (before rounding), ``dX``,
    ``M``, ``Q``, ``P``, ``R``, ``B``, ``P_tilde``, ``col_norms``.
    """
    X, G, M, Q = _f64(X), _f64(G), _f64(M), _f64(Q)
    m, n = X.shape
    if G.shape != (m, n) or M.shape != (m, n) or Q.shape[0] != n:
        raise ValueError("shape mismatch")
    B = _momentum_accumulate(M, G)
    P_tilde = _power_left(B, Q)
    P = _orthonormalize(P_tilde)
    R = _power_right(B, P)
    M_new = _error_feedback(B, P, R, mu)
    Q_new, norms = _column_normalize(R)
    X_exact, dX = _weight_update(X, P, Q_new, lr, scale)
    return dict(X=round_to_dtype(X_exact, x_dtype), X_exact=X_exact, dX=dX,
                M=M_new, Q=Q_new, P=P, R=R, B=B, P_tilde=P_tilde, col_norms=norms)


# ----------------------------------------------------------------------------
# Newton-Schulz (Muon)
# ----------------------------------------------------------------------------

def newton_schulz(G, steps: int = 5, abc=MUON_ABC, eps: float = NS_EPS) -> np.ndarray:
    """Newton-Schulz orthogonalisation of one matrix, in fp64.

    Works on the wide orientation (rows <= cols) so that the Gram matrix is the
    small one, normalises by the Frobenius norm, then repeats
    A = X X^T,  Bp = b A + c A A,  X = a X + Bp X   ``steps`` times.
    For the quintic f(s) = a s + b s^3 + c s^5 this maps G = U S V^T to
    U f(...f(S / (|G|_F + eps))...) V^T.
    """
    a, b, c = (float(v) for v in abc)
    G = _f64(G)
    tall = G.shape[0] > G.shape[1]
    Xk = _ns_normalize(G.T if tall else G, eps)
    for _ in range(steps):
        Xk = _ns_step(Xk, a, b, c)
    return Xk.T if tall else Xk


def _ns_normalize(G, eps):
    return G / (np.linalg.norm(G) + eps)


def _ns_step(Xk, a, b, c):
    A = Xk @ Xk.T
    Bp = b * A + c * (A @ A)
    return a * Xk + Bp @ Xk


def gram_newton_schulz(G, steps: int = 5, abc=MUON_ABC, eps: float = NS_EPS) -> np.ndarray:
    """The Newton-Schulz iteration run on the Gram side, in fp64.

    hysenlabs "Microsoft Dion: orthonormal optimizers that assume DTensor
    parallelism", section on installing from git with the optional kernels,
    names a Gram Newton-Schulz option; the pages give no formula.  The reading:
    the same iteration as ``newton_schulz``, expressed through the small Gram
    matrix.  On the wide orientation (rows <= cols) with X_0 the normalised
    input, every iterate is X_k = Q_k X_0 for an m x m matrix Q_k, and
        A_0     = X_0 X_0^T
        A_k     = Q_k A_0 Q_k^T                (= X_k X_k^T)
        Q_{k+1} = (a I + b A_k + c A_k A_k) Q_k,   Q_0 = I
    so the result Q_steps X_0 equals ``newton_schulz`` up to rounding, while the
    wide matrix takes part in two products only.
    """
    a, b, c = (float(v) for v in abc)
    G = _f64(G)
    tall = G.shape[0] > G.shape[1]
    X0 = _ns_normalize(G.T if tall else G, eps)
    A0 = X0 @ X0.T
    Q = np.eye(X0.shape[0])
    for _ in range(steps):
        Q = _gram_ns_step(Q, A0, a, b, c)
    out = Q @ X0
    return out.T if tall else out


def _gram_ns_step(Q, A0, a, b, c):
    A = Q @ A0 @ Q.T
    return (a * np.eye(Q.shape[0]) + b * A + c * (A @ A)) @ Q


# ----------------------------------------------------------------------------
# Muon step: momentum buffer, Newton-Schulz orthogonalisation, SGD-form update
# ----------------------------------------------------------------------------

def _muon_momentum(M, G, mu):
    """Heavy-ball momentum buffer M' = mu M + G (the plainest reading; the pages
    name Muon's momentum but print no formula for it)."""
    return mu * M + G


def muon_step(X, G, M, mu: float, lr: float, scale: float = 1.0, steps: int = 5,
              abc=MUON_ABC, eps: float = NS_EPS, x_dtype: str = "bf16") -> dict:
    """One Muon step on one matrix, in fp64.

    MSR talk "Dion: The distributed orthonormal update revolution is here":
    Muon orthogonalises the momentum-accumulated gradient with Newton-Schulz
    iterations (passage on Muon's dense matrix products) and applies it in the
    SGD form X - lr * update (passage contrasting SGD with orthonormal updates).
        M' = mu M + G
        U  = newton_schulz(M', steps, abc, eps)
        X' = X - lr * scale * U, rounded to ``x_dtype``
    Returns ``X`` (rounded), ``X_exact``, ``dX`` (= -lr * scale * U), ``M`` and
    ``U``.
    """
    X, G, M = _f64(X), _f64(G), _f64(M)
    M_new = _muon_momentum(M, G, float(mu))
    U = newton_schulz(M_new, steps, abc, eps)
    dX = -float(lr) * float(scale) * U
    X_exact = X + dX
    return dict(X=round_to_dtype(X_exact, x_dtype), X_exact=X_exact, dX=dX, M=M_new, U=U)


def row_normalize(U):
    """Neuron-wise normalisation of an orthogonalised update, in fp64.

    Pages: agentlenshq "microsoft/dion", section "How it works" (NorMuon adds
    neuron-wise normalisation to Muon), and hysenlabs "Microsoft Dion:
    orthonormal optimizers that assume DTensor parallelism", section "Dion3 is
    not a retuning of Dion2, and the README says so" (per-neuron normalisation
    redistributes the update across rows).
    Neither page prints a formula; the plainest reading they support is a
    stateless rescale of each row (one output neuron) to a common norm that
    keeps the update's total Frobenius norm:
        t   = ||U||_F / sqrt(m)
        V_i = U_i * t / ||U_i||_2      (a zero row stays zero)
    """
    U = _f64(U)
    m = U.shape[0]
    row_sq = np.einsum("ij,ij->i", U, U)
    target = np.sqrt(row_sq.sum() / m) if m > 0 else 0.0
    f = np.zeros(m)
    nz = row_sq > 0.0
    f[nz] = target / np.sqrt(row_sq[nz])
    return U * f[:, None]


def normuon_step(X, G, M, mu: float, lr: float, scale: float = 1.0, steps: int = 5,
                 abc=MUON_ABC, eps: float = NS_EPS, x_dtype: str = "bf16") -> dict:
    """One NorMuon step: the Muon step with the orthogonalised momentum
    normalised per neuron (row) before it is applied.
        M' = mu M + G
        U  = newton_schulz(M', steps, abc, eps)
        V  = row_normalize(U)
        X' = X - lr * scale * V, rounded to ``x_dtype``
    Returns ``X`` (rounded), ``X_exact``, ``dX`` (= -lr * scale * V), ``M``,
    ``U`` and ``V``.
    """
    X, G, M = _f64(X), _f64(G), _f64(M)
    M_new = _muon_momentum(M, G, float(mu))
    U = newton_schulz(M_new, steps, abc, eps)
    V = row_normalize(U)
    dX = -float(lr) * float(scale) * V
    X_exact = X + dX
    return dict(X=round_to_dtype(X_exact, x_dtype), X_exact=X_exact, dX=dX, M=M_new, U=U, V=V)


# ----------------------------------------------------------------------------
# Dion2: submatrix selection with error feedback
# ----------------------------------------------------------------------------

def select_rows(B, k: int) -> np.ndarray:
    """Indices of the k rows of B with the largest l2 norm, largest first; equal
    norms are ordered by row index (lower first), so the choice is unique.
    A row whose norm is NaN is ordered after every other row."""
    B = _f64(B)
    sq = np.einsum("ij,ij->i", B, B)
    key = np.where(np.isnan(sq), -1.0, sq)
    order = sorted(range(B.shape[0]), key=lambda i: (-key[i], i))
    return np.asarray(order[:k], dtype=np.int64)


def dion2_step(X, G, M, k: int, mu: float, lr: float, scale: float = 1.0, steps: int = 5,
               abc=MUON_ABC, eps: float = NS_EPS, x_dtype: str = "bf16",
               selected=None) -> dict:
    """One Dion2 step on one matrix, in fp64.

    agentlenshq "microsoft/dion", sections "How it works" (Dion2 selects a
    submatrix; every Dion variant keeps error feedback) and "Highlights" (only a
    fraction of the momentum takes part); hysenlabs "Microsoft Dion: orthonormal
    optimizers that assume DTensor parallelism", section "Dion3 is not a
    retuning of Dion2, and the README says so" (mu is Dion2's error-feedback
    decay).  No selection rule or formula is printed; the reading:
        B   = M + G
        S   = the k rows of B with the largest l2 norm (select_rows)
        U   = newton_schulz(B[S], steps, abc, eps)      (orthonormalised block)
        X'  = X, with rows S replaced by X[S] - lr * scale * U, rounded to x_dtype
        M'  = B, with rows S replaced by mu * B[S]      (error feedback: the
              applied block keeps the fraction mu, the rest is kept whole)
    ``selected`` overrides S (the rows, in the order they are stacked into the
    block).  Returns X (rounded), X_exact, dX, M, U, B, S.
    """
    X, G, M = _f64(X), _f64(G), _f64(M)
    B = _momentum_accumulate(M, G)
    import oracle.dion_ref as _self   # the module attribute, so a pin can replace it
    S = _self.select_rows(B, k) if selected is None else np.asarray(selected, dtype=np.int64)
    U = newton_schulz(B[S], steps, abc, eps)
    dX = np.zeros_like(X)
    dX[S] = -float(lr) * float(scale) * U
    X_exact = X + dX
    M_new = _dion2_feedback(B, S, float(mu))
    return dict(X=round_to_dtype(X_exact, x_dtype), X_exact=X_exact, dX=dX, M=M_new, U=U, B=B, S=S)


def _dion2_feedback(B, S, mu):
    # the applied rows keep the fraction mu; every other row is kept whole
    M_new = B.copy()
    M_new[S] = mu * B[S]
    return M_new

