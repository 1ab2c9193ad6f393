"""Second, independent fp64 formulation for tiny inputs.  TEST INFRASTRUCTURE.

Pure-Python loops with exactly rounded sums (``math.fsum``) and modified
Gram-Schmidt with one re-orthogonalisation pass in place of Householder QR.
It shares no helper with ``oracle.dion_ref``; the pin tests use it to check the
numpy formulation step by step on inputs small enough for loops.
"""

from __future__ import annotations

import math


def _mat(a):
    return [[float(v) for v in row] for row in a]


def matmul(A, B):
    n, k, m = len(A), len(B), len(B[0])
    return [[math.fsum(A[i][t] * B[t][j] for t in range(k)) for j in range(m)]
            for i in range(n)]


def transpose(A):
    return [list(col) for col in zip(*A)]


def mgs_qr(A):
    """Modified Gram-Schmidt, run twice per column; the norms are positive, so
    the triangular factor has a positive diagonal."""
    rows, cols = len(A), len(A[0])
    basis = []
    for j in range(cols):
        v = [A[i][j] for i in range(rows)]
        for _ in range(2):
            for q in basis:
                d = math.fsum(q[i] * v[i] for i in range(rows))
                v = [v[i] - d * q[i] for i in range(rows)]
        nrm = math.sqrt(math.fsum(x * x for x in v))
        basis.append([x / nrm for x in v])
    return [[basis[j][i] for j in range(cols)] for i in range(rows)]


def dion_step(X, G, M, Q, mu, lr, scale=1.0):
    """Returns (X_exact, M_new, Q_new, P, R) as nested lists."""
    X, G, M, Q = _mat(X), _mat(G), _mat(M), _mat(Q)
    m, n, r = len(X), len(X[0]), len(Q[0])
    B = [[M[i][j] + G[i][j] for j in range(n)] for i in range(m)]
    P = mgs_qr(matmul(B, Q))
    R = matmul(transpose(B), P)
    PRt = matmul(P, transpose(R))
    M_new = [[B[i][j] - (1.0 - mu) * PRt[i][j] for j in range(n)] for i in range(m)]
    norms = [math.sqrt(math.fsum(R[i][k] ** 2 for i in range(n))) for k in range(r)]
    Q_new = [[R[i][k] / norms[k] for k in range(r)] for i in range(n)]
    PQt = matmul(P, transpose(Q_new))
    X_new = [[X[i][j] - lr * scale * PQt[i][j] for j in range(n)] for i in range(m)]
    return X_new, M_new, Q_new, P, R


def newton_schulz(G, steps, abc, eps):
    a, b, c = abc
    G = _mat(G)
    tall = len(G) > len(G[0])
    Xk = transpose(G) if tall else G
    fro = math.sqrt(math.fsum(v * v for row in Xk for v in row))
    Xk = [[v / (fro + eps) for v in row] for row in Xk]
    for _ in range(steps):
        A = matmul(Xk, transpose(Xk))
        AA = matmul(A, A)
        Bp = [[b * A[i][j] + c * AA[i][j] for j in range(len(A))] for i in range(len(A))]
        BX = matmul(Bp, Xk)
        Xk = [[a * Xk[i][j] + BX[i][j] for j in range(len(Xk[0]))] for i in range(len(Xk))]
    return transpose(Xk) if tall else Xk


def row_normalize(U):
    """Rows rescaled to the common norm sqrt(sum of all squares / rows), each
    by its own exactly rounded norm; zero rows stay zero."""
    U = _mat(U)
    m = len(U)
    norms = [math.sqrt(math.fsum(v * v for v in row)) for row in U]
    total = math.sqrt(math.fsum(v * v for row in U for v in row))
    target = total / math.sqrt(m)
    return [[v * target / nrm for v in row] if nrm > 0.0 else [0.0] * len(row)
            for row, nrm in zip(U, norms)]
