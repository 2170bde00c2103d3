"""Brute-force check of the oracle on tiny inputs: pure Python loops.

TEST INFRASTRUCTURE ONLY (see oracle/oracle.py for who may import it).

Each dot product is ``math.fsum`` over the products, so every sum is correctly
rounded; a product of two fp32 (or bf16) values is exact in float64, so the
first-layer products are exactly rounded results. GeLU is written in its
equivalent logistic form, x * sigma(2 s) with s = sqrt(2/pi)(x + 0.044715 x^3)
(because (1 + tanh s)/2 = sigma(2 s)), and its derivative is derived from that
form: sigma(2s) + x * 2 sigma(2s)(1 - sigma(2s)) * s'. This is a second,
independently written route to the same functions as oracle/oracle.py, so a
dropped term, a wrong sign or a transposed operand in either one shows up as a
disagreement.

Matrices are lists of lists of floats; shapes follow oracle/oracle.py.
"""
from __future__ import annotations

import math

_C = math.sqrt(2.0 / math.pi)
_K = 0.044715


def _sigmoid(z: float) -> float:
    if z >= 0:
        return 1.0 / (1.0 + math.exp(-z))
    e = math.exp(z)
    return e / (1.0 + e)


def gelu(x: float) -> float:
    s = _C * (x + _K * x * x * x)
    return x * _sigmoid(2.0 * s)


def gelu_grad(x: float) -> float:
    s = _C * (x + _K * x * x * x)
    ds = _C * (1.0 + 3.0 * _K * x * x)
    g = _sigmoid(2.0 * s)
    return g + x * 2.0 * g * (1.0 - g) * ds


def matmul(L, R):
    """C[i][j] = fsum_k L[i][k] R[k][j]."""
    n_k = len(R)
    n_j = len(R[0])
    cols = [[R[k][j] for k in range(n_k)] for j in range(n_j)]
    return [[math.fsum(li[k] * cj[k] for k in range(n_k)) for cj in cols] for li in L]


def transpose(M):
    return [list(r) for r in zip(*M)]


def colsum(M):
    return [math.fsum(M[t][j] for t in range(len(M))) for j in range(len(M[0]))]


def mlp_step(X, A, a, B, b, dZ, p):
    """Forward + backward of the column/row-split MLP, shard by shard, and the
    sums over shards, as plain loops. Returns the same names as oracle.tp_mlp
    (for every shard) plus Z and dX."""
    T = len(X)
    h = len(X[0])
    n = len(A[0])
    w = n // p
    out = {}
    Z_parts, dX_parts = [], []
    for i in range(p):
        A_i = [row[i * w:(i + 1) * w] for row in A]
        a_i = None if a is None else a[i * w:(i + 1) * w]
        B_i = B[i * w:(i + 1) * w]
        XA = matmul(X, A_i)
        U = [[XA[t][j] + (0.0 if a_i is None else a_i[j]) for j in range(w)] for t in range(T)]
        Y = [[gelu(u) for u in row] for row in U]
        Zp = matmul(Y, B_i)
        dY = matmul(dZ, transpose(B_i))
        dU = [[dY[t][j] * gelu_grad(U[t][j]) for j in range(w)] for t in range(T)]
        dB = matmul(transpose(Y), dZ)
        dA = matmul(transpose(X), dU)
        dXp = matmul(dU, transpose(A_i))
        out.update({f"U_{i}": U, f"Y_{i}": Y, f"Zp_{i}": Zp, f"dU_{i}": dU,
                    f"dB_{i}": dB, f"dA_{i}": dA, f"dXp_{i}": dXp})
        if a is not None:
            out[f"da_{i}"] = colsum(dU)
        Z_parts.append(Zp)
        dX_parts.append(dXp)
    out["Z"] = [[math.fsum([Z_parts[i][t][j] for i in range(p)]) + (0.0 if b is None else b[j])
                 for j in range(h)] for t in range(T)]
    out["dX"] = [[math.fsum([dX_parts[i][t][j] for i in range(p)]) for j in range(h)]
                 for t in range(T)]
    if b is not None:
        out["db"] = colsum(dZ)
    return out
