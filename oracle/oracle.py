"""CPU oracle for the tensor-parallel MLP / attention-projection shard (float64).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP path; the only common code is the seeded input generator
``tp_inputs``.

Every step is the plain definition, in float64, with numpy's ``@`` as the matrix
product, applied to the exact stored input values (bf16 or fp32, widened). No
intermediate is rounded to the device's storage types: the oracle computes the
exact-arithmetic result (up to float64 rounding) that the device approximates.

Sources (page titles as printed; sections by their headings):
  [M]  "Megatron" (zzmblog.top), section "Tensor Parallelism" / "mathematical
       principles": the column split Y = [X A_1, ..., X A_p] and the row split
       Z = Y_1 B_1 + ... + Y_p B_p followed by an All-Reduce sum.
  [M'] same page, "Transformer-layer tensor parallelism": QKV projection and
       MLP fc1 column-split, attention output projection and MLP fc2 row-split,
       one All-Reduce after each row-split layer.
  [M"] same page, training-script listing: ``activation_func="gelu"``.
The backward products are not on the pages; they are the textbook derivatives
of the forward definitions (d(XW)/dX = dOut W^T, d(XW)/dW = X^T dOut, bias grad
= column sum), and the GeLU derivative is the derivative of the tanh form.

Readings where the pages are silent: rows of X are
tokens; weights are stored [in, out]; shards are contiguous equal blocks; GeLU is
the tanh form with constants sqrt(2/pi) and 0.044715 (Hendrycks & Gimpel); the
row-parallel bias is added once, after the sum over shards.

Parity status: every function here is pinned by a test in
tests/test_oracle_pins.py (brute force with exactly rounded sums, split
invariants, p-invariance, GeLU closed forms and an independent sigmoid
formulation, finite differences, special cases).
"""
from __future__ import annotations

import math

import numpy as np

SQRT_2_OVER_PI = math.sqrt(2.0 / math.pi)
GELU_CUBIC = 0.044715


# --------------------------------------------------------------------------- #
# Activation                                                                   #
# --------------------------------------------------------------------------- #
def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GeLU, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))). [M"]"""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(SQRT_2_OVER_PI * (x + GELU_CUBIC * x ** 3)))


def gelu_tanh_grad(x: np.ndarray) -> np.ndarray:
    """d/dx of gelu_tanh: with t = tanh(s), s = sqrt(2/pi)(x + 0.044715 x^3),
    0.5 (1 + t) + 0.5 x (1 - t^2) sqrt(2/pi) (1 + 3 * 0.044715 x^2)."""
    x = np.asarray(x, dtype=np.float64)
    t = np.tanh(SQRT_2_OVER_PI * (x + GELU_CUBIC * x ** 3))
    return 0.5 * (1.0 + t) + 0.5 * x * (1.0 - t * t) * SQRT_2_OVER_PI * (
        1.0 + 3.0 * GELU_CUBIC * x * x
    )


def _act(act: str):
    if act == "gelu":
        return gelu_tanh
    if act == "none":
        return lambda u: u
    raise ValueError(f"unknown activation {act!r}")


# --------------------------------------------------------------------------- #
# Sharding: contiguous equal blocks                                            #
# --------------------------------------------------------------------------- #
def shard_columns(A: np.ndarray, p: int, i: int) -> np.ndarray:
    """A_i of A = [A_1, ..., A_p] (split by output columns). [M]"""
    n = A.shape[-1]
    assert n % p == 0
    w = n // p
    return A[..., i * w:(i + 1) * w]


def shard_rows(B: np.ndarray, p: int, i: int) -> np.ndarray:
    """B_i of B stacked as [B_1; ...; B_p] (split by input rows). [M]"""
    n = B.shape[0]
    assert n % p == 0
    w = n // p
    return B[i * w:(i + 1) * w]


# --------------------------------------------------------------------------- #
# The five operations of the shard                                            #
# --------------------------------------------------------------------------- #
def column_linear_fwd(X, A_i, a_i=None, act="none"):
    """Column-parallel forward on shard i: U_i = X A_i (+ a_i), Y_i = act(U_i).
    X is replicated, so no exchange is needed. [M], [M']"""
    U = np.asarray(X, np.float64) @ np.asarray(A_i, np.float64)
    if a_i is not None:
        U = U + np.asarray(a_i, np.float64)[None, :]
    return U, _act(act)(U)


def row_linear_fwd_partial(Y_i, B_i):
    """Row-parallel forward on shard i: the partial Y_i B_i (no bias). [M]"""
    return np.asarray(Y_i, np.float64) @ np.asarray(B_i, np.float64)


def reduce_partials(partials, bias=None):
    """The All-Reduce sum of the row-parallel partials, Z = sum_i Zp_i (+ b),
    with the bias added once after the sum. [M], [M']"""
    Z = np.zeros_like(np.asarray(partials[0], np.float64))
    for P in partials:
        Z = Z + np.asarray(P, np.float64)
    if bias is not None:
        Z = Z + np.asarray(bias, np.float64)[None, :]
    return Z


def linear_bwd_dgrad(dOut, W, U=None, act="none"):
    """Input gradient of Out = act(In W): dIn = (dOut W^T) * act'(U) for the
    activation's derivative at the pre-activation U (act = "gelu"), or
    dOut W^T when there is no activation. W is stored [in, out]."""
    d = np.asarray(dOut, np.float64) @ np.asarray(W, np.float64).T
    if act == "gelu":
        d = d * gelu_tanh_grad(U)
    elif act != "none":
        raise ValueError(act)
    return d


def linear_bwd_wgrad(In, dOut):
    """Weight and bias gradients of Out = In W + c: dW = In^T dOut,
    dc = sum over tokens of dOut."""
    In = np.asarray(In, np.float64)
    dOut = np.asarray(dOut, np.float64)
    return In.T @ dOut, dOut.sum(axis=0)


# --------------------------------------------------------------------------- #
# Whole shard step: forward + backward over the p shards                       #
# --------------------------------------------------------------------------- #
def tp_mlp(X, A, a, B, b, dZ, p, shards=None, weights_are_shards=False):
    """MLP of a Transformer layer with fc1 column-split and fc2 row-split over
    p shards [M], [M']; forward then backward.

    Returns per-shard U_i, Y_i, Zp_i, dY_i, dU_i, dB_i, dA_i, da_i, dXp_i and the
    sums Z (forward, bias added once) and dX (backward, sum of dXp_i) when every
    shard ran. ``weights_are_shards``: A, a, B are already the one shard in
    ``shards`` (the 175B-class workload draws only shard 0).
    """
    shards = tuple(range(p)) if shards is None else tuple(shards)
    out = {}
    Zp, dXp = [], []
    for i in shards:
        if weights_are_shards:
            A_i, B_i = A, B
            a_i = a
        else:
            A_i, B_i = shard_columns(A, p, i), shard_rows(B, p, i)
            a_i = None if a is None else shard_columns(a, p, i)
        U_i, Y_i = column_linear_fwd(X, A_i, a_i, "gelu")
        Zp_i = row_linear_fwd_partial(Y_i, B_i)
        dU_i = linear_bwd_dgrad(dZ, B_i, U_i, "gelu")
        dB_i, _ = linear_bwd_wgrad(Y_i, dZ)
        dA_i, da_i = linear_bwd_wgrad(X, dU_i)
        dXp_i = linear_bwd_dgrad(dU_i, A_i, None, "none")
        out.update({f"U_{i}": U_i, f"Y_{i}": Y_i, f"Zp_{i}": Zp_i, f"dU_{i}": dU_i,
                    f"dB_{i}": dB_i, f"dA_{i}": dA_i, f"dXp_{i}": dXp_i})
        if a is not None:
            out[f"da_{i}"] = da_i
        Zp.append(Zp_i)
        dXp.append(dXp_i)
    if b is not None:
        out["db"] = np.asarray(dZ, np.float64).sum(axis=0)
    if len(shards) == p:
        out["Z"] = reduce_partials(Zp, b)
        out["dX"] = reduce_partials(dXp, None)
    return out


def tp_attn_proj(X, W, C, Ow, dQKV, dZa, p, shards=None):
    """Attention projections of a Transformer layer: QKV column-split, output
    projection row-split [M']; no activation, no bias. C (the attention core's
    output) and the upstream gradients are inputs."""
    shards = tuple(range(p)) if shards is None else tuple(shards)
    out = {}
    Zp, dXp = [], []
    for i in shards:
        W_i, C_i, Ow_i = shard_columns(W, p, i), shard_columns(C, p, i), shard_rows(Ow, p, i)
        dQKV_i = shard_columns(dQKV, p, i)
        QKV_i, _ = column_linear_fwd(X, W_i, None, "none")
        Zpa_i = row_linear_fwd_partial(C_i, Ow_i)
        dC_i = linear_bwd_dgrad(dZa, Ow_i, None, "none")
        dOw_i, _ = linear_bwd_wgrad(C_i, dZa)
        dW_i, _ = linear_bwd_wgrad(X, dQKV_i)
        dXq_i = linear_bwd_dgrad(dQKV_i, W_i, None, "none")
        out.update({f"QKV_{i}": QKV_i, f"Zpa_{i}": Zpa_i, f"dC_{i}": dC_i,
                    f"dOw_{i}": dOw_i, f"dW_{i}": dW_i, f"dXqp_{i}": dXq_i})
        Zp.append(Zpa_i)
        dXp.append(dXq_i)
    if len(shards) == p:
        out["Za"] = reduce_partials(Zp, None)
        out["dXq"] = reduce_partials(dXp, None)
    return out


def mlp_unsharded(X, A, a, B, b, dZ):
    """The same MLP without splitting (p = 1): the right-hand sides of the
    column- and row-split identities. [M]"""
    U, Y = column_linear_fwd(X, A, a, "gelu")
    Z = reduce_partials([row_linear_fwd_partial(Y, B)], b)
    dU = linear_bwd_dgrad(dZ, B, U, "gelu")
    dB, db = linear_bwd_wgrad(Y, dZ)
    dA, da = linear_bwd_wgrad(X, dU)
    dX = linear_bwd_dgrad(dU, A, None, "none")
    return {"U": U, "Y": Y, "Z": Z, "dU": dU, "dB": dB, "db": db, "dA": dA,
            "da": da, "dX": dX}


def run_config(cfg, inputs, attn_core: bool = False) -> dict:
    """All outputs of one fwd+bwd step of a workload (names as in tp_mlp /
    tp_attn_proj), from the HostTensors of tp_inputs.make_inputs. With
    attn_core the attention workloads run the whole attention block
    (oracle.attention.tp_attn_block: the core between the projections, C_i
    and dQKV_i computed rather than drawn)."""
    g = {k: v.f64() for k, v in inputs.items()}
    out = {}
    if cfg.mlp:
        out.update(tp_mlp(g["X"], g["A"], g.get("a"), g["B"], g.get("b"), g["dZ"],
                          cfg.p, cfg.shards, weights_are_shards=not cfg.full_weights))
    if cfg.attn and attn_core:
        from .attention import tp_attn_block
        out.update(tp_attn_block(g["X"], g["W"], g["Ow"], g["dZa"], cfg.p, cfg.micro_batch,
                                 cfg.seq, cfg.heads, cfg.shards))
    elif cfg.attn:
        out.update(tp_attn_proj(g["X"], g["W"], g["C"], g["Ow"], g["dQKV"], g["dZa"],
                                cfg.p, cfg.shards))
    return out


# --------------------------------------------------------------------------- #
# Sampled entries for full-size checks                                         #
# --------------------------------------------------------------------------- #
def sampled_dot(L: np.ndarray, R: np.ndarray, rows, cols, transpose_left=False,
                transpose_right=False) -> np.ndarray:
    """Entries (rows[s], cols[s]) of op(L) @ op(R), each one a float64 dot
    product, without forming the whole product."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    lv = (L[:, rows].T if transpose_left else L[rows, :]).astype(np.float64)
    rv = (R[cols, :] if transpose_right else R[:, cols].T).astype(np.float64)
    return np.einsum("sk,sk->s", lv, rv)


def rel_fro(got, ref) -> float:
    """Relative Frobenius error ||got - ref||_F / ||ref||_F, in float64."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((got - ref).ravel())
    if den == 0.0:
        return float(num)
    return float(num / den)
