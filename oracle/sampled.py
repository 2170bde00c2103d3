"""Sampled rows / columns of the oracle's outputs, for full-size workloads.

TEST INFRASTRUCTURE ONLY (see oracle/oracle.py for who may import it).

A row of a product is the product of that row, and a column of a product is
the product with that column: (X A)[R, :] = X[R, :] A and (X A)[:, C] = X A[:, C].
So every function here calls the float64 oracle functions of oracle/oracle.py on
row or column slices of the exact inputs and returns exactly (up to float64
rounding) the corresponding slices of the full oracle's outputs; tests pin them
against the full oracle on small workloads.

Sampled outputs, per shard i:
  rows R of the token axis:  U_i, Y_i, Zp_i, dU_i, dXp_i (and Z, dX when every
                             shard runs); attention QKV_i, Zpa_i, dC_i, dXqp_i (Za, dXq)
  columns Cf of the shard:   dB_i[Cf, :], dA_i[:, Cf], da_i[Cf];
                             attention dOw_i[Co, :], dW_i[:, Cq]
  db in full (a column sum of dZ).
"""
from __future__ import annotations

import numpy as np

from .oracle import (
    column_linear_fwd,
    gelu_tanh,
    linear_bwd_dgrad,
    linear_bwd_wgrad,
    reduce_partials,
    row_linear_fwd_partial,
    shard_columns,
    shard_rows,
)


def mlp_sampled(X, A, a, B, b, dZ, p, rows, cols, shards=None, weights_are_shards=False):
    shards = tuple(range(p)) if shards is None else tuple(shards)
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    out = {}
    Zp, dXp = [], []
    Xr, dZr = X[rows], dZ[rows]
    for i in shards:
        if weights_are_shards:
            A_i, B_i, a_i = A, B, a
        else:
            A_i, B_i = shard_columns(A, p, i), shard_rows(B, p, i)
            a_i = None if a is None else shard_columns(a, p, i)
        # token rows
        U_r, Y_r = column_linear_fwd(Xr, A_i, a_i, "gelu")
        Zp_r = row_linear_fwd_partial(Y_r, B_i)
        dU_r = linear_bwd_dgrad(dZr, B_i, U_r, "gelu")
        dXp_r = linear_bwd_dgrad(dU_r, A_i, None, "none")
        # shard columns, over every token
        A_c = A_i[:, cols]
        a_c = None if a_i is None else a_i[cols]
        U_c, Y_c = column_linear_fwd(X, A_c, a_c, "gelu")
        dU_c = linear_bwd_dgrad(dZ, B_i[cols, :], U_c, "gelu")
        dB_c, _ = linear_bwd_wgrad(Y_c, dZ)          # rows Cf of dB_i
        dA_c, da_c = linear_bwd_wgrad(X, dU_c)       # columns Cf of dA_i
        out.update({f"U_{i}": U_r, f"Y_{i}": Y_r, f"Zp_{i}": Zp_r, f"dU_{i}": dU_r,
                    f"dXp_{i}": dXp_r, f"dB_{i}": dB_c, f"dA_{i}": dA_c})
        if a is not None:
            out[f"da_{i}"] = da_c
        Zp.append(Zp_r)
        dXp.append(dXp_r)
    if b is not None:
        out["db"] = np.asarray(dZ, np.float64).sum(axis=0)
    if len(shards) == p:
        out["Z"] = reduce_partials(Zp, b)
        out["dX"] = reduce_partials(dXp, None)
    return out


def attn_sampled(X, W, C, Ow, dQKV, dZa, p, rows, cols_q, cols_o, shards=None):
    shards = tuple(range(p)) if shards is None else tuple(shards)
    rows = np.asarray(rows)
    out = {}
    Zp, dXp = [], []
    for i in shards:
        W_i, C_i, Ow_i = shard_columns(W, p, i), shard_columns(C, p, i), shard_rows(Ow, p, i)
        dQKV_i = shard_columns(dQKV, p, i)
        QKV_r, _ = column_linear_fwd(X[rows], W_i, None, "none")
        Zpa_r = row_linear_fwd_partial(C_i[rows], Ow_i)
        dC_r = linear_bwd_dgrad(dZa[rows], Ow_i, None, "none")
        dXq_r = linear_bwd_dgrad(dQKV_i[rows], W_i, None, "none")
        dOw_c, _ = linear_bwd_wgrad(C_i[:, cols_o], dZa)      # rows Co of dOw_i
        dW_c, _ = linear_bwd_wgrad(X, dQKV_i[:, cols_q])       # columns Cq of dW_i
        out.update({f"QKV_{i}": QKV_r, f"Zpa_{i}": Zpa_r, f"dC_{i}": dC_r,
                    f"dXqp_{i}": dXq_r, f"dOw_{i}": dOw_c, f"dW_{i}": dW_c})
        Zp.append(Zpa_r)
        dXp.append(dXq_r)
    if len(shards) == p:
        out["Za"] = reduce_partials(Zp, None)
        out["dXq"] = reduce_partials(dXp, None)
    return out


def attn_block_sampled(X, W, Ow, dZa, p, batch, seq, heads, seqs, shards=None):
    """Token-row outputs of the attention block (oracle.attention.tp_attn_block)
    for the whole sequences `seqs`: attention stays inside a sequence, so the
    block on those sequences' rows gives exactly those rows of QKV_i, C_i,
    Zpa_i, dC_i, dQKV_i, dXqp_i, Za and dXq, and lse_i of those sequences. The
    weight gradients sum over every token and are not returned."""
    from .attention import tp_attn_block
    seqs = np.asarray(seqs)
    rows = (seqs[:, None] * seq + np.arange(seq)[None, :]).reshape(-1)
    g = tp_attn_block(np.asarray(X)[rows], W, Ow, np.asarray(dZa)[rows], p, len(seqs), seq,
                      heads, shards)
    return {k: v for k, v in g.items() if not k.startswith(("dW_", "dOw_"))}


# which axis of each device output the sample indexes
ROW_SAMPLED = ("U", "Y", "Zp", "dU", "dXp", "Z", "dX", "QKV", "Zpa", "dC", "dXqp", "Za", "dXq")


def sample_device_output(name: str, arr: np.ndarray, rows, cols_f=None, cols_q=None,
                         cols_o=None) -> np.ndarray:
    """The same slice of a full device output that the sampled oracle returns."""
    base = name.split("_")[0]
    if base in ROW_SAMPLED:
        return arr[np.asarray(rows)]
    if base == "dB":
        return arr[np.asarray(cols_f)]
    if base == "dA":
        return arr[:, np.asarray(cols_f)]
    if base == "da":
        return arr[np.asarray(cols_f)]
    if base == "dOw":
        return arr[np.asarray(cols_o)]
    if base == "dW":
        return arr[:, np.asarray(cols_q)]
    return arr  # db


def run_config_sampled(cfg, inputs, rows, cols_f=None, cols_q=None, cols_o=None) -> dict:
    g = {k: v.f64() for k, v in inputs.items()}
    out = {}
    if cfg.mlp:
        out.update(mlp_sampled(g["X"], g["A"], g.get("a"), g["B"], g.get("b"), g["dZ"], cfg.p,
                               rows, cols_f, cfg.shards, weights_are_shards=not cfg.full_weights))
    if cfg.attn:
        out.update(attn_sampled(g["X"], g["W"], g["C"], g["Ow"], g["dQKV"], g["dZa"], cfg.p,
                                rows, cols_q, cols_o, cfg.shards))
    return out


__all__ = ["mlp_sampled", "attn_sampled", "attn_block_sampled", "run_config_sampled",
           "sample_device_output", "gelu_tanh"]
