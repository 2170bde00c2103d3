"""CPU oracle of one shard's attention core (float64).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP path and imports nothing from it.

Source: the "Megatron" page (zzmblog.top), "Transformer-layer tensor
parallelism": the QKV projection is split by output columns and the output
projection by input rows, so each shard holds whole heads and runs their
attention on its own Q, K and V; the result C_i feeds the row-split output
projection. The same page's optimisation list recommends a fused
(FlashAttention-style) attention kernel. The pages do not write the attention
out; this is the textbook scaled dot-product attention of a GPT decoder, with
these readings:

  * QKV_i [T, 3*H*d] holds [Q | K | V], each third head-major: head j at
    columns j*d .. j*d+d-1 of its third;
  * T = batch * seq tokens, sequence-major; attention stays inside a sequence;
  * causal: position q attends to positions k <= q;
  * scores are scaled by 1/sqrt(d);
  * C_i [T, H*d]: head j's output at columns j*d ..;
  * lse[b, j, q] = log(sum_k exp(score[b, j, q, k])) (natural log), the
    softmax normaliser a backward pass needs.

Every step is the plain definition in float64 on the exact stored input values.
Pinned by tests/test_oracle_attention.py: the forward by a pure-Python brute
force, closed forms for Q = 0 and for the first position, one-hot attention,
causal/non-causal agreement on the last row, sequence independence and
normalisation; the backward by central finite differences of a scalar loss
through the forward, the closed form of dV, a pure-Python brute force of the
chain rule, and the zero-sum of each query's score gradient.
"""
from __future__ import annotations

import math

import numpy as np


def split_qkv(QKV, batch: int, seq: int, heads: int, d: int):
    """Q, K, V as [batch, seq, heads, d] views of QKV [batch*seq, 3*heads*d]."""
    X = np.asarray(QKV, dtype=np.float64).reshape(batch, seq, 3, heads, d)
    return X[:, :, 0], X[:, :, 1], X[:, :, 2]


def attention_core_fwd(QKV, batch: int, seq: int, heads: int, d: int, causal: bool = True):
    """C [batch*seq, heads*d] and lse [batch, heads, seq] of softmax(Q K^T / sqrt(d)) V."""
    q, k, v = split_qkv(QKV, batch, seq, heads, d)
    s = np.einsum("bqhd,bkhd->bhqk", q, k) / math.sqrt(d)
    if causal:
        s = np.where(np.tril(np.ones((seq, seq), dtype=bool)), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    den = e.sum(axis=-1, keepdims=True)
    o = np.einsum("bhqk,bkhd->bqhd", e / den, v)
    return o.reshape(batch * seq, heads * d), (m + np.log(den))[..., 0]


def attention_core_bwd(QKV, dC, batch: int, seq: int, heads: int, d: int, causal: bool = True):
    """dQKV [batch*seq, 3*heads*d] ([dQ | dK | dV], laid out as QKV) for upstream dC.

    With S = Q K^T / sqrt(d) (masked), P = softmax(S), C = P V: dV = P^T dC,
    dP = dC V^T, dS = P * (dP - rowsum(dP * P)), dQ = dS K / sqrt(d),
    dK = dS^T Q / sqrt(d). rowsum(dP * P) equals rowsum(dC * C), the form a
    fused backward uses; the oracle takes the definition.
    """
    q, k, v = split_qkv(QKV, batch, seq, heads, d)
    dc = np.asarray(dC, dtype=np.float64).reshape(batch, seq, heads, d)
    s = np.einsum("bqhd,bkhd->bhqk", q, k) / math.sqrt(d)
    if causal:
        s = np.where(np.tril(np.ones((seq, seq), dtype=bool)), s, -np.inf)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    pr = e / e.sum(axis=-1, keepdims=True)
    dv = np.einsum("bhqk,bqhd->bkhd", pr, dc)
    dp = np.einsum("bqhd,bkhd->bhqk", dc, v)
    ds = pr * (dp - (dp * pr).sum(axis=-1, keepdims=True))
    dq = np.einsum("bhqk,bkhd->bqhd", ds, k) / math.sqrt(d)
    dk = np.einsum("bhqk,bqhd->bkhd", ds, q) / math.sqrt(d)
    return np.stack([dq, dk, dv], axis=2).reshape(batch * seq, 3 * heads * d)


def tp_attn_block(X, W, Ow, dZa, p: int, batch: int, seq: int, heads: int, shards=None,
                  d: int = 64, causal: bool = True):
    """The attention block of a Transformer layer over p tensor-parallel
    shards, forward then backward, with the attention core between the
    projections ("Megatron" page, "Transformer-layer tensor parallelism": the
    QKV projection split by output columns, the output projection by input
    rows, each shard running the attention of its own heads).

    Per shard i, with W_i = W[:, i*Q:(i+1)*Q] (Q = 3*heads*d/p, read as
    [Q | K | V] of the shard's heads/p heads) and Ow_i = Ow[i*O:(i+1)*O, :]
    (O = heads*d/p):
        QKV_i = X W_i;  C_i, lse_i = attention core of QKV_i;  Zpa_i = C_i Ow_i
        dC_i = dZa Ow_i^T;  dOw_i = C_i^T dZa;  dQKV_i = core backward of dC_i
        dW_i = X^T dQKV_i;  dXqp_i = dQKV_i W_i^T
    and the sums over shards Za = sum_i Zpa_i, dXq = sum_i dXqp_i (every shard ran).
    """
    from .oracle import (column_linear_fwd, linear_bwd_dgrad, linear_bwd_wgrad,
                         reduce_partials, row_linear_fwd_partial, shard_columns, shard_rows)
    if heads % p:
        raise ValueError("the heads must split evenly over the shards")
    shards = tuple(range(p)) if shards is None else tuple(shards)
    H = heads // p
    out = {}
    Zp, dXp = [], []
    for i in shards:
        W_i, Ow_i = shard_columns(W, p, i), shard_rows(Ow, p, i)
        QKV_i, _ = column_linear_fwd(X, W_i, None, "none")
        C_i, lse_i = attention_core_fwd(QKV_i, batch, seq, H, d, causal)
        Zpa_i = row_linear_fwd_partial(C_i, Ow_i)
        dC_i = linear_bwd_dgrad(dZa, Ow_i, None, "none")
        dOw_i, _ = linear_bwd_wgrad(C_i, dZa)
        dQKV_i = attention_core_bwd(QKV_i, dC_i, batch, seq, H, d, causal)
        dW_i, _ = linear_bwd_wgrad(X, dQKV_i)
        dXq_i = linear_bwd_dgrad(dQKV_i, W_i, None, "none")
        out.update({f"QKV_{i}": QKV_i, f"C_{i}": C_i, f"lse_{i}": lse_i, f"Zpa_{i}": Zpa_i,
                    f"dC_{i}": dC_i, f"dOw_{i}": dOw_i, f"dQKV_{i}": dQKV_i, f"dW_{i}": dW_i,
                    f"dXqp_{i}": dXq_i})
        Zp.append(Zpa_i)
        dXp.append(dXq_i)
    if len(shards) == p:
        out["Za"] = reduce_partials(Zp, None)
        out["dXq"] = reduce_partials(dXp, None)
    return out
