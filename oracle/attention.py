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
