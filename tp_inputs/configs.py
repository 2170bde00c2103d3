"""The five workloads of the tensor-parallel shard, as shapes and distributions.

Notation follows the Megatron page (zzmblog.top), section "Tensor Parallelism /
mathematical principles": X in R^{b x h} with b read as tokens T (micro-batch x
sequence, flattened), the first MLP weight A in R^{h x 4h} split by columns into
p shards A_i in R^{h x 4h/p}, the second weight B in R^{4h x h} split by rows into
B_i in R^{4h/p x h}. Section "Transformer-layer tensor parallelism" of the same
page applies the column split to the attention QKV projection and the row split
to the attention output projection.

Per shard:  F = 4h/p (fc1 output width), Q = 3h/p (QKV output width),
O = h/p (output-projection input width).
"""
from __future__ import annotations

from dataclasses import dataclass


@dataclass(frozen=True)
class TPConfig:
    name: str
    index: int  # 1-based workload number; it seeds the draws
    dtype: str  # "f32" or "bf16" (bf16 storage, fp32 accumulation)
    micro_batch: int
    seq: int
    h: int
    p: int
    shards: tuple  # shard indices that run on the device
    mlp: bool
    attn: bool
    w_std: float
    bias: str  # "zero" | "normal" | "none"
    b_std: float = 0.0
    heads: int = 0
    full_weights: bool = True  # False: only the run shards are drawn, at shard shape

    @property
    def T(self) -> int:
        return self.micro_batch * self.seq

    @property
    def F(self) -> int:
        return 4 * self.h // self.p

    @property
    def Q(self) -> int:
        return 3 * self.h // self.p

    @property
    def O(self) -> int:
        return self.h // self.p

    @property
    def has_bias(self) -> bool:
        return self.bias != "none"

    def gemm_flops(self) -> int:
        """Algorithmic GEMM flops (2*M*N*K per product) of one fwd+bwd step over
        the shards that run: each linear costs one forward, one dgrad and one
        wgrad product of equal size."""
        T, h = self.T, self.h
        n = len(self.shards)
        f = 0
        if self.mlp:
            f += n * 2 * (3 * 2 * T * h * self.F)  # fc1 + fc2, three products each
        if self.attn:
            f += n * 3 * 2 * T * h * self.Q  # QKV
            f += n * 3 * 2 * T * self.O * h  # output projection
        return f


CONFIGS = {
    # Tiny fp32 check, the shape of the quick-start model on the Megatron-LM guide
    # page (hidden 12, seq 64, batch 8).
    "tiny": TPConfig(
        name="tiny", index=1, dtype="f32", micro_batch=8, seq=64, h=12, p=2,
        shards=(0, 1), mlp=True, attn=False, w_std=0.02, bias="zero",
    ),
    # GPT-2-small (h=768, seq 1024) with TP=2.
    "gpt2s": TPConfig(
        name="gpt2s", index=2, dtype="bf16", micro_batch=4, seq=1024, h=768, p=2,
        shards=(0, 1), mlp=True, attn=False, w_std=0.02, bias="normal", b_std=0.01,
    ),
    # Attention projections, h=1024, 16 heads, TP=2.
    "attn": TPConfig(
        name="attn", index=3, dtype="bf16", micro_batch=8, seq=512, h=1024, p=2,
        shards=(0, 1), mlp=False, attn=True, w_std=0.02, bias="none", heads=16,
    ),
    # ~350M GPT layer (h=1024), TP=4: MLP and attention projections.
    "gpt350m": TPConfig(
        name="gpt350m", index=4, dtype="bf16", micro_batch=6, seq=1024, h=1024, p=4,
        shards=(0, 1, 2, 3), mlp=True, attn=True, w_std=0.02, bias="none", heads=16,
    ),
    # 175B-class layer (h=12288), TP=8: one GPU's shard at its real shape.
    "gpt175b": TPConfig(
        name="gpt175b", index=5, dtype="bf16", micro_batch=1, seq=2048, h=12288, p=8,
        shards=(0,), mlp=True, attn=False, w_std=0.006, bias="none",
        full_weights=False,
    ),
}


def get_config(name: str) -> TPConfig:
    if name not in CONFIGS:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
    return CONFIGS[name]
