"""Seeded draws of the unsharded tensors of a workload.

Every tensor is drawn in float64 from ``numpy.random.default_rng((0, n, j))``
(n = workload number, j = position in ``INPUT_ORDER``; the 0 follows the
``random_seed=0`` of the mock dataset on the Megatron-LM guide page, section
"3.3 data preparation"), scaled by its standard deviation, converted to float32
and, for bf16 workloads, rounded to bfloat16 with round-to-nearest-even. Both the
oracle and the device path consume exactly these values: the oracle widens them
to float64, the device path uploads the raw bits.

Shapes (unsharded; ``p`` shards are contiguous blocks of them):
  MLP:        X[T,h]  A[h,pF]  a[pF]  B[pF,h]  b[h]  dZ[T,h]
  attention:  W[h,pQ]  C[T,pO]  Ow[pO,h]  dQKV[T,pQ]  dZa[T,h]
For a workload with ``full_weights=False`` only the run shard is drawn, at its
shard shape (A[h,F], B[F,h]).
"""
from __future__ import annotations

import numpy as np

from .configs import TPConfig

INPUT_ORDER = ("X", "A", "a", "B", "b", "dZ", "W", "C", "Ow", "dQKV", "dZa")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest, ties to even.
    NaN stays NaN (quiet bit set)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


class HostTensor:
    """One input tensor in its storage type.

    ``raw``  : np.float32 (f32 workloads) or np.uint16 bf16 bits (bf16 workloads)
    ``f64()``: the exact stored values widened to float64
    """

    def __init__(self, raw: np.ndarray, dtype: str):
        self.raw = raw
        self.dtype = dtype

    @property
    def shape(self):
        return self.raw.shape

    def f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.raw)
        return self.raw

    def f64(self) -> np.ndarray:
        return self.f32().astype(np.float64)


def _draw(cfg: TPConfig, name: str, shape, std: float) -> HostTensor:
    j = INPUT_ORDER.index(name)
    rng = np.random.default_rng((0, cfg.index, j))
    x32 = (rng.standard_normal(shape) * std).astype(np.float32)
    if cfg.dtype == "bf16":
        return HostTensor(f32_to_bf16_bits(x32), "bf16")
    return HostTensor(x32, "f32")


def _zeros(cfg: TPConfig, shape) -> HostTensor:
    if cfg.dtype == "bf16":
        return HostTensor(np.zeros(shape, np.uint16), "bf16")
    return HostTensor(np.zeros(shape, np.float32), "f32")


def input_shapes(cfg: TPConfig) -> dict:
    T, h, p = cfg.T, cfg.h, cfg.p
    wp = p if cfg.full_weights else 1
    shapes = {}
    if cfg.mlp:
        shapes["X"] = (T, h)
        shapes["A"] = (h, wp * cfg.F)
        if cfg.has_bias:
            shapes["a"] = (wp * cfg.F,)
        shapes["B"] = (wp * cfg.F, h)
        if cfg.has_bias:
            shapes["b"] = (h,)
        shapes["dZ"] = (T, h)
    if cfg.attn:
        shapes["X"] = (T, h)
        shapes["W"] = (h, wp * cfg.Q)
        shapes["C"] = (T, wp * cfg.O)
        shapes["Ow"] = (wp * cfg.O, h)
        shapes["dQKV"] = (T, wp * cfg.Q)
        shapes["dZa"] = (T, h)
    return shapes


def make_inputs(cfg: TPConfig, names=None) -> dict:
    """Draw the workload's inputs (all, or only ``names``) as HostTensors."""
    shapes = input_shapes(cfg)
    std = {
        "X": 1.0, "A": cfg.w_std, "B": cfg.w_std, "dZ": 1.0,
        "W": cfg.w_std, "C": 1.0, "Ow": cfg.w_std, "dQKV": 1.0, "dZa": 1.0,
        "a": cfg.b_std, "b": cfg.b_std,
    }
    out = {}
    for name in INPUT_ORDER:
        if name not in shapes or (names is not None and name not in names):
            continue
        if name in ("a", "b") and cfg.bias == "zero":
            out[name] = _zeros(cfg, shapes[name])
        else:
            out[name] = _draw(cfg, name, shapes[name], std[name])
    return out
