"""Seeded input generator: reproducibility, shapes, bf16 rounding (CPU only)."""
import numpy as np
import pytest
import torch

from tp_inputs import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, get_config, make_inputs
from tp_inputs.generate import input_shapes


def test_bf16_rne_known_values():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.0, 0.0, -0.0, 3.0e38, 1e-40,
                  np.inf, -np.inf], np.float32)
    bits = f32_to_bf16_bits(x)
    # 1+2^-8 is a tie between 1 and 1+2^-7: to even (1.0); 1+3*2^-8 ties up to 1+2^-6
    assert bits.tolist()[:6] == [0x3F80, 0x3F80, 0x3F82, 0xC000, 0x0000, 0x8000]
    assert bits[8] == 0x7F80 and bits[9] == 0xFF80
    assert np.isnan(bf16_bits_to_f32(f32_to_bf16_bits(np.array([np.nan], np.float32))))[0]


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-20, 20, 100000)).astype(np.float32)
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(bf16_bits_to_f32(ours), torch.from_numpy(ours.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_reproducible_and_distinct():
    cfg = get_config("gpt2s")
    a = make_inputs(cfg, names=("X", "a"))
    b = make_inputs(cfg, names=("X", "a"))
    np.testing.assert_array_equal(a["X"].raw, b["X"].raw)
    assert abs(float(np.std(a["X"].f64())) - 1.0) < 0.01
    assert abs(float(np.std(a["a"].f64())) - 0.01) < 0.001
    other = make_inputs(get_config("attn"), names=("X",))
    assert not np.array_equal(a["X"].raw[:16, :16], other["X"].raw[:16, :16])


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_shapes(name):
    cfg = get_config(name)
    shp = input_shapes(cfg)
    T, h = cfg.T, cfg.h
    assert shp["X"] == (T, h)
    if cfg.mlp:
        wp = cfg.p if cfg.full_weights else 1
        assert shp["A"] == (h, wp * cfg.F) and shp["B"] == (wp * cfg.F, h)
        assert cfg.F * cfg.p == 4 * h
    if cfg.attn:
        assert shp["W"] == (h, cfg.p * cfg.Q) and shp["Ow"] == (cfg.p * cfg.O, h)


def test_workload_flops():
    # six GEMMs of 2*T*h*F per shard for the MLP pair
    c = get_config("gpt2s")
    assert c.gemm_flops() == 2 * 6 * 2 * 4096 * 768 * 1536
    assert abs(c.gemm_flops() / 1e9 - 115.96) < 0.01
    assert abs(get_config("gpt175b").gemm_flops() / 1e9 - 1855.43) < 0.01
    assert abs(get_config("gpt350m").gemm_flops() / 1e9 - 463.86) < 0.01
    assert abs(get_config("attn").gemm_flops() / 1e9 - 103.08) < 0.01
