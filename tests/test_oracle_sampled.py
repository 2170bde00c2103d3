"""The sampled oracle returns exactly the slices of the full oracle (CPU only)."""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import sampled
from tp_inputs import get_config, make_inputs


def _small(name, micro_batch, seq):
    return dataclasses.replace(get_config(name), micro_batch=micro_batch, seq=seq)


@pytest.mark.parametrize("name,mb,seq", [("tiny", 8, 64), ("gpt2s", 1, 96), ("gpt350m", 1, 80),
                                         ("attn", 1, 72)])
def test_sampled_equals_full_slices(name, mb, seq):
    cfg = _small(name, mb, seq)
    inp = make_inputs(cfg)
    full = oracle.run_config(cfg, inp)
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(cfg.T, 9, replace=False))
    cols_f = np.sort(rng.choice(cfg.F, 5, replace=False)) if cfg.mlp else None
    cols_q = np.sort(rng.choice(cfg.Q, 5, replace=False)) if cfg.attn else None
    cols_o = np.sort(rng.choice(cfg.O, 5, replace=False)) if cfg.attn else None
    smp = sampled.run_config_sampled(cfg, inp, rows, cols_f, cols_q, cols_o)
    assert set(smp) == set(full)
    for k, v in smp.items():
        want = sampled.sample_device_output(k, full[k], rows, cols_f, cols_q, cols_o)
        assert v.shape == want.shape, k
        assert oracle.rel_fro(v, want) <= 1e-13, k


def test_sampled_shard_only_weights():
    """The 175B-class layout (only shard 0 drawn, at shard shape) at a small size."""
    cfg = dataclasses.replace(get_config("gpt175b"), h=64, seq=48)
    inp = make_inputs(cfg)
    assert inp["A"].shape == (64, cfg.F) and inp["B"].shape == (cfg.F, 64)
    full = oracle.run_config(cfg, inp)
    assert "Z" not in full and "Zp_0" in full
    rows, cols = np.array([0, 5, 47]), np.array([1, 2, 31])
    smp = sampled.run_config_sampled(cfg, inp, rows, cols)
    for k, v in smp.items():
        want = sampled.sample_device_output(k, full[k], rows, cols)
        assert oracle.rel_fro(v, want) <= 1e-13, k
