"""GPU parity of tp_attn_proj_step, every shard's attention projections (one
persistent launch for QKV, the output projection with its sum, dC and the dXq
partials with their sum, then the weight gradients as two products over the
stacked shards), against the float64 oracle and against the per-product calls,
stage by stage against one call, and on repeated calls.

Tolerance: 5e-3 relative Frobenius error per output against the oracle (bf16
storage). Against the per-product calls, which run the same K order per output
element, every output other than the weight gradients agrees bitwise; the
stacked weight-gradient products may split K otherwise than the per-shard
calls, so dO_i and dW_i agree within 1e-5 relative.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from tp_inputs import get_config, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a ROCm GPU")
    import tensor_transformer_layer_fwd_amd as tp  # noqa: F401  (fails loudly if not built)
    return torch.device("cuda:0")


def _cfg(name, **kw):
    return dataclasses.replace(get_config(name), mlp=False, **kw)


CASES = [
    ("attn", dict(micro_batch=2, seq=512)),      # T = 1024: 128 x 128 tiles, p = 2
    ("attn", dict(micro_batch=4, seq=512)),      # T = 2048: 256 x 128 tiles
    ("gpt350m", dict(micro_batch=1, seq=2048)),  # p = 4, Q = 768, O = 256
]


@pytest.mark.parametrize("name,kw", CASES)
def test_attn_proj_step_against_the_oracle(dev, name, kw):
    from tensor_transformer_layer_fwd_amd import _lib as L
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = _cfg(name, **kw)
    assert L.tp_attn_proj_step_plan(cfg.T, cfg.h, cfg.Q, cfg.O, cfg.p, L.TP_BF16)
    _say(f"attn proj step {name} T={cfg.T} h={cfg.h} Q={cfg.Q} O={cfg.O} p={cfg.p}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev)
    assert step.proj_call
    step.run_eager()
    got = step.results()
    assert int(step.proj_ws[:4].view(torch.int32).item()) == 0, "a sum's wait gave up"
    ref = oracle.run_config(cfg, inputs)
    worst = (0.0, None)
    for k, r in ref.items():
        e = oracle.rel_fro(got[k], r)
        worst = max(worst, (e, k))
        assert e <= 5e-3, (k, e)
    _say(f"  worst rel err {worst[0]:.3e} ({worst[1]})")


@pytest.mark.parametrize("name,kw", CASES[1:])
def test_attn_proj_step_against_per_product_calls(dev, name, kw):
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = _cfg(name, **kw)
    _say(f"attn proj step vs per-product calls {name} T={cfg.T}")
    inputs = make_inputs(cfg)
    ref_step = ShardStep(cfg, inputs, dev, step_call=False)
    assert not ref_step.proj_call
    ref_step.run_eager()
    want = ref_step.results()
    del ref_step
    step = ShardStep(cfg, inputs, dev)
    step.run_eager()
    got = step.results()
    for k in want:
        if k.startswith(("dOw_", "dW_")):
            assert oracle.rel_fro(got[k], want[k]) <= 1e-5, k
        else:
            np.testing.assert_array_equal(got[k], want[k], err_msg=k)


def test_attn_proj_step_stages_and_repeats(dev):
    """The five stages as five calls give the one call's outputs bit for bit,
    and so do a second and third call on the same workspace (the counters
    are left zeroed)."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = _cfg("attn", micro_batch=4, seq=512)
    _say(f"attn proj step stages T={cfg.T}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev)
    step.proj_step(31)
    want = step.results()
    for stage in (1, 2, 4, 8, 16):
        step.proj_step(stage)
    got = step.results()
    for k in want:
        np.testing.assert_array_equal(got[k], want[k], err_msg=f"stages: {k}")
    for rep in range(2):
        step.proj_step(31)
        got = step.results()
        for k in want:
            np.testing.assert_array_equal(got[k], want[k], err_msg=f"call {rep + 2}: {k}")
    assert int(step.proj_ws[:4].view(torch.int32).item()) == 0


@pytest.mark.parametrize("kw", [dict(micro_batch=1, seq=680),          # ragged T: per-product path
                                dict(micro_batch=1, seq=512, dtype="f32")])  # fp32: per-product path
def test_attn_proj_step_outside_the_fused_shapes(dev, kw):
    """Shapes and dtypes the persistent launch does not take run the same
    stages as per-product calls inside tp_attn_proj_step; against the oracle
    (fp32: 1e-5)."""
    from tensor_transformer_layer_fwd_amd import _lib as L
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = _cfg("attn", **kw)
    dt = L.TP_BF16 if cfg.dtype == "bf16" else L.TP_F32
    assert not L.tp_attn_proj_step_plan(cfg.T, cfg.h, cfg.Q, cfg.O, cfg.p, dt)
    _say(f"attn proj step outside the fused shapes T={cfg.T} dtype={cfg.dtype}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev)
    assert step.proj_call
    step.run_eager()
    got = step.results()
    ref = oracle.run_config(cfg, inputs)
    tol = 5e-3 if cfg.dtype == "bf16" else 1e-5
    for k, r in ref.items():
        e = oracle.rel_fro(got[k], r)
        assert e <= tol, (k, e)
