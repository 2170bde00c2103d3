"""GPU parity of tp_mlp_step, the whole MLP step of every shard (one
persistent launch for the forward, the sums and the data gradients, then the
weight gradients as two products over the stacked shards), against the
float64 oracle and against the per-product calls, plus its queue bookkeeping:
consecutive calls, graph replay, the two halves called separately, and a
dependency wait forced to give up.

Tolerance: 5e-3 relative Frobenius error per output against the oracle (bf16
storage). The weight-gradient launch runs the tiles past the last whole
multiple of the CU count as K slices added by a second launch (288 tiles at
h = 768 leave 32, each in 8 slices on a 256-CU device); the h = 384 cases have
fewer tiles than CUs, so every tile is sliced. Against the per-product calls, which run the same K order per
output element in every fused tile, the forward outputs and data gradients
agree bitwise; the stacked weight-gradient products may split K otherwise
than the per-shard calls, so the weight gradients agree within 1e-5 relative.
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


def _mlp_cfg(name, **kw):
    if "p" in kw:
        kw["shards"] = tuple(range(kw["p"]))
    return dataclasses.replace(get_config(name), attn=False, **kw)


CASES = [
    ("gpt2s", dict(micro_batch=1, seq=1024)),                   # T = 1024: one row block per XCD
    ("gpt2s", dict(micro_batch=2, seq=1024)),                   # T = 2048
    ("gpt350m", dict(micro_batch=1, seq=2048)),                 # p = 4, F = h = 1024, no bias
    ("gpt2s", dict(micro_batch=1, seq=1024, p=1)),              # one shard, F = 3072
    ("gpt2s", dict(micro_batch=1, seq=1024, h=256, p=8)),       # F = 128, p = 8
    # 72 weight-gradient tiles, fewer than the CUs: every tile as K slices,
    # two of 512 rows (T = 1024) or three of 1024 rows (T = 3072)
    ("gpt2s", dict(micro_batch=1, seq=1024, h=384)),
    ("gpt2s", dict(micro_batch=3, seq=1024, h=384)),
]


@pytest.mark.parametrize("name,kw", CASES)
def test_mlp_step_against_the_oracle(dev, name, kw):
    from tensor_transformer_layer_fwd_amd import _lib as L
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = _mlp_cfg(name, **kw)
    assert L.tp_mlp_step_plan(cfg.T, cfg.h, cfg.F, cfg.p, L.TP_BF16), "expected the fused path"
    _say(f"mlp step {name} T={cfg.T} h={cfg.h} F={cfg.F} p={cfg.p} bias={cfg.has_bias}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev)
    assert step.step_call
    step.run_eager()
    got = step.results()
    assert int(step.step_ws[:4].view(torch.int32).item()) == 0, "a dependency wait gave up"
    ref = oracle.run_config(cfg, inputs)
    worst = (0.0, None)
    for k, r in ref.items():
        e = oracle.rel_fro(got[k], r)
        worst = max(worst, (e, k))
        assert e <= 5e-3, (k, e)
    _say(f"  worst rel err {worst[0]:.3e} ({worst[1]})")


@pytest.mark.parametrize("name", ["gpt2s", "gpt350m"])
def test_mlp_step_against_per_product_calls(dev, name):
    """The full-size MLP of the workload: fused step against the per-product
    calls on the same inputs."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = _mlp_cfg(name)
    _say(f"mlp step vs per-product calls {name} T={cfg.T}")
    inputs = make_inputs(cfg)
    ref_step = ShardStep(cfg, inputs, dev, step_call=False)
    ref_step.run_eager()
    want = ref_step.results()
    del ref_step
    step = ShardStep(cfg, inputs, dev)
    step.run_eager()
    got = step.results()
    for k in want:
        if k.startswith(("dB_", "dA_", "da_")) or k == "db":
            assert oracle.rel_fro(got[k], want[k]) <= 1e-5, k
        else:
            np.testing.assert_array_equal(got[k], want[k], err_msg=k)


def test_mlp_step_repeats_replays_and_halves(dev):
    """Three consecutive calls, graph replays with eager work between them, and
    rows-then-wgrad as two calls all give the first call's bits: the queues'
    counters are back at zero after every call."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = _mlp_cfg("gpt2s", micro_batch=2, seq=1024)
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev)
    step.run_eager()
    want = step.results()
    for rep in range(2):
        step.run_eager()
        got = step.results()
        for k in want:
            np.testing.assert_array_equal(got[k], want[k], err_msg=f"call {rep + 2}: {k}")
    for v in step.out.values():
        v.fill_(float("nan"))
    step.mlp_step("rows")
    step.mlp_step("wgrad")
    got = step.results()
    for k in want:
        np.testing.assert_array_equal(got[k], want[k], err_msg=f"rows + wgrad: {k}")
    step.capture()
    for rep in range(3):
        for v in step.out.values():
            v.fill_(float("nan"))
        step.run()
        torch.cuda.synchronize()
        got = step.results()
        for k in want:
            np.testing.assert_array_equal(got[k], want[k], err_msg=f"replay {rep}: {k}")
    assert int(step.step_ws[:4].view(torch.int32).item()) == 0


def test_mlp_step_wait_that_gives_up_still_ends(dev):
    """With the wait limit forced to give up at the first unmet check, the
    call still runs to its end (every block exits) and the error word tells;
    the next call with the default limit is exact again (the counters were
    reset by the launch that gave up)."""
    from tensor_transformer_layer_fwd_amd import _lib as L
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = _mlp_cfg("gpt2s", micro_batch=1, seq=1024)
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev)
    step.run_eager()
    want = step.results()
    try:
        L.tp_set_wait_limit(-1)
        step.run_eager()
        torch.cuda.synchronize()  # returns: every block exited
    finally:
        L.tp_set_wait_limit(0)
    err = int(step.step_ws[:4].view(torch.int32).item())
    _say(f"  error word after the forced give-up: {err}")
    step.step_ws[:4].zero_()
    step.run_eager()
    got = step.results()
    assert int(step.step_ws[:4].view(torch.int32).item()) == 0
    for k in want:
        np.testing.assert_array_equal(got[k], want[k], err_msg=k)


def test_mlp_step_clock_counters(dev):
    """Block 0 of the first launch leaves its shader and real-time clock
    readings in the workspace: the clock they imply is a plausible engine
    clock (0.5 to 2.6 GHz)."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = _mlp_cfg("gpt2s")
    step = ShardStep(cfg, make_inputs(cfg), dev)
    step.run_eager()
    torch.cuda.synchronize()
    c = step.step_ws[64:96].view(torch.int64).cpu().tolist()
    mhz = (c[2] - c[0]) / ((c[3] - c[1]) / 100e6) / 1e6
    _say(f"  engine clock over the persistent launch: {mhz:.0f} MHz")
    assert 500 <= mhz <= 2600
