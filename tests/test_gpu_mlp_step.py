"""GPU parity of tp_mlp_step, the whole MLP step of every shard (one
persistent launch for the forward, the sums and the data gradients, then the
weight gradients as two products over the stacked shards), against the
float64 oracle and against the per-product calls, plus its queue bookkeeping:
consecutive calls, graph replay, the two halves called separately, the
forward and backward calls (with and without recompute), and a dependency wait
forced to give up.

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


def _mlp_buffers(cfg, dev):
    """Fresh stacked buffers of tp_mlp_step for cfg (outputs filled with a
    value no step leaves, so that anything not written shows)."""
    T, h, F, p = cfg.T, cfg.h, cfg.F, cfg.p
    bf = dict(device=dev, dtype=torch.bfloat16)
    f32 = dict(device=dev, dtype=torch.float32)
    m = {"U": torch.empty(T, p * F, **bf), "Y": torch.empty(T, p * F, **bf),
         "dU": torch.empty(T, p * F, **bf), "Zp": torch.empty(p, T, h, **f32),
         "dXp": torch.empty(p, T, h, **f32), "Z": torch.empty(T, h, **bf),
         "dX": torch.empty(T, h, **bf), "dB": torch.empty(p * F, h, **f32),
         "dA": torch.empty(h, p * F, **f32), "db": torch.empty(h, **f32),
         "da": torch.empty(p * F, **f32)}
    for t in m.values():
        t.fill_(-7.0)
    from tensor_transformer_layer_fwd_amd import _lib as L
    m["ws"] = torch.zeros(L.tp_mlp_step_workspace_size(T, h, F, p, L.TP_BF16), dtype=torch.uint8,
                          device=dev)
    return m


def _mlp_call(inp, m, part, recompute=False):
    from tensor_transformer_layer_fwd_amd import _lib as L
    L.tp_mlp_step(inp["X"], inp["A"], inp.get("a"), inp["B"], inp.get("b"), inp["dZ"], m["U"],
                  m["Y"], m["Zp"], m["Z"], m["dU"], m["dB"], m["db"] if "b" in inp else None,
                  m["dA"], m["da"] if "a" in inp else None, m["dXp"], m["dX"], m["ws"], part=part,
                  recompute=recompute)


SPLIT_CASES = [("gpt2s", dict(micro_batch=1, seq=1024)), ("gpt350m", dict(micro_batch=1, seq=2048)),
               ("gpt2s", dict(micro_batch=1, seq=1024, h=384))]


@pytest.mark.parametrize("name,kw", SPLIT_CASES)
def test_mlp_step_forward_then_backward_is_the_step(dev, name, kw):
    """tp_mlp_step_fwd then tp_mlp_step_bwd (recompute off) leave every
    output of tp_mlp_step bit for bit; the forward alone writes the forward's
    outputs and no gradient."""
    from tensor_transformer_layer_fwd_amd.shard import to_device
    cfg = _mlp_cfg(name, **kw)
    _say(f"mlp step fwd + bwd {name} T={cfg.T} h={cfg.h} p={cfg.p}")
    inp = {k: to_device(v, dev) for k, v in make_inputs(cfg).items()}
    one = _mlp_buffers(cfg, dev)
    _mlp_call(inp, one, "step")
    two = _mlp_buffers(cfg, dev)
    _mlp_call(inp, two, "fwd")
    torch.cuda.synchronize()
    for k in ("dU", "dXp", "dX", "dB", "dA"):
        assert bool((two[k] == -7.0).all()), f"the forward wrote {k}"
    for k in ("U", "Y", "Zp", "Z"):
        assert torch.equal(one[k], two[k]), k
    _mlp_call(inp, two, "bwd")
    torch.cuda.synchronize()
    for k in one:
        if k == "ws" or (k == "db" and "b" not in inp) or (k == "da" and "a" not in inp):
            continue
        assert torch.equal(one[k], two[k]), k
    assert int(two["ws"][:4].view(torch.int32).item()) == 0, "a dependency wait gave up"


@pytest.mark.parametrize("name,kw", SPLIT_CASES)
def test_mlp_step_backward_rebuilds_y(dev, name, kw):
    """With recompute the backward rebuilds Y from U after the forward's Y
    was overwritten: Y equals what tp_linear_bwd_dgrad_recompute rebuilds for
    each shard, bit for bit; every output that does not read Y equals the
    stored step's bit for bit, and dB (which reads the rebuilt Y) is within
    the step tolerance of the oracle."""
    from tensor_transformer_layer_fwd_amd import _lib as L
    from tensor_transformer_layer_fwd_amd.shard import to_device
    cfg = _mlp_cfg(name, **kw)
    _say(f"mlp step bwd recompute {name} T={cfg.T} h={cfg.h} p={cfg.p}")
    inputs = make_inputs(cfg)
    inp = {k: to_device(v, dev) for k, v in inputs.items()}
    ref = _mlp_buffers(cfg, dev)
    _mlp_call(inp, ref, "step")
    m = _mlp_buffers(cfg, dev)
    _mlp_call(inp, m, "fwd")
    m["Y"].fill_(3.0)  # Y is transient between the calls
    _mlp_call(inp, m, "bwd", recompute=True)
    torch.cuda.synchronize()
    F = cfg.F
    for i in range(cfg.p):
        cols = slice(i * F, (i + 1) * F)
        y = torch.empty(cfg.T, F, device=dev, dtype=torch.bfloat16)
        du = torch.empty_like(y)
        L.tp_linear_bwd_dgrad_recompute(inp["dZ"], inp["B"][cols], m["U"][:, cols], du, y)
        torch.cuda.synchronize()
        assert torch.equal(m["Y"][:, cols], y), f"Y_{i}"
        assert torch.equal(m["dU"][:, cols], du), f"dU_{i}"
    for k in ("U", "Zp", "Z", "dU", "dXp", "dX", "dA") + (("da",) if "a" in inp else ()) + \
            (("db",) if "b" in inp else ()):
        assert torch.equal(ref[k], m[k]), k
    want = oracle.run_config(cfg, inputs)
    for i in range(cfg.p):
        e = oracle.rel_fro(m["dB"][i * F:(i + 1) * F].double().cpu().numpy(), want[f"dB_{i}"])
        assert e <= 5e-3, (i, e)
    assert int(m["ws"][:4].view(torch.int32).item()) == 0, "a dependency wait gave up"


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


def test_mlp_step_per_product_call_leaves_the_counters(dev):
    """A call that runs the step as per-product calls (here: a bias that is
    not 16-byte aligned) on the workspace of fused calls uses only the scratch
    past the persistent launch's counters: the next fused call gives the
    first one's bits, and the per-product call's outputs match the oracle."""
    from tensor_transformer_layer_fwd_amd import _lib as L
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = _mlp_cfg("gpt2s", micro_batch=1, seq=1024)
    _say(f"mlp step per-product call on a fused workspace T={cfg.T}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev)
    step.run_eager()
    want = step.results()
    inp, m, o = step.inp, step.mlp, step.out
    pF = inp["a"].shape[0]
    a_off = torch.empty(pF + 1, dtype=inp["a"].dtype, device=dev)[1:]  # 2 bytes off
    a_off.copy_(inp["a"])
    assert a_off.data_ptr() % 16 != 0
    for v in o.values():
        v.fill_(float("nan"))
    L.tp_mlp_step(inp["X"], inp["A"], a_off, inp["B"], inp.get("b"), inp["dZ"], m["U"], m["Y"],
                  m["Zp"], o["Z"], m["dU"], m["dB"], o.get("db"), m["dA"], m.get("da"), m["dXp"],
                  o["dX"], step.step_ws)
    torch.cuda.synchronize()
    got = step.results()
    ref = oracle.run_config(cfg, inputs)
    for k, r in ref.items():
        e = oracle.rel_fro(got[k], r)
        assert e <= 5e-3, (k, e)
    step.run_eager()
    got = step.results()
    for k in want:
        np.testing.assert_array_equal(got[k], want[k], err_msg=f"fused call after: {k}")
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
