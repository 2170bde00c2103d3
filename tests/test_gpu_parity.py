"""GPU parity: the HIP path (through the C ABI) against the float64 CPU oracle.

Tolerance: maximum relative Frobenius error 1e-5 for fp32 and 5e-3 for bf16
(bf16 storage, fp32 accumulation), per output tensor.

- every entry point on odd, ragged and tile-multiple shapes, with row strides
  wider than the rows and NaN guard bands around every output;
- the hand-worked example of tests/golden (exact values) in fp32 and bf16;
- each workload at a reduced token count (every output compared in full) and
  at its full size in the launch configuration the benchmark times (graph
  replay), compared on sampled rows and columns;
- determinism (bitwise-equal reruns) and graph replay against eager runs.
"""
import dataclasses
import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import sampled
from tp_inputs import bf16_bits_to_f32, f32_to_bf16_bits, get_config, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"bf16": 5e-3, "f32": 1e-5}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tensor_transformer_layer_fwd_amd as tp  # noqa: F401  (fails loudly if not built)
    return torch.device("cuda:0")


# --------------------------------------------------------------------------- #
# helpers                                                                     #
# --------------------------------------------------------------------------- #
def rand(rng, shape, std, dt):
    """Seeded values exactly representable in dt; returns (float64 array, device-ready array)."""
    x = (rng.standard_normal(shape) * std).astype(np.float32)
    if dt == "bf16":
        bits = f32_to_bf16_bits(x)
        return bf16_bits_to_f32(bits).astype(np.float64), bits
    return x.astype(np.float64), x


def upload(raw, dt, device, pad=0):
    """Device tensor (row stride = cols + pad) holding raw values."""
    if raw.ndim == 1:
        t = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16) if dt == "bf16" \
            else torch.from_numpy(raw)
        return t.to(device)
    r, c = raw.shape
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    buf = torch.zeros(r, c + pad, dtype=tdt, device=device)
    src = torch.from_numpy(raw.view(np.int16)).view(torch.bfloat16) if dt == "bf16" \
        else torch.from_numpy(raw)
    buf[:, :c] = src.to(device)
    return buf[:, :c]


class Guarded:
    """An output view inside a NaN-filled buffer: rows x cols with row stride
    cols + pad, plus guard rows above and below."""

    def __init__(self, rows, cols, dt, device, pad=3, guard_rows=2):
        self.tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        self.buf = torch.full((rows + 2 * guard_rows, cols + pad), float("nan"), dtype=self.tdt,
                              device=device)
        self.rows, self.cols, self.g = rows, cols, guard_rows
        self.view = self.buf[guard_rows:guard_rows + rows, :cols]

    def check_guards(self):
        b = self.buf.float().cpu().numpy()
        mask = np.ones(b.shape, bool)
        mask[self.g:self.g + self.rows, :self.cols] = False
        assert np.all(np.isnan(b[mask])), "a kernel wrote outside its output"

    def value(self):
        self.check_guards()
        return self.view.float().cpu().numpy().astype(np.float64)


def err(got, ref):
    return oracle.rel_fro(got, ref)


DTS = ["bf16", "f32"]
SHAPES = [(1, 1, 1), (17, 63, 65), (129, 65, 17), (300, 129, 200), (256, 256, 256),
          (512, 128, 384), (130, 520, 264)]


# --------------------------------------------------------------------------- #
# entry points on odd shapes                                                   #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("T,h,n", SHAPES)
@pytest.mark.parametrize("act,bias", [("gelu", True), ("gelu", False), ("none", False)])
def test_column_linear_fwd(dev, dt, T, h, n, act, bias):
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"column_fwd dt={dt} T={T} h={h} n={n} act={act} bias={bias}")
    rng = np.random.default_rng(T * 7 + h * 3 + n)
    X, Xr = rand(rng, (T, h), 1.0, dt)
    A, Ar = rand(rng, (h, n), 0.05, dt)
    a, ar = rand(rng, (n,), 0.1, dt) if bias else (None, None)
    Y = Guarded(T, n, dt, dev)
    U = Guarded(T, n, dt, dev) if act == "gelu" else None  # same row stride as Y
    tp.tp_column_linear_fwd(upload(Xr, dt, dev, pad=5), upload(Ar, dt, dev, pad=9),
                            None if ar is None else upload(ar, dt, dev), Y.view,
                            None if U is None else U.view, act=act)
    torch.cuda.synchronize()
    U_ref, Y_ref = oracle.column_linear_fwd(X, A, a, act)
    assert err(Y.value(), Y_ref) <= TOL[dt]
    if U is not None:
        assert err(U.value(), U_ref) <= TOL[dt]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("T,k,h", SHAPES)
def test_row_linear_fwd_partial(dev, dt, T, k, h):
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"row_partial dt={dt} T={T} k={k} h={h}")
    rng = np.random.default_rng(T + 5 * k + 11 * h)
    Y, Yr = rand(rng, (T, k), 1.0, dt)
    B, Br = rand(rng, (k, h), 0.05, dt)
    Z = Guarded(T, h, "f32", dev)
    tp.tp_row_linear_fwd_partial(upload(Yr, dt, dev, pad=1), upload(Br, dt, dev, pad=8), Z.view)
    torch.cuda.synchronize()
    # fp32 output of a bf16 product: only accumulation order differs
    assert err(Z.value(), oracle.row_linear_fwd_partial(Y, B)) <= (1e-5 if dt == "f32" else 1e-5)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("T,k,n", SHAPES)
@pytest.mark.parametrize("act,out_dt", [("gelu", "same"), ("none", "f32"), ("none", "same")])
def test_linear_bwd_dgrad(dev, dt, T, k, n, act, out_dt):
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"dgrad dt={dt} T={T} k={k} n={n} act={act} out={out_dt}")
    odt = dt if out_dt == "same" else "f32"
    rng = np.random.default_rng(3 * T + k + 13 * n)
    dO, dOr = rand(rng, (T, n), 1.0, dt)
    W, Wr = rand(rng, (k, n), 0.05, dt)
    U, Ur = rand(rng, (T, k), 1.5, dt)
    dIn = Guarded(T, k, odt, dev)
    tp.tp_linear_bwd_dgrad(upload(dOr, dt, dev, pad=2), upload(Wr, dt, dev, pad=6),
                           upload(Ur, dt, dev, pad=4) if act == "gelu" else None, dIn.view,
                           act=act)
    torch.cuda.synchronize()
    ref = oracle.linear_bwd_dgrad(dO, W, U if act == "gelu" else None, act)
    assert err(dIn.value(), ref) <= TOL[odt if odt == "bf16" else dt]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("T,k,n", SHAPES + [(4096, 256, 256), (2000, 130, 96), (4096, 768, 128)])
@pytest.mark.parametrize("accumulate,bias", [(False, True), (True, True), (False, False)])
def test_linear_bwd_wgrad(dev, dt, T, k, n, accumulate, bias):
    import tensor_transformer_layer_fwd_amd as tp
    from tensor_transformer_layer_fwd_amd import _lib as L
    _say(f"wgrad dt={dt} T={T} k={k} n={n} acc={accumulate} bias={bias}")
    rng = np.random.default_rng(T + 17 * k + n)
    In, Inr = rand(rng, (T, k), 1.0, dt)
    dO, dOr = rand(rng, (T, n), 1.0, dt)
    dW = Guarded(k, n, "f32", dev)
    db = torch.full((n + 8,), float("nan"), device=dev)
    dbv = db[4:4 + n]
    prev_w = rng.standard_normal((k, n)).astype(np.float32)
    prev_b = rng.standard_normal(n).astype(np.float32)
    if accumulate:
        dW.view.copy_(torch.from_numpy(prev_w))
        dbv.copy_(torch.from_numpy(prev_b))
    wsb = L.tp_linear_bwd_wgrad_workspace_size(T, k, n, L.TP_BF16 if dt == "bf16" else L.TP_F32)
    ws = torch.full((max(wsb, 16),), 255, dtype=torch.uint8, device=dev)  # garbage on entry
    tp.tp_linear_bwd_wgrad(upload(Inr, dt, dev, pad=3), upload(dOr, dt, dev, pad=5), dW.view,
                           dbv if bias else None, accumulate=accumulate, workspace=ws)
    torch.cuda.synchronize()
    rw, rb = oracle.linear_bwd_wgrad(In, dO)
    if accumulate:
        rw = rw + prev_w
        rb = rb + prev_b
    # fp32 output: only the summation order differs from the exact result
    assert err(dW.value(), rw) <= 1e-5
    got_b = db.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(got_b[:4])) and np.all(np.isnan(got_b[4 + n:]))
    if bias:
        assert err(got_b[4:4 + n], rb) <= 1e-5
    else:  # no bias gradient requested: dbias untouched
        assert np.all(np.isnan(got_b[4:4 + n]))


@pytest.mark.parametrize("out_dt", DTS)
@pytest.mark.parametrize("p", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("T,h", [(1, 1), (7, 13), (64, 768), (33, 1028)])
@pytest.mark.parametrize("pad", [3, 8])
def test_reduce_partials(dev, out_dt, p, T, h, pad):
    """Output row stride h + pad: pad 8 keeps 16-byte aligned rows, which takes
    the eight-column path where h is a multiple of 8."""
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"reduce out={out_dt} p={p} T={T} h={h} pad={pad}")
    rng = np.random.default_rng(p * 100 + T + h)
    parts = [rng.standard_normal((T, h)).astype(np.float32) for _ in range(p)]
    bias, biasr = rand(rng, (h,), 0.5, out_dt)
    big = torch.zeros(p, T, h + 4, device=dev)
    for i in range(p):
        big[i, :, :h] = torch.from_numpy(parts[i])
    views = [big[i, :, :h] for i in range(p)]
    out = Guarded(T, h, out_dt, dev, pad=pad)
    tp.tp_reduce_partials(views, upload(biasr, out_dt, dev), out.view)
    torch.cuda.synchronize()
    ref = oracle.reduce_partials([x.astype(np.float64) for x in parts], bias)
    got = out.value()
    if out_dt == "bf16":
        assert err(got, ref) <= TOL["bf16"]
    else:
        # p fp32 additions (bias included), each with relative error <= 2^-24:
        # |got - exact| <= p * 2^-24 * (sum_i |part_i| + |bias|) elementwise
        mag = sum(np.abs(x.astype(np.float64)) for x in parts) + np.abs(bias)[None, :]
        assert np.all(np.abs(got - ref) <= p * 2.0 ** -24 * mag * 1.0001)


def test_bf16_rounding_is_rne(dev):
    """fp32 -> bf16 on the device (one partial, bf16 output) equals round to
    nearest even bit for bit: ties, denormals, huge values, infinities, NaN."""
    import tensor_transformer_layer_fwd_amd as tp
    rng = np.random.default_rng(123)
    x = (rng.standard_normal(60000) * 10.0 ** rng.integers(-40, 38, 60000)).astype(np.float32)
    ties = (f32_to_bf16_bits(rng.standard_normal(2000).astype(np.float32)).astype(np.uint32) << 16)
    ties = (ties | 0x8000).view(np.float32)  # exactly half-way between two bf16 values
    special = np.array([0.0, -0.0, 1e-45, -1e-45, 1.1754942e-38, 3.4028235e38, -3.4028235e38,
                        np.inf, -np.inf], np.float32)
    x = np.concatenate([x, ties, special])
    n = x.size
    out = torch.empty(1, n, dtype=torch.bfloat16, device=dev)
    tp.tp_reduce_partials([torch.from_numpy(x).view(1, n).to(dev)], None, out)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)[0]
    np.testing.assert_array_equal(got, f32_to_bf16_bits(x))
    nan = torch.full((1, 8), float("nan"), device=dev)
    outn = torch.empty(1, 8, dtype=torch.bfloat16, device=dev)
    tp.tp_reduce_partials([nan], None, outn)
    torch.cuda.synchronize()
    assert torch.isnan(outn.float()).all()


def test_reduce_partials_order_and_rounding(dev):
    """Sum in fp32 in shard order, bias last, one rounding: reproduce it exactly."""
    import tensor_transformer_layer_fwd_amd as tp
    rng = np.random.default_rng(77)
    T, h, p = 16, 64, 5
    parts = [(rng.standard_normal((T, h)) * 10.0 ** rng.integers(-3, 4)).astype(np.float32)
             for _ in range(p)]
    bias = rng.standard_normal(h).astype(np.float32)
    out = torch.empty(T, h, device=dev)
    tp.tp_reduce_partials([torch.from_numpy(x).to(dev) for x in parts],
                          torch.from_numpy(bias).to(dev), out)
    torch.cuda.synchronize()
    want = parts[0].copy()
    for x in parts[1:]:
        want = (want + x).astype(np.float32)
    want = (want + bias[None, :]).astype(np.float32)
    np.testing.assert_array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("in_dt,out_dt", [("f32", "bf16"), ("bf16", "bf16"), ("f32", "f32")])
@pytest.mark.parametrize("T,n", [(3, 5), (64, 1536), (17, 260)])
@pytest.mark.parametrize("pad,with_bias", [(3, True), (8, True), (8, False)])
def test_bias_act(dev, in_dt, out_dt, T, n, pad, with_bias):
    """Output row stride n + pad: pad 8 keeps 16-byte aligned rows (the
    eight-column path for fp32 or bf16 U and bf16 Y where n is a multiple of 8)."""
    import tensor_transformer_layer_fwd_amd as tp
    rng = np.random.default_rng(T * n)
    U, Ur = rand(rng, (T, n), 2.0, in_dt)
    b, br = rand(rng, (n,), 0.1, in_dt)
    if not with_bias:
        b = np.zeros_like(b)
    Y = Guarded(T, n, out_dt, dev, pad=pad)
    tp.tp_bias_act(upload(Ur, in_dt, dev), upload(br, in_dt, dev) if with_bias else None, Y.view,
                   act="gelu")
    torch.cuda.synchronize()
    ref = oracle.gelu_tanh(U + b[None, :])
    assert err(Y.value(), ref) <= (TOL["bf16"] if out_dt == "bf16" else 1e-6)


def test_gelu_extremes(dev):
    """Zero, tiny, saturated and huge pre-activations through the fused GeLU
    epilogue and the GeLU-derivative epilogue (fp32, identity weight so U = X
    exactly); a NaN input row stays NaN."""
    import tensor_transformer_layer_fwd_amd as tp
    x = np.array([[0.0, 1e-30, -1e-30, 0.5, -0.5, 3.0, -3.0, 9.5, -9.5, 40.0, -40.0, 88.0,
                   -88.0, 1e4, -1e4, 3e38, -3e38]], np.float32)
    n = x.shape[1]
    X = torch.from_numpy(x).to(dev)
    A = torch.eye(n, device=dev)
    Y, U, dU = (torch.empty(1, n, device=dev) for _ in range(3))
    tp.tp_column_linear_fwd(X, A, None, Y, U, act="gelu")
    tp.tp_linear_bwd_dgrad(torch.ones(1, n, device=dev), A, U, dU, act="gelu")
    torch.cuda.synchronize()
    xs = x[0].astype(np.float64)
    np.testing.assert_array_equal(U.cpu().numpy()[0], x[0])
    # the oracle's tanh form cancels (1 + tanh(s) = 0 in float64) for x below
    # about -8, where the true values are below 1e-30: absolute floor 1e-30
    np.testing.assert_allclose(Y.cpu().numpy()[0], oracle.gelu_tanh(xs), rtol=2e-6, atol=1e-30)
    np.testing.assert_allclose(dU.cpu().numpy()[0], oracle.gelu_tanh_grad(xs), rtol=2e-6,
                               atol=1e-30)
    xn = np.array([[1.0, np.nan, 2.0]], np.float32)
    Xn = torch.from_numpy(xn).to(dev)
    Yn, Un, dUn = (torch.empty(1, 3, device=dev) for _ in range(3))
    tp.tp_column_linear_fwd(Xn, torch.eye(3, device=dev), None, Yn, Un, act="gelu")
    tp.tp_linear_bwd_dgrad(torch.ones(1, 3, device=dev), torch.eye(3, device=dev), Un, dUn,
                           act="gelu")
    torch.cuda.synchronize()
    assert np.isnan(Yn.cpu().numpy()).all() and np.isnan(dUn.cpu().numpy()).all()


# --------------------------------------------------------------------------- #
# hand-worked example (exact)                                                  #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("dt", DTS)
def test_hand_worked_example(dev, dt, golden_dir):
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    from tp_inputs.configs import TPConfig
    from tp_inputs.generate import HostTensor
    g = json.load(open(os.path.join(golden_dir, "hand_worked_tp_mlp.json")))
    cfg = TPConfig(name="hand", index=0, dtype=dt, micro_batch=1, seq=2, h=2, p=2, shards=(0, 1),
                   mlp=True, attn=False, w_std=0.0, bias="normal")

    def ht(name):
        x = np.asarray(g[name], np.float32)
        return HostTensor(f32_to_bf16_bits(x) if dt == "bf16" else x, dt)

    inputs = {k: ht(k) for k in ("X", "A", "a", "B", "b", "dZ")}
    step = ShardStep(cfg, inputs, dev)
    step.run_eager()
    got = step.results()
    exp = {k: np.asarray(v, np.float64) for k, v in g["expected"].items()}
    cat = lambda k, ax=1: np.concatenate([got[f"{k}_0"], got[f"{k}_1"]], ax)  # noqa: E731
    np.testing.assert_array_equal(cat("U"), exp["U"])
    np.testing.assert_array_equal(cat("Y"), exp["Y"])
    np.testing.assert_array_equal(got["Zp_0"], exp["Zp_0"])
    np.testing.assert_array_equal(got["Zp_1"], exp["Zp_1"])
    np.testing.assert_array_equal(got["Z"], exp["Z"])
    np.testing.assert_array_equal(cat("dU"), exp["dU"])
    np.testing.assert_array_equal(cat("dB", 0), exp["dB"])
    np.testing.assert_array_equal(got["db"], exp["db"])
    np.testing.assert_array_equal(cat("dA"), exp["dA"])
    np.testing.assert_array_equal(np.concatenate([got["da_0"], got["da_1"]]), exp["da"])
    np.testing.assert_array_equal(got["dXp_0"], exp["dXp_0"])
    np.testing.assert_array_equal(got["dXp_1"], exp["dXp_1"])
    np.testing.assert_array_equal(got["dX"], exp["dX"])


# --------------------------------------------------------------------------- #
# workloads                                                                    #
# --------------------------------------------------------------------------- #
def _compare_all(cfg, got, ref, tol):
    worst = (0.0, None)
    for k, r in ref.items():
        assert k in got, k
        assert got[k].shape == r.shape, (k, got[k].shape, r.shape)
        e = err(got[k], r)
        if e > worst[0]:
            worst = (e, k)
        assert e <= tol, (cfg.name, k, e)
    return worst


REDUCED = [("tiny", 8, 64), ("gpt2s", 1, 680), ("attn", 1, 552), ("gpt350m", 1, 520),
           ("gpt175b", 1, 200)]


@pytest.mark.parametrize("name,mb,seq", REDUCED)
def test_workload_reduced_tokens(dev, name, mb, seq):
    """Every output in full at a token count the oracle finishes in seconds
    (ragged against the 128/256 tiles); the 175B-class shard also at h=1024."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = dataclasses.replace(get_config(name), micro_batch=mb, seq=seq)
    if name == "gpt175b":
        cfg = dataclasses.replace(cfg, h=1024)
    _say(f"workload {name} T={cfg.T} h={cfg.h}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev)
    step.run_eager()
    got = step.results()
    ref = oracle.run_config(cfg, inputs)
    worst = _compare_all(cfg, got, ref, TOL[cfg.dtype])
    _say(f"  worst rel err {worst[0]:.3e} ({worst[1]})")


FULL = ["gpt2s", "attn", "gpt350m", "gpt175b"]


@pytest.mark.parametrize("name", FULL)
def test_workload_full_size_sampled(dev, name):
    """Full-size workload, graph-replayed as the benchmark runs it; outputs
    compared on sampled token rows and shard columns."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = get_config(name)
    _say(f"full workload {name} T={cfg.T} h={cfg.h} p={cfg.p}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev)
    step.capture()
    for _ in range(2):
        step.run()
    got = step.results()
    rng = np.random.default_rng(cfg.index)
    rows = np.sort(rng.choice(cfg.T, 24, replace=False))
    rows[-1] = cfg.T - 1
    cf = np.sort(rng.choice(cfg.F, 16, replace=False)) if cfg.mlp else None
    cq = np.sort(rng.choice(cfg.Q, 16, replace=False)) if cfg.attn else None
    co = np.sort(rng.choice(cfg.O, 16, replace=False)) if cfg.attn else None
    ref = sampled.run_config_sampled(cfg, inputs, rows, cf, cq, co)
    got_s = {k: sampled.sample_device_output(k, got[k], rows, cf, cq, co) for k in ref}
    worst = _compare_all(cfg, got_s, ref, TOL[cfg.dtype])
    _say(f"  worst rel err {worst[0]:.3e} ({worst[1]})")
    for k, v in got.items():
        assert np.all(np.isfinite(v)), k


@pytest.mark.parametrize("name", ["gpt2s", "gpt350m"])
def test_fused_backward_step_matches_two_calls(dev, name):
    """The step with each layer's gradients in one tp_linear_bwd call equals the
    step with separate dgrad and wgrad calls: data gradients and forward outputs
    bitwise, weight and bias gradients within fp32 summation order (their K
    slices may differ)."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = get_config(name)
    _say(f"fused vs two-call backward {name} T={cfg.T}")
    inputs = make_inputs(cfg)
    two = ShardStep(cfg, inputs, dev, fused_bwd=False)
    two.run_eager()
    want = two.results()
    del two
    step = ShardStep(cfg, inputs, dev)
    step.run_eager()
    got = step.results()
    for key in want:
        if key[:2] in ("dA", "dB", "dW") or key[:3] in ("dOw",) or key in ("db",) or \
                key.startswith("da_"):
            assert err(got[key], want[key]) <= 1e-6, key
        else:
            np.testing.assert_array_equal(got[key], want[key], err_msg=key)


def test_determinism_and_graph_replay(dev):
    """Two eager runs are bitwise equal; graph replays (with eager work and
    synchronisations between them) equal the eager result bitwise."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = dataclasses.replace(get_config("gpt2s"), micro_batch=1, seq=1024)
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev)
    step.run_eager()
    first = step.results()
    for t in step.out.values():
        t.fill_(float("nan"))
    step.run_eager()
    second = step.results()
    for k in first:
        np.testing.assert_array_equal(first[k], second[k], err_msg=k)
    step.capture()
    for rep in range(3):
        for t in step.out.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        step.run()
        got = step.results()
        for k in first:
            np.testing.assert_array_equal(first[k], got[k], err_msg=f"replay {rep}: {k}")
        # eager work between replays
        torch.randn(1000, device=dev).sum().item()


# --------------------------------------------------------------------------- #
# every pipelined tile configuration, in every operand layout                  #
# --------------------------------------------------------------------------- #
_TILE_MN = {10: (256, 256), 11: (256, 128), 12: (128, 256), 13: (128, 128), 14: (256, 192),
            15: (128, 192)}


@pytest.mark.parametrize("tile", sorted(_TILE_MN))
@pytest.mark.parametrize("op", ["fwd_gelu", "row_partial", "dgrad_gelu", "dgrad_f32", "wgrad",
                                "wgrad_split", "wgrad_split_acc"])
@pytest.mark.parametrize("kt", [2, 18])
def test_pipelined_tiles(dev, tile, op, kt):
    """Each pipelined tile forced on a grid of 8 tiles (XCD remap path), with
    kt 32-wide K-tiles per block: 2 runs only the guarded tail, 18 the
    steady-state loop and a 6-tile tail. The split cases use 3 K slices; the
    weight gradients carry the bias column sums, once accumulating into
    existing dW and dbias."""
    import tensor_transformer_layer_fwd_amd as tp
    from tensor_transformer_layer_fwd_amd import _lib as L
    split = op.startswith("wgrad_split")
    bm, bn = _TILE_MN[tile]
    M, N, K = 4 * bm, 2 * bn, 32 * kt * (3 if split else 1)
    tp.tp_set_gemm_override(tile, 3 if split else 1)
    try:
        plan = L.tp_gemm_plan(M, N, K, op.startswith("wgrad"))
    finally:
        tp.tp_set_gemm_override(0)
    assert plan[0] == tile and (plan[1] == 3) == split, plan
    _say(f"pipelined tile={tile} op={op} M={M} N={N} K={K}")
    tp.tp_set_gemm_override(tile, 3 if split else 1)
    try:
        _run_tile_op(dev, tile, op, M, N, K)
    finally:
        tp.tp_set_gemm_override(0)


def _run_tile_op(dev, tile, op, M, N, K):
    import tensor_transformer_layer_fwd_amd as tp
    from tensor_transformer_layer_fwd_amd import _lib as L
    rng = np.random.default_rng(tile * 100 + len(op))
    dt = "bf16"
    if op in ("fwd_gelu", "row_partial"):
        X, Xr = rand(rng, (M, K), 1.0, dt)
        W, Wr = rand(rng, (K, N), 0.05, dt)
        if op == "fwd_gelu":
            b, br = rand(rng, (N,), 0.1, dt)
            Y, U = torch.empty(M, N, dtype=torch.bfloat16, device=dev), \
                torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            tp.tp_column_linear_fwd(upload(Xr, dt, dev), upload(Wr, dt, dev), upload(br, dt, dev),
                                    Y, U, act="gelu")
            torch.cuda.synchronize()
            U_ref, Y_ref = oracle.column_linear_fwd(X, W, b, "gelu")
            assert err(Y.float().cpu().numpy(), Y_ref) <= TOL[dt]
            assert err(U.float().cpu().numpy(), U_ref) <= TOL[dt]
        else:
            Z = torch.empty(M, N, device=dev)
            tp.tp_row_linear_fwd_partial(upload(Xr, dt, dev), upload(Wr, dt, dev), Z)
            torch.cuda.synchronize()
            assert err(Z.cpu().numpy(), oracle.row_linear_fwd_partial(X, W)) <= 1e-5
    elif op.startswith("dgrad"):
        dO, dOr = rand(rng, (M, K), 1.0, dt)
        W, Wr = rand(rng, (N, K), 0.05, dt)
        if op == "dgrad_gelu":
            U, Ur = rand(rng, (M, N), 1.5, dt)
            dI = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            tp.tp_linear_bwd_dgrad(upload(dOr, dt, dev), upload(Wr, dt, dev), upload(Ur, dt, dev),
                                   dI, act="gelu")
            torch.cuda.synchronize()
            assert err(dI.float().cpu().numpy(), oracle.linear_bwd_dgrad(dO, W, U, "gelu")) <= TOL[dt]
        else:
            dI = torch.empty(M, N, device=dev)
            tp.tp_linear_bwd_dgrad(upload(dOr, dt, dev), upload(Wr, dt, dev), None, dI)
            torch.cuda.synchronize()
            assert err(dI.cpu().numpy(), oracle.linear_bwd_dgrad(dO, W)) <= 1e-5
    else:
        In, Inr = rand(rng, (K, M), 1.0, dt)
        dO, dOr = rand(rng, (K, N), 1.0, dt)
        acc = op.endswith("_acc")
        prev_w = rng.standard_normal((M, N)).astype(np.float32)
        prev_b = rng.standard_normal(N).astype(np.float32)
        dW = torch.from_numpy(prev_w).to(dev) if acc else torch.empty(M, N, device=dev)
        db = torch.from_numpy(prev_b).to(dev) if acc else torch.empty(N, device=dev)
        ws = torch.full((max(16, L.tp_linear_bwd_wgrad_workspace_size(K, M, N, L.TP_BF16)),), 255,
                        dtype=torch.uint8, device=dev)  # garbage on entry
        tp.tp_linear_bwd_wgrad(upload(Inr, dt, dev), upload(dOr, dt, dev), dW, db, accumulate=acc,
                               workspace=ws)
        torch.cuda.synchronize()
        rw, rb = oracle.linear_bwd_wgrad(In, dO)
        if acc:
            rw, rb = rw + prev_w, rb + prev_b
        assert err(dW.cpu().numpy(), rw) <= 1e-5
        assert err(db.cpu().numpy(), rb) <= 1e-5


# --------------------------------------------------------------------------- #
# the backward of one linear layer in one call (tp_linear_bwd)                 #
# --------------------------------------------------------------------------- #
# (data-gradient tile id, BM, BN): the tiles on which a layer's data and weight
# gradients share one launch (beside 128x192 the weight gradient takes 128x128);
# k is a multiple of BM and BN, n of BN and 128
_PAIR_TILES = [(15, 128, 192), (13, 128, 128), (14, 256, 192)]


@pytest.mark.parametrize("tile,bm,bn", _PAIR_TILES)
@pytest.mark.parametrize("split", [1, 2, 4])
@pytest.mark.parametrize("kind", ["gelu_bias", "f32_out", "bf16_out_acc"])
def test_linear_bwd_paired(dev, tile, bm, bn, split, kind):
    """Both gradients of a layer in one launch (tile and K slices forced), against
    the oracle; dIn bitwise equal to tp_linear_bwd_dgrad on the same tile."""
    import tensor_transformer_layer_fwd_amd as tp
    from tensor_transformer_layer_fwd_amd import _lib as L
    lcm = bm * bn // np.gcd(bm, bn)
    T, k, n = 2 * bm * split if bm * split >= 256 else 512, lcm, 2 * bn
    _say(f"paired bwd tile={tile} split={split} kind={kind} T={T} k={k} n={n}")
    rng = np.random.default_rng(tile * 10 + split + len(kind))
    dt = "bf16"
    dO, dOr = rand(rng, (T, n), 1.0, dt)
    W, Wr = rand(rng, (k, n), 0.05, dt)
    In, Inr = rand(rng, (T, k), 1.0, dt)
    act = "gelu" if kind == "gelu_bias" else "none"
    out_dt = "f32" if kind == "f32_out" else "bf16"
    U, Ur = rand(rng, (T, k), 1.5, dt)
    acc = kind.endswith("_acc")
    prev_w = rng.standard_normal((k, n)).astype(np.float32)
    prev_b = rng.standard_normal(n).astype(np.float32)
    dI = Guarded(T, k, out_dt, dev, pad=8)
    dW = torch.from_numpy(prev_w).to(dev) if acc else torch.empty(k, n, device=dev)
    db = None if kind == "f32_out" else (torch.from_numpy(prev_b).to(dev) if acc
                                          else torch.empty(n, device=dev))
    tp.tp_set_gemm_override(tile, split)
    try:
        ws = torch.full((max(16, L.tp_linear_bwd_workspace_size(T, k, n, L.TP_BF16)),), 255,
                        dtype=torch.uint8, device=dev)  # garbage on entry
        dOd, Wd, Ind = upload(dOr, dt, dev), upload(Wr, dt, dev), upload(Inr, dt, dev)
        Ud = upload(Ur, dt, dev) if act == "gelu" else None
        tp.tp_linear_bwd(dOd, Wd, Ud, Ind, dI.view, dW, db, act=act, accumulate=acc,
                         workspace=ws)
        dI_alone = torch.empty_like(dI.view)
        tp.tp_linear_bwd_dgrad(dOd, Wd, Ud, dI_alone, act=act)
        torch.cuda.synchronize()
    finally:
        tp.tp_set_gemm_override(0)
    got = dI.value()
    ref = oracle.linear_bwd_dgrad(dO, W, U if act == "gelu" else None, act)
    assert err(got, ref) <= (TOL["bf16"] if out_dt == "bf16" else 1e-5)
    np.testing.assert_array_equal(got, dI_alone.float().cpu().numpy().astype(np.float64))
    rw, rb = oracle.linear_bwd_wgrad(In, dO)
    if acc:
        rw, rb = rw + prev_w, rb + prev_b
    assert err(dW.cpu().numpy(), rw) <= 1e-5
    if db is not None:
        assert err(db.cpu().numpy(), rb) <= 1e-5


@pytest.mark.parametrize("dt,T,k,n,ws_kind", [
    ("f32", 300, 129, 200, "full"),    # fp32 operands: the two calls
    ("bf16", 130, 520, 264, "full"),   # ragged against every tile
    ("bf16", 4096, 1536, 768, "wgrad_only"),  # pairable, workspace sized for the wgrad alone
    ("bf16", 4096, 1536, 768, "full"),  # the GPT-2-small fc2 layer, paired
    ("bf16", 4096, 768, 1536, "full"),  # the GPT-2-small fc1 layer, paired
])
def test_linear_bwd_shapes(dev, dt, T, k, n, ws_kind):
    """tp_linear_bwd on the planner's own choice, paired or as two calls, against
    the oracle (sampled rows for the large shapes)."""
    import tensor_transformer_layer_fwd_amd as tp
    from tensor_transformer_layer_fwd_amd import _lib as L
    _say(f"linear bwd dt={dt} T={T} k={k} n={n} ws={ws_kind}")
    rng = np.random.default_rng(T + k + n)
    dO, dOr = rand(rng, (T, n), 1.0, dt)
    W, Wr = rand(rng, (k, n), 0.05, dt)
    In, Inr = rand(rng, (T, k), 1.0, dt)
    U, Ur = rand(rng, (T, k), 1.5, dt)
    tdt = L.TP_BF16 if dt == "bf16" else L.TP_F32
    nbytes = (L.tp_linear_bwd_workspace_size(T, k, n, tdt) if ws_kind == "full"
              else L.tp_linear_bwd_wgrad_workspace_size(T, k, n, tdt))
    ws = torch.full((max(16, nbytes),), 255, dtype=torch.uint8, device=dev)
    dI = Guarded(T, k, dt, dev, pad=8)
    dW = torch.empty(k, n, device=dev)
    db = torch.empty(n, device=dev)
    tp.tp_linear_bwd(upload(dOr, dt, dev), upload(Wr, dt, dev), upload(Ur, dt, dev),
                     upload(Inr, dt, dev), dI.view, dW, db, act="gelu", workspace=ws)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 512 else np.sort(rng.choice(T, 64, replace=False))
    ref = oracle.linear_bwd_dgrad(dO[rows], W, U[rows], "gelu")
    assert err(dI.value()[rows], ref) <= TOL[dt]
    rw, rb = oracle.linear_bwd_wgrad(In, dO)
    assert err(dW.cpu().numpy(), rw) <= 1e-5
    assert err(db.cpu().numpy(), rb) <= 1e-5


@pytest.mark.parametrize("T,h,F,acc,bias,tile", [
    (4096, 768, 1536, False, True, 0),    # the GPT-2-small shard: both layers paired, fc2's
                                          # fix-up and fc1's bias gradient riding in fc1's launch
    (1024, 768, 1536, True, True, 0),     # accumulating into existing gradients
    (6144, 1024, 1024, False, False, 0),  # the ~350M shard's MLP, no bias
    (2048, 768, 1536, False, True, 14),   # 256x192 tiles (8 waves), column partials of 256 rows
    (2048, 768, 1536, True, True, 14),
    (300, 129, 200, False, True, 0),      # ragged: the two layers one after the other
])
def test_mlp_bwd(dev, T, h, F, acc, bias, tile):
    """The backward of one shard's MLP block against the oracle's chain
    (sampled token rows of the data gradients on the large shapes); tile != 0
    forces that pipelined tile on every product that fits it."""
    import tensor_transformer_layer_fwd_amd as tp
    from tensor_transformer_layer_fwd_amd import _lib as L
    _say(f"mlp bwd T={T} h={h} F={F} acc={acc} bias={bias} tile={tile}")
    rng = np.random.default_rng(T + h + F + acc)
    dt = "bf16"
    dZ, dZr = rand(rng, (T, h), 1.0, dt)
    X, Xr = rand(rng, (T, h), 1.0, dt)
    A, Ar = rand(rng, (h, F), 0.02, dt)
    B, Br = rand(rng, (F, h), 0.02, dt)
    U, Ur = rand(rng, (T, F), 1.0, dt)
    Y, Yr = rand(rng, (T, F), 1.0, dt)
    prev = {k: rng.standard_normal(s).astype(np.float32)
            for k, s in (("dB", (F, h)), ("dA", (h, F)), ("db", (h,)), ("da", (F,)))}
    out = {}
    for k, shp in (("dB", (F, h)), ("dA", (h, F)), ("db", (h,)), ("da", (F,))):
        out[k] = torch.from_numpy(prev[k]).to(dev) if acc else torch.empty(*shp, device=dev)
    dU = torch.empty(T, F, dtype=torch.bfloat16, device=dev)
    dXp = torch.empty(T, h, device=dev)
    tp.tp_set_gemm_override(tile, 1)
    try:
        ws = torch.full((max(16, L.tp_mlp_bwd_workspace_size(T, h, F, L.TP_BF16)),), 255,
                        dtype=torch.uint8, device=dev)
        tp.tp_mlp_bwd(upload(dZr, dt, dev), upload(Xr, dt, dev), upload(Ar, dt, dev),
                      upload(Br, dt, dev), upload(Ur, dt, dev), upload(Yr, dt, dev), dU,
                      out["dB"], out["db"] if bias else None, dXp, out["dA"],
                      out["da"] if bias else None, accumulate=acc, workspace=ws)
        torch.cuda.synchronize()
    finally:
        tp.tp_set_gemm_override(0)
    dU_ref = oracle.linear_bwd_dgrad(dZ, B, U, "gelu")
    dB_ref, db_ref = oracle.linear_bwd_wgrad(Y, dZ)
    dA_ref, da_ref = oracle.linear_bwd_wgrad(X, dU_ref)
    rows = np.arange(T) if T <= 512 else np.sort(rng.choice(T, 64, replace=False))
    dXp_ref = oracle.linear_bwd_dgrad(dU_ref[rows], A)
    assert err(dU.float().cpu().numpy()[rows], dU_ref[rows]) <= TOL[dt]
    assert err(dXp.cpu().numpy()[rows], dXp_ref) <= TOL[dt]
    got = {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}
    ref = {"dB": dB_ref, "dA": dA_ref, "db": db_ref, "da": da_ref}
    for k in ("dB", "dA") + (("db", "da") if bias else ()):
        want = ref[k] + prev[k] if acc else ref[k]
        # dB reads only stored inputs; dA and da read the device's bf16 dU
        assert err(got[k], want) <= (1e-5 if k in ("dB", "db") else TOL[dt]), k


# --------------------------------------------------------------------------- #
# attention core of one shard (forward)                                        #
# --------------------------------------------------------------------------- #
@pytest.mark.parametrize("batch,seq,heads,causal", [
    (1, 1, 2, True), (1, 64, 1, True), (2, 100, 3, True), (2, 100, 3, False),
    (3, 257, 2, True), (1, 384, 1, False),
    (8, 512, 8, True),    # the attention-projection workload's shard: 8 x 512 tokens, 8 heads
    (6, 1024, 4, True),   # the ~350M-layer workload's shard: 6 x 1024 tokens, 4 heads
    (2, 1024, 32, True),  # 512 query blocks: one key group per block
    (4, 200, 80, False),  # 640 query blocks, ragged
])
def test_attention_fwd(dev, batch, seq, heads, causal):
    import tensor_transformer_layer_fwd_amd as tp
    from oracle.attention import attention_core_fwd
    _say(f"attention batch={batch} seq={seq} heads={heads} causal={causal}")
    rng = np.random.default_rng(batch * 1000 + seq + heads)
    T, hd = batch * seq, heads * 64
    QKV, QKVr = rand(rng, (T, 3 * hd), 1.0, "bf16")
    C = Guarded(T, hd, "bf16", dev, pad=4)
    lse = torch.full((batch * heads * seq + 8,), float("nan"), device=dev)
    tp.tp_attention_fwd(upload(QKVr, "bf16", dev, pad=8), C.view, lse[4:4 + batch * heads * seq],
                        batch, seq, heads, causal=causal)
    torch.cuda.synchronize()
    C_ref, lse_ref = attention_core_fwd(QKV, batch, seq, heads, 64, causal)
    assert err(C.value(), C_ref) <= TOL["bf16"]
    got = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(got[:4])) and np.all(np.isnan(got[4 + batch * heads * seq:]))
    np.testing.assert_allclose(got[4:4 + batch * heads * seq], lse_ref.reshape(-1), rtol=0,
                               atol=1e-4)


def test_attention_fwd_deterministic_and_lse_optional(dev):
    import tensor_transformer_layer_fwd_amd as tp
    rng = np.random.default_rng(77)
    batch, seq, heads = 2, 320, 2
    _, QKVr = rand(rng, (batch * seq, 3 * heads * 64), 1.0, "bf16")
    x = upload(QKVr, "bf16", dev)
    outs = []
    for with_lse in (True, False, True):
        C = torch.empty(batch * seq, heads * 64, dtype=torch.bfloat16, device=dev)
        lse = torch.empty(batch * heads * seq, device=dev) if with_lse else None
        tp.tp_attention_fwd(x, C, lse, batch, seq, heads)
        outs.append(C.cpu())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def _attn_bwd_case(dev, batch, seq, heads, causal, seed, from_oracle=False):
    import tensor_transformer_layer_fwd_amd as tp
    from oracle.attention import attention_core_bwd, attention_core_fwd
    rng = np.random.default_rng(seed)
    T, hd = batch * seq, heads * 64
    QKV, QKVr = rand(rng, (T, 3 * hd), 1.0, "bf16")
    dC, dCr = rand(rng, (T, hd), 1.0, "bf16")
    x = upload(QKVr, "bf16", dev, pad=8)
    n = batch * heads * seq
    if from_oracle:
        # the backward alone, on the oracle's forward (C rounded to bf16)
        C_ref, lse_ref = attention_core_fwd(QKV, batch, seq, heads, 64, causal)
        C = upload(f32_to_bf16_bits(C_ref.astype(np.float32)), "bf16", dev, pad=8)
        lse = torch.from_numpy(lse_ref.reshape(-1).astype(np.float32)).to(dev)
    else:
        Cg = Guarded(T, hd, "bf16", dev, pad=8)
        C = Cg.view
        lse = torch.empty(n, device=dev)
        tp.tp_attention_fwd(x, C, lse, batch, seq, heads, causal=causal)
    delta = torch.full((n + 8,), float("nan"), device=dev)
    dQKV = Guarded(T, 3 * hd, "bf16", dev, pad=4)
    tp.tp_attention_bwd(x, C, upload(dCr, "bf16", dev, pad=8), lse, delta[4:4 + n], dQKV.view,
                        batch, seq, heads, causal=causal)
    torch.cuda.synchronize()
    got = dQKV.value()
    d = delta.cpu().numpy()
    assert np.all(np.isnan(d[:4])) and np.all(np.isnan(d[4 + n:])), "delta written out of range"
    ref = attention_core_bwd(QKV, dC, batch, seq, heads, 64, causal)
    errs = [err(got[:, i * hd:(i + 1) * hd], ref[:, i * hd:(i + 1) * hd]) for i in range(3)]
    _say(f"  dQ/dK/dV rel err {errs[0]:.2e} {errs[1]:.2e} {errs[2]:.2e}")
    return errs


@pytest.mark.gpu
@pytest.mark.parametrize("batch,seq,heads,causal", [
    (1, 1, 2, True), (1, 64, 1, True), (2, 100, 3, True), (2, 100, 3, False),
    (3, 257, 2, True), (1, 384, 1, False), (1, 130, 1, True),
    (8, 512, 8, True),    # the attention-projection workload's shard: 8 x 512 tokens, 8 heads
    (6, 1024, 4, True),   # the ~350M-layer workload's shard: 6 x 1024 tokens, 4 heads
    (2, 1024, 32, True),  # 512 key and query blocks: one group per block
    (4, 200, 80, False),  # 640 blocks, ragged
])
def test_attention_bwd(dev, batch, seq, heads, causal):
    """dQKV of the GPU forward -> backward chain against the oracle's gradient
    of the same attention core (one third at a time)."""
    _say(f"attention bwd batch={batch} seq={seq} heads={heads} causal={causal}")
    errs = _attn_bwd_case(dev, batch, seq, heads, causal, batch * 1000 + seq + heads)
    assert max(errs) <= TOL["bf16"], errs


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [True, False])
def test_attention_bwd_on_oracle_forward(dev, causal):
    """The backward fed the oracle's C and lse: its own error, apart from the forward's."""
    _say(f"attention bwd on the oracle's forward causal={causal}")
    errs = _attn_bwd_case(dev, 2, 200, 2, causal, 31, from_oracle=True)
    assert max(errs) <= TOL["bf16"], errs


@pytest.mark.gpu
def test_attention_bwd_deterministic(dev):
    import tensor_transformer_layer_fwd_amd as tp
    rng = np.random.default_rng(78)
    batch, seq, heads = 2, 320, 2
    T, hd = batch * seq, heads * 64
    x = upload(rand(rng, (T, 3 * hd), 1.0, "bf16")[1], "bf16", dev)
    dC = upload(rand(rng, (T, hd), 1.0, "bf16")[1], "bf16", dev)
    C = torch.empty(T, hd, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(batch * heads * seq, device=dev)
    tp.tp_attention_fwd(x, C, lse, batch, seq, heads)
    outs = []
    for _ in range(3):
        d = torch.empty(T, 3 * hd, dtype=torch.bfloat16, device=dev)
        tp.tp_attention_bwd(x, C, dC, lse, torch.empty_like(lse), d, batch, seq, heads)
        outs.append(d.cpu())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("mode", ["step", "pair", "products"])
@pytest.mark.parametrize("name,mb,seq", [("tiny", 8, 64), ("gpt2s", 1, 680), ("gpt2s", 1, 1024),
                                         ("gpt350m", 1, 520)])
def test_workload_recompute(dev, name, mb, seq, mode):
    """The step with activation recompute: every output the oracle defines
    except the Y_i it no longer keeps, and the recomputed Y of the last shard
    (left in the transient buffer) against the oracle's Y. mode "step": the
    fused forward and backward calls where the shapes take them (the backward
    rebuilds every Y_i in fc2's data-gradient epilogue); "pair": the paired
    backward, Y_i rebuilt by an elementwise pass where fc2 pairs; "products":
    one call per product, Y_i rebuilt in the fc2 dgrad epilogue."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = dataclasses.replace(get_config(name), micro_batch=mb, seq=seq)
    _say(f"workload {name} with recompute T={cfg.T} mode={mode}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev, recompute=True, fused_bwd=mode != "products",
                     step_call=mode == "step")
    aligned = name == "gpt2s" and seq == 1024
    # the aligned GPT-2-small shard runs the fused calls; with them off it
    # pairs fc2's gradients, and Y_i is rebuilt by a pass
    assert step.step_call == (mode == "step" and aligned)
    assert step.rebuild_y == (mode == "pair" and aligned)
    step.run_eager()
    got = step.results()
    ref = oracle.run_config(cfg, inputs)
    assert not any(k.startswith("Y_") for k in got)
    last = cfg.shards[-1]
    y_ref = ref[f"Y_{last}"]
    ref = {k: v for k, v in ref.items() if not k.startswith("Y_")}
    worst = _compare_all(cfg, got, ref, TOL[cfg.dtype])
    e = err(got["Yt"], y_ref)
    _say(f"  worst rel err {worst[0]:.3e} ({worst[1]}); recomputed Y {e:.3e}")
    assert e <= TOL[cfg.dtype]


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("T,k,n", [(300, 129, 200), (512, 256, 384), (4096, 1536, 768)])
def test_linear_bwd_dgrad_recompute(dev, dt, T, k, n):
    """dU equals tp_linear_bwd_dgrad's bitwise; Y = GeLU(U) against the oracle's
    GeLU of the same stored U; guards around both outputs."""
    import tensor_transformer_layer_fwd_amd as tp
    rng = np.random.default_rng(T + k + n)
    dZ, dZr = rand(rng, (T, n), 1.0, dt)
    B, Br = rand(rng, (k, n), 0.05, dt)
    U, Ur = rand(rng, (T, k), 2.0, dt)
    dZd, Bd, Ud = upload(dZr, dt, dev, pad=8), upload(Br, dt, dev), upload(Ur, dt, dev, pad=16)
    dU = Guarded(T, k, dt, dev, pad=8)
    Y = Guarded(T, k, dt, dev, pad=24)
    tp.tp_linear_bwd_dgrad_recompute(dZd, Bd, Ud, dU.view, Y.view)
    dU2 = torch.empty(T, k, dtype=dU.tdt, device=dev)
    tp.tp_linear_bwd_dgrad(dZd, Bd, Ud, dU2, act="gelu")
    torch.cuda.synchronize()
    assert torch.equal(dU.view, dU2)
    assert err(dU.value(), oracle.linear_bwd_dgrad(dZ, B, U, "gelu")) <= TOL[dt]
    assert err(Y.value(), oracle.gelu_tanh(U)) <= TOL[dt]
