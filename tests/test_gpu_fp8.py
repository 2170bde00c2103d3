"""GPU parity of the FP8 variant (quantiser and the four shard GEMMs) against
the float64 FP8 oracle (oracle/fp8.py).

The quantiser's codes and 1/s factors must equal the oracle's bit for bit
(the decision is taken in fp32 on both sides). Each GEMM then runs on the
device's codes and the oracle's GEMM on its own codes; as the codes are equal,
the results differ only by the matrix cores' summation or by the bf16
rounding of the output (5e-3). The FP8 instruction sums its 64 products with
less than fp32 precision (the ISA does not specify it): the relative error of
fp32 outputs measured 1.2e-5 (an E5M2 operand) to 1.5e-5 (E4M3 x E4M3) at
every K from 256 to 4096, i.e. about 2^-16 per 64-product block, not growing
with K. fp32 outputs of FP8 products are therefore held to 1e-4; a wrong code,
scale or K-tile moves the result by 1e-2 or more.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F
from tp_inputs import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

TOL = {"bf16": 5e-3, "f32": 1e-4}
FMT = {"e4m3": F.E4M3, "e5m2": F.E5M2}


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a ROCm GPU")
    import tensor_transformer_layer_fwd_amd as tp  # noqa: F401  (fails loudly if not built)
    return torch.device("cuda:0")


def rand_bf16(rng, shape, std):
    bits = f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))
    return bf16_bits_to_f32(bits).astype(np.float64), bits


def to_dev_bf16(bits, dev, pad=0):
    r, c = bits.shape
    buf = torch.zeros(r, c + pad, dtype=torch.bfloat16, device=dev)
    buf[:, :c] = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    return buf[:, :c]


class Codes:
    """A uint8 code buffer (row stride cols + pad) inside guard bytes."""

    def __init__(self, rows, cols, dev, pad=0):
        self.buf = torch.full((rows + 2, cols + pad), 0xAB, dtype=torch.uint8, device=dev)
        self.rows, self.cols = rows, cols
        self.view = self.buf[1:1 + rows, :cols]

    def value(self):
        b = self.buf.cpu().numpy()
        mask = np.ones(b.shape, bool)
        mask[1:1 + self.rows, :self.cols] = False
        assert np.all(b[mask] == 0xAB), "the quantiser wrote outside its output"
        return b[1:1 + self.rows, :self.cols]


def quantize_dev(tp, X, fmt, transpose, dev, pad=0):
    rows, cols = X.shape
    Q = Codes(cols if transpose else rows, rows if transpose else cols, dev, pad)
    si = torch.full((1,), float("nan"), device=dev)
    ws = torch.empty(tp.tp_fp8_quantize_workspace_size(rows, cols), dtype=torch.uint8, device=dev)
    tp.tp_fp8_quantize(X, Q.view, si, ws, fmt=fmt, transpose=transpose)
    return Q, si


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols,transpose,pad", [
    (1, 1, False, 0), (37, 53, False, 3), (37, 53, True, 5), (256, 384, False, 0),
    (256, 384, True, 0), (300, 1000, True, 16), (4096, 768, False, 0), (768, 4096, True, 0),
])
def test_quantize_bit_exact(dev, dt, fmt, rows, cols, transpose, pad):
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"fp8 quantize {dt} {fmt} {rows}x{cols} transpose={transpose}")
    rng = np.random.default_rng(rows * 7 + cols)
    if dt == "bf16":
        Xf, bits = rand_bf16(rng, (rows, cols), 2.5)
        X = to_dev_bf16(bits, dev, pad=8)
    else:
        Xf = (rng.standard_normal((rows, cols)) * 2.5).astype(np.float32).astype(np.float64)
        X = torch.from_numpy(Xf.astype(np.float32)).to(dev)
    Xf[rows // 2, cols // 3] = -np.max(np.abs(Xf)) * 3   # a distinct negative amax
    X[rows // 2, cols // 3] = float(Xf[rows // 2, cols // 3])
    Xf[rows // 2, cols // 3] = X[rows // 2, cols // 3].double().item()
    Q, si = quantize_dev(tp, X, fmt, transpose, dev, pad)
    torch.cuda.synchronize()
    q_ref, _, sinv_ref = F.quantize(Xf, FMT[fmt], transpose)
    got = Q.value()
    if not np.array_equal(got, q_ref):
        bad = np.argwhere(got != q_ref)
        i = tuple(bad[0])
        raise AssertionError(f"{len(bad)} codes differ, first at {i}: {got[i]:#x} vs {q_ref[i]:#x}")
    assert si.item() == float(sinv_ref)


def test_quantize_zeros_and_powers_of_two(dev):
    import tensor_transformer_layer_fwd_amd as tp
    X = torch.zeros(128, 256, dtype=torch.bfloat16, device=dev)
    Q, si = quantize_dev(tp, X, "e4m3", False, dev)
    torch.cuda.synchronize()
    assert si.item() == 1.0 and not Q.value().any()
    # every E4M3 value times a power of two: codes are the values' own
    codes = np.arange(256, dtype=np.uint8)
    vals = F.fp8_decode(codes, F.E4M3)
    ok = np.isfinite(vals)
    v = np.tile(vals[ok], 4)[:512].reshape(2, 256) * 2.0 ** -3
    Xd = torch.from_numpy(v.astype(np.float32)).to(dev)
    Q, si = quantize_dev(tp, Xd, "e4m3", False, dev)
    torch.cuda.synchronize()
    q_ref, _, sinv = F.quantize(v, F.E4M3)
    assert np.array_equal(Q.value(), q_ref) and si.item() == float(sinv) == 2.0 ** -3


def _quant_both(tp, Xf, bits, fmt, transpose, dev):
    X = to_dev_bf16(bits, dev)
    Q, si = quantize_dev(tp, X, fmt, transpose, dev)
    q_ref, _, sinv = F.quantize(Xf, FMT[fmt], transpose)
    return Q, si, q_ref, sinv


def _err(got, ref):
    return oracle.rel_fro(got, ref)


SHAPES = [(256, 384, 512), (512, 768, 1536), (4096, 1536, 768)]


@pytest.mark.parametrize("T,h,n", SHAPES)
def test_fp8_column_linear_fwd(dev, T, h, n):
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"fp8 column fwd T={T} h={h} n={n}")
    rng = np.random.default_rng(T + h + n)
    Xf, Xb = rand_bf16(rng, (T, h), 1.0)
    Af, Ab = rand_bf16(rng, (h, n), 0.02)
    af, ab = rand_bf16(rng, (1, n), 0.01)
    Xq, xsi, qx, sx = _quant_both(tp, Xf, Xb, "e4m3", False, dev)
    Aq, asi, qa, sa = _quant_both(tp, Af, Ab, "e4m3", True, dev)
    Y = torch.full((T, n), float("nan"), dtype=torch.bfloat16, device=dev)
    U = torch.full((T, n), float("nan"), dtype=torch.bfloat16, device=dev)
    tp.tp_fp8_column_linear_fwd(Xq.view, Aq.view, xsi, asi, to_dev_bf16(ab, dev)[0], Y, U)
    torch.cuda.synchronize()
    assert np.array_equal(Xq.value(), qx) and np.array_equal(Aq.value(), qa)
    Y_ref, U_ref = F.fp8_linear(qx, qa, 0, 0, sx, sa, bias=af[0], act="gelu")
    eu, ey = _err(U.double().cpu().numpy(), U_ref), _err(Y.double().cpu().numpy(), Y_ref)
    _say(f"  U {eu:.2e} Y {ey:.2e}")
    assert eu <= TOL["bf16"] and ey <= TOL["bf16"]


@pytest.mark.parametrize("T,k,h", SHAPES)
def test_fp8_row_linear_fwd_partial(dev, T, k, h):
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"fp8 row fwd T={T} k={k} h={h}")
    rng = np.random.default_rng(T * 3 + k + h)
    Yf, Yb = rand_bf16(rng, (T, k), 1.0)
    Bf, Bb = rand_bf16(rng, (k, h), 0.02)
    Yq, ysi, qy, sy = _quant_both(tp, Yf, Yb, "e4m3", False, dev)
    Bq, bsi, qb, sb = _quant_both(tp, Bf, Bb, "e4m3", True, dev)
    Zp = torch.full((T, h), float("nan"), device=dev)
    tp.tp_fp8_row_linear_fwd_partial(Yq.view, Bq.view, ysi, bsi, Zp)
    torch.cuda.synchronize()
    assert np.array_equal(Yq.value(), qy) and np.array_equal(Bq.value(), qb)
    e = _err(Zp.double().cpu().numpy(), F.fp8_linear(qy, qb, 0, 0, sy, sb))
    _say(f"  Zp {e:.2e}")
    assert e <= TOL["f32"]


@pytest.mark.parametrize("fmt", ["e5m2", "e4m3"])
@pytest.mark.parametrize("act", ["gelu", "none"])
@pytest.mark.parametrize("T,k,n", SHAPES)
def test_fp8_linear_bwd_dgrad(dev, fmt, act, T, k, n):
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"fp8 dgrad {fmt} {act} T={T} k={k} n={n}")
    rng = np.random.default_rng(T * 5 + k + n)
    dZf, dZb = rand_bf16(rng, (T, n), 1.0)
    Wf, Wb = rand_bf16(rng, (k, n), 0.02)
    Uf, Ub = rand_bf16(rng, (T, k), 1.5)
    dq, dsi, qd, sd = _quant_both(tp, dZf, dZb, fmt, False, dev)
    Wq, wsi, qw, sw = _quant_both(tp, Wf, Wb, "e4m3", False, dev)
    out_dt = torch.bfloat16 if act == "gelu" else torch.float32
    dIn = torch.full((T, k), float("nan"), dtype=out_dt, device=dev)
    tp.tp_fp8_linear_bwd_dgrad(dq.view, Wq.view, dsi, wsi, dIn,
                               U=to_dev_bf16(Ub, dev) if act == "gelu" else None, act=act,
                               dout_fmt=fmt)
    torch.cuda.synchronize()
    assert np.array_equal(dq.value(), qd) and np.array_equal(Wq.value(), qw)
    ref = F.fp8_linear(qd, qw, FMT[fmt], 0, sd, sw, act="dgelu" if act == "gelu" else "none",
                       U=Uf)
    e = _err(dIn.double().cpu().numpy(), ref)
    _say(f"  dIn {e:.2e}")
    assert e <= TOL["bf16" if act == "gelu" else "f32"]


@pytest.mark.parametrize("fmt", ["e5m2", "e4m3"])
@pytest.mark.parametrize("T,k,n,bias", [(512, 256, 384, True), (4096, 1536, 768, True),
                                        (4096, 768, 1536, False), (1024, 1024, 1024, True)])
def test_fp8_linear_bwd_wgrad(dev, fmt, T, k, n, bias):
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"fp8 wgrad {fmt} T={T} k={k} n={n} bias={bias}")
    rng = np.random.default_rng(T * 11 + k + n)
    Inf, Inb = rand_bf16(rng, (T, k), 1.0)
    dOf, dOb = rand_bf16(rng, (T, n), 1.0)
    Iq, isi, qi, si_ = _quant_both(tp, Inf, Inb, "e4m3", True, dev)
    dO = to_dev_bf16(dOb, dev)
    Q, dsi = quantize_dev(tp, dO, fmt, True, dev)
    qd, _, sd = F.quantize(dOf, FMT[fmt], True)
    dW = torch.full((k, n), float("nan"), device=dev)
    db = torch.full((n,), float("nan"), device=dev) if bias else None
    ws = torch.empty(max(16, tp.tp_fp8_linear_bwd_wgrad_workspace_size(T, k, n)),
                     dtype=torch.uint8, device=dev)
    tp.tp_fp8_linear_bwd_wgrad(Iq.view, Q.view, isi, dsi, dW, dOut=dO if bias else None,
                               dbias=db, dout_fmt=fmt, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(Iq.value(), qi) and np.array_equal(Q.value(), qd)
    e = _err(dW.double().cpu().numpy(), F.fp8_linear(qi, qd, 0, FMT[fmt], si_, sd))
    _say(f"  dW {e:.2e}")
    assert e <= TOL["f32"]
    if bias:
        assert _err(db.double().cpu().numpy(), dOf.sum(axis=0)) <= TOL["f32"]


@pytest.mark.parametrize("tile,split", [(12, 1), (13, 1), (14, 1), (15, 1), (13, 3), (12, 2)])
def test_fp8_tiles(dev, tile, split):
    """Every FP8 tile, forced, on a weight gradient (fp32 store, split K) and a
    forward with bias + GeLU."""
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"fp8 tile {tile} split {split}")
    rng = np.random.default_rng(tile * 10 + split)
    T, k, n = 1536, 768, 768
    Inf, Inb = rand_bf16(rng, (T, k), 1.0)
    dOf, dOb = rand_bf16(rng, (T, n), 1.0)
    Atf, Atb = rand_bf16(rng, (n, k), 0.02)
    try:
        tp.tp_set_gemm_override(tile, split)
        Iq, isi, qi, si_ = _quant_both(tp, Inf, Inb, "e4m3", True, dev)
        Dq, dsi, qd, sd = _quant_both(tp, dOf, dOb, "e5m2", True, dev)
        dW = torch.full((k, n), float("nan"), device=dev)
        ws = torch.empty(max(16, tp.tp_fp8_linear_bwd_wgrad_workspace_size(T, k, n)),
                         dtype=torch.uint8, device=dev)
        tp.tp_fp8_linear_bwd_wgrad(Iq.view, Dq.view, isi, dsi, dW, dout_fmt="e5m2", workspace=ws)
        Xq, xsi, qx, sx = _quant_both(tp, Inf, Inb, "e4m3", False, dev)
        Aq, asi, qa, sa = _quant_both(tp, Atf, Atb, "e4m3", False, dev)   # A^T [n, k]
        Y = torch.empty(T, n, dtype=torch.bfloat16, device=dev)
        U = torch.empty(T, n, dtype=torch.bfloat16, device=dev)
        tp.tp_fp8_column_linear_fwd(Xq.view, Aq.view, xsi, asi, None, Y, U)
        torch.cuda.synchronize()
    finally:
        tp.tp_set_gemm_override(0)
    assert _err(dW.double().cpu().numpy(), F.fp8_linear(qi, qd, 0, 1, si_, sd)) <= TOL["f32"]
    Y_ref, U_ref = F.fp8_linear(qx, qa, 0, 0, sx, sa, act="gelu")
    assert _err(U.double().cpu().numpy(), U_ref) <= TOL["bf16"]
    assert _err(Y.double().cpu().numpy(), Y_ref) <= TOL["bf16"]


def test_fp8_deterministic(dev):
    import tensor_transformer_layer_fwd_amd as tp
    rng = np.random.default_rng(99)
    T, k, n = 4096, 1536, 768
    _, Inb = rand_bf16(rng, (T, k), 1.0)
    _, dOb = rand_bf16(rng, (T, n), 1.0)
    outs = []
    for _ in range(3):
        Iq, isi = quantize_dev(tp, to_dev_bf16(Inb, dev), "e4m3", True, dev)
        Dq, dsi = quantize_dev(tp, to_dev_bf16(dOb, dev), "e5m2", True, dev)
        dW = torch.empty(k, n, device=dev)
        ws = torch.empty(max(16, tp.tp_fp8_linear_bwd_wgrad_workspace_size(T, k, n)),
                         dtype=torch.uint8, device=dev)
        tp.tp_fp8_linear_bwd_wgrad(Iq.view, Dq.view, isi, dsi, dW, workspace=ws)
        outs.append(dW.cpu())
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


@pytest.mark.parametrize("name,mb,seq", [("gpt2s", 1, 640), ("gpt2s", 2, 512),
                                         ("gpt175b", 1, 256)])
def test_workload_fp8_step(dev, name, mb, seq):
    """The whole MLP step in FP8 against the oracle's FP8 step (every output).
    Both quantise the same stored values; the intermediates U_i, Y_i, dU_i
    differ only where fp32 and float64 round to different bf16 neighbours,
    and a code then flips only where an FP8 boundary lies between them, so
    the outputs stay within the bf16 bar."""
    import dataclasses
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    from tp_inputs import get_config, make_inputs
    cfg = dataclasses.replace(get_config(name), micro_batch=mb, seq=seq)
    if name == "gpt175b":
        cfg = dataclasses.replace(cfg, h=1024)
    _say(f"fp8 step {name} T={cfg.T} h={cfg.h}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev, fp8=True)
    step.run_eager()
    got = step.results()
    ref = F.run_config_fp8(cfg, inputs)
    worst = (0.0, None)
    for k, r in ref.items():
        e = _err(got[k], r)
        worst = max(worst, (e, k))
        assert e <= TOL["bf16"], (k, e)
    _say(f"  worst {worst[0]:.2e} ({worst[1]})")


def test_fp8_step_graph_replay(dev):
    """The FP8 step captured into a HIP graph replays bitwise like the eager step."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    from tp_inputs import get_config, make_inputs
    cfg = get_config("gpt2s")
    step = ShardStep(cfg, make_inputs(cfg), dev, fp8=True)
    step.run_eager()
    eager = {k: v.clone() for k, v in step.out.items()}
    step.capture()
    for _ in range(3):
        step.run()
        torch.cuda.synchronize()
        for k, v in step.out.items():
            assert torch.equal(v, eager[k]), k


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("rows,cols", [(37, 53), (300, 1000), (768, 4096)])
def test_quantize_both_equals_two_calls(dev, fmt, rows, cols):
    """Both layouts from one read: the codes of each layout and the scale
    equal the oracle's (as for the single-layout calls)."""
    import tensor_transformer_layer_fwd_amd as tp
    rng = np.random.default_rng(rows + cols + len(fmt))
    Xf, bits = rand_bf16(rng, (rows, cols), 1.5)
    X = to_dev_bf16(bits, dev, pad=8)
    Q, Qt = Codes(rows, cols, dev, pad=16), Codes(cols, rows, dev, pad=16)
    si = torch.full((1,), float("nan"), device=dev)
    ws = torch.empty(tp.tp_fp8_quantize_workspace_size(rows, cols), dtype=torch.uint8, device=dev)
    tp.tp_fp8_quantize_both(X, Q.view, Qt.view, si, ws, fmt=fmt)
    torch.cuda.synchronize()
    q_ref, _, sinv = F.quantize(Xf, FMT[fmt])
    assert np.array_equal(Q.value(), q_ref) and np.array_equal(Qt.value(), q_ref.T)
    assert si.item() == float(sinv)


@pytest.mark.parametrize("n", [1, 3, 6])
def test_quantize_both_multi(dev, n):
    """Several tensors in two launches: each tensor's codes in both layouts and
    its scale equal the oracle's, and nothing lands outside any output."""
    import tensor_transformer_layer_fwd_amd as tp
    shapes = [(37, 53, "bf16", "e4m3"), (300, 1000, "f32", "e5m2"), (768, 4096, "bf16", "e4m3"),
              (1, 1, "bf16", "e5m2"), (256, 384, "f32", "e4m3"), (64, 1536, "bf16", "e5m2")][:n]
    _say(f"fp8 quantize_both_multi n={n}")
    rng = np.random.default_rng(100 + n)
    items, refs = [], []
    for k, (rows, cols, dt, fmt) in enumerate(shapes):
        scale = 0.5 * (k + 1)   # a different maximum, so a mixed-up scale shows
        if dt == "bf16":
            Xf, bits = rand_bf16(rng, (rows, cols), scale)
            X = to_dev_bf16(bits, dev, pad=8)
        else:
            Xf = (rng.standard_normal((rows, cols)) * scale).astype(np.float32).astype(np.float64)
            X = torch.from_numpy(Xf.astype(np.float32)).to(dev)
        Q, Qt = Codes(rows, cols, dev, pad=16), Codes(cols, rows, dev, pad=16)
        si = torch.full((1,), float("nan"), device=dev)
        items.append((X, Q.view, Qt.view, si, fmt))
        refs.append((Xf, fmt, Q, Qt, si))
    ws = torch.empty(tp.tp_fp8_quantize_multi_workspace_size(n), dtype=torch.uint8, device=dev)
    tp.tp_fp8_quantize_both_multi(items, ws)
    torch.cuda.synchronize()
    for Xf, fmt, Q, Qt, si in refs:
        q_ref, _, sinv = F.quantize(Xf, FMT[fmt])
        assert np.array_equal(Q.value(), q_ref) and np.array_equal(Qt.value(), q_ref.T)
        assert si.item() == float(sinv)


@pytest.mark.parametrize("tile", [0, 12, 13, 14, 15])
def test_fp8_amax_epilogues_give_the_two_pass_codes(dev, tile):
    """fc1's bias + GeLU epilogue and fc2 dgrad's GeLU' epilogue leave the
    largest |stored value| per (tile, wave) slot; the one-launch quantiser on
    those slots gives exactly the codes and 1/s of the two-pass quantiser on
    the same output, and of the oracle's quantiser (every FP8 tile forced)."""
    import tensor_transformer_layer_fwd_amd as tp
    _say(f"fp8 amax epilogues tile {tile}")
    rng = np.random.default_rng(70 + tile)
    T, h, n = 1536, 768, 768
    Xf, Xb = rand_bf16(rng, (T, h), 1.0)
    Atf, Atb = rand_bf16(rng, (n, h), 0.05)
    af, ab = rand_bf16(rng, (1, n), 0.1)
    dZf, dZb = rand_bf16(rng, (T, h), 1.0)
    Bf, Bb = rand_bf16(rng, (n, h), 0.05)     # B_i [F, h] as stored
    try:
        tp.tp_set_gemm_override(tile)
        Xq, xsi, _, _ = _quant_both(tp, Xf, Xb, "e4m3", False, dev)
        Aq, asi, _, _ = _quant_both(tp, Atf, Atb, "e4m3", False, dev)
        dq, dsi, _, _ = _quant_both(tp, dZf, dZb, "e5m2", False, dev)
        Bq, bsi, _, _ = _quant_both(tp, Bf, Bb, "e4m3", False, dev)
        slots = tp.tp_fp8_amax_slots(T, n, h)
        outs = []
        for what in ("fwd", "dgrad"):
            Y = torch.empty(T, n, dtype=torch.bfloat16, device=dev)
            U = torch.empty(T, n, dtype=torch.bfloat16, device=dev)
            amax = torch.full((slots,), float("nan"), device=dev)
            fmt = "e4m3" if what == "fwd" else "e5m2"
            if what == "fwd":
                tp.tp_fp8_column_linear_fwd(Xq.view, Aq.view, xsi, asi, to_dev_bf16(ab, dev)[0],
                                            Y, U, amax=amax)
            else:
                Ud = to_dev_bf16(f32_to_bf16_bits((rng.standard_normal((T, n)) * 1.5)
                                                  .astype(np.float32)), dev)
                tp.tp_fp8_linear_bwd_dgrad(dq.view, Bq.view, dsi, bsi, Y, U=Ud, act="gelu",
                                           dout_fmt="e5m2", amax=amax)
            Q1, Qt1 = Codes(T, n, dev), Codes(n, T, dev)
            s1 = torch.full((1,), float("nan"), device=dev)
            tp.tp_fp8_quantize_both_from_amax(Y, Q1.view, Qt1.view, s1, amax, slots, fmt=fmt)
            Q2, Qt2 = Codes(T, n, dev), Codes(n, T, dev)
            s2 = torch.full((1,), float("nan"), device=dev)
            ws = torch.empty(tp.tp_fp8_quantize_workspace_size(T, n), dtype=torch.uint8,
                             device=dev)
            tp.tp_fp8_quantize_both(Y, Q2.view, Qt2.view, s2, ws, fmt=fmt)
            torch.cuda.synchronize()
            outs.append((what, Y, amax, (Q1, Qt1, s1), (Q2, Qt2, s2), fmt))
    finally:
        tp.tp_set_gemm_override(0)
    for what, Y, amax, (Q1, Qt1, s1), (Q2, Qt2, s2), fmt in outs:
        y = Y.double().cpu().numpy()
        a = amax.cpu().numpy()
        assert not np.isnan(a).any(), f"{what}: a slot was not written"
        assert a.max() == np.abs(y).max(), (what, a.max(), np.abs(y).max())
        assert np.array_equal(Q1.value(), Q2.value()) and np.array_equal(Qt1.value(), Qt2.value())
        assert s1.item() == s2.item()
        q_ref, _, sinv = F.quantize(y, FMT[fmt])
        assert np.array_equal(Q1.value(), q_ref) and np.array_equal(Qt1.value(), q_ref.T)
        assert s1.item() == np.float32(sinv)
