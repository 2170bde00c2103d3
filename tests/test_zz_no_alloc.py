"""The allocation-free weight-gradient entry point against tp_linear_bwd_wgrad.

tp_linear_bwd_wgrad_noalloc runs the kernels of tp_linear_bwd_wgrad on the
library's static per-GPU scratch array instead of a caller workspace, so its
results must equal that call's bit for bit; the oracle's dW = In^T dOut and
column sums hold both to the fp32 bound of the other weight-gradient tests.
Two calls in a row, the second on a smaller shape, show that what one call
leaves in the array does not leak into the next.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from tp_inputs import bf16_bits_to_f32, f32_to_bf16_bits

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _upload(rng, rows, cols, dt, pad):
    """Seeded values exact in dt, as a strided device view (row stride cols + pad)."""
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        bits = f32_to_bf16_bits(x)
        exact = bf16_bits_to_f32(bits).astype(np.float64)
        src = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    else:
        exact, src = x.astype(np.float64), torch.from_numpy(x)
    buf = torch.zeros(rows, cols + pad, dtype=tdt, device=DEV)
    buf[:, :cols] = src.to(DEV)
    return exact, buf[:, :cols]


def _run(T, k, n, dt, bias, accumulate, seed):
    import tensor_transformer_layer_fwd_amd as tp
    from tensor_transformer_layer_fwd_amd import _lib as L
    _say(f"noalloc wgrad T={T} k={k} n={n} dt={dt} bias={bias} acc={accumulate}")
    rng = np.random.default_rng(seed)
    In, In_d = _upload(rng, T, k, dt, 3)
    dO, dO_d = _upload(rng, T, n, dt, 5)
    prev_w = rng.standard_normal((k, n)).astype(np.float32)
    prev_b = rng.standard_normal(n).astype(np.float32)
    outs = []
    for call in ("workspace", "noalloc"):
        wbuf = torch.full((k, n + 4), float("nan"), device=DEV)
        dW = wbuf[:, :n]
        db = torch.full((n,), float("nan"), device=DEV)
        if accumulate:
            dW.copy_(torch.from_numpy(prev_w))
            db.copy_(torch.from_numpy(prev_b))
        if call == "workspace":
            wsb = L.tp_linear_bwd_wgrad_workspace_size(
                T, k, n, L.TP_BF16 if dt == "bf16" else L.TP_F32)
            ws = torch.full((max(wsb, 16),), 255, dtype=torch.uint8, device=DEV)
            tp.tp_linear_bwd_wgrad(In_d, dO_d, dW, db if bias else None, accumulate=accumulate,
                                   workspace=ws)
        else:
            L.tp_linear_bwd_wgrad_noalloc(In_d, dO_d, dW, db if bias else None,
                                          accumulate=accumulate)
        torch.cuda.synchronize()
        assert torch.isnan(wbuf[:, n:]).all(), "a kernel wrote outside dW"
        outs.append((dW.cpu().numpy().astype(np.float64), db.cpu().numpy().astype(np.float64)))
    (w_ref, b_ref), (w_got, b_got) = outs
    assert np.array_equal(w_ref, w_got), np.abs(w_ref - w_got).max()
    rw, rb = oracle.linear_bwd_wgrad(In, dO)
    if accumulate:
        rw, rb = rw + prev_w, rb + prev_b
    assert oracle.rel_fro(w_got, rw) <= 1e-5
    if bias:
        assert np.array_equal(b_ref, b_got), np.abs(b_ref - b_got).max()
        assert oracle.rel_fro(b_got, rb) <= 1e-5
    else:  # no bias gradient requested: dbias untouched
        assert np.all(np.isnan(b_got))


@pytest.mark.parametrize("accumulate", [False, True])
def test_noalloc_two_calls_second_smaller(accumulate):
    # a split-K shape of the GPT-2-small shard (scratch holds split-K and
    # column-sum partials), then a small ragged one over the leftovers
    _run(4096, 768, 1536, "bf16", True, accumulate, 11)
    _run(513, 200, 136, "bf16", True, accumulate, 12)


def test_noalloc_no_bias_and_fp32():
    _run(2048, 384, 256, "bf16", False, False, 21)
    _run(300, 96, 72, "f32", True, False, 22)
