"""GPU parity of the attention block: the column-split QKV projection, the
shard's attention core and the row-split output projection, forward and
backward, through the C ABI, against oracle.attention.tp_attn_block.

Tolerance 5e-3 relative Frobenius error per output tensor, as for every bf16
output. lse (fp32, the natural log of each query's softmax normaliser) is
held to a bound derived from the arithmetic: the device's scores come from
QKV_i rounded to bf16, so each product q_d k_d carries a relative error of at
most (1 + 2^-8)^2 - 1, a score s_qk = sum_d q_d k_d / 8 an absolute error of at
most that times sum_d |q_d k_d| / 8, and lse (a softmax-weighted mean of the
scores to first order) at most the largest of those over the keys the query
sees, plus 1e-5 for the fp32 sums.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.sampled import attn_block_sampled
from tp_inputs import get_config, make_inputs

pytestmark = pytest.mark.gpu

TOL = 5e-3


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a ROCm GPU")
    import tensor_transformer_layer_fwd_amd as tp  # noqa: F401  (fails loudly if not built)
    return torch.device("cuda:0")


def _lse_bound(QKV, batch, seq, heads, causal=True):
    """Per-query bound [batch, heads, seq] on |lse_device - lse_exact| from the
    bf16 rounding of Q and K (module docstring)."""
    x = np.abs(np.asarray(QKV, np.float64)).reshape(batch, seq, 3, heads, 64)
    q, k = x[:, :, 0], x[:, :, 1]
    m = np.einsum("bqhd,bkhd->bhqk", q, k, optimize=True) / 8.0
    if causal:
        m = np.where(np.tril(np.ones((seq, seq), dtype=bool)), m, 0.0)
    rel = (1.0 + 2.0 ** -8) ** 2 - 1.0
    return rel * m.max(axis=-1) + 1e-5


def _check(got, ref, keys=None, cfg=None):
    worst = (0.0, None)
    for k in (keys or ref):
        r = ref[k]
        g = got[k].reshape(r.shape)
        if k.startswith("lse_"):
            i = k.split("_")[1]
            H = cfg.heads // cfg.p
            bound = _lse_bound(ref[f"QKV_{i}"], r.shape[0], cfg.seq, H)
            d = np.abs(g - r)
            assert np.all(d <= bound), (k, float(d.max()), float(bound.min()))
            continue
        e = oracle.rel_fro(g, r)
        worst = max(worst, (e, k))
        assert e <= TOL, (k, e)
    return worst


@pytest.mark.parametrize("name,mb", [("attn", 2), ("gpt350m", 1)])
def test_attention_block_reduced(dev, name, mb):
    """Whole sequences of the workload (fewer of them): every output of the
    block and of the MLP (the ~350M layer) in full."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = dataclasses.replace(get_config(name), micro_batch=mb)
    _say(f"attention block {name} T={cfg.T} h={cfg.h} p={cfg.p}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev, attn_core=True)
    step.run_eager()
    got = step.results()
    ref = oracle.run_config(cfg, inputs, attn_core=True)
    assert set(ref) <= set(got), set(ref) - set(got)
    worst = _check(got, ref, cfg=cfg)
    _say(f"  worst rel err {worst[0]:.3e} ({worst[1]})")


@pytest.mark.parametrize("name", ["attn", "gpt350m"])
def test_attention_block_full_size(dev, name):
    """The full workload, graph-replayed as the benchmark runs it: the token
    rows of two whole sequences (the first and the last) against the oracle's
    block on those sequences; for the attention-projection workload also the
    weight gradients in full (the oracle's whole block)."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = get_config(name)
    _say(f"attention block full {name} T={cfg.T} h={cfg.h} p={cfg.p}")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev, attn_core=True)
    step.capture()
    for _ in range(2):
        step.run()
    got = step.results()
    for k, v in got.items():
        assert np.all(np.isfinite(v)), k
    g = {k: v.f64() for k, v in inputs.items()}
    seqs = [0, cfg.micro_batch - 1]
    ref = attn_block_sampled(g["X"], g["W"], g["Ow"], g["dZa"], cfg.p, cfg.micro_batch, cfg.seq,
                             cfg.heads, seqs)
    rows = np.concatenate([np.arange(s * cfg.seq, (s + 1) * cfg.seq) for s in seqs])
    got_s = {}
    for k in ref:
        v = got[k]
        got_s[k] = v[seqs] if k.startswith("lse_") else v[rows]
    worst = _check(got_s, ref, cfg=cfg)
    _say(f"  sampled sequences: worst rel err {worst[0]:.3e} ({worst[1]})")
    if name == "attn":
        from oracle.attention import tp_attn_block
        full = tp_attn_block(g["X"], g["W"], g["Ow"], g["dZa"], cfg.p, cfg.micro_batch, cfg.seq,
                             cfg.heads)
        keys = [k for k in full if k.startswith(("dW_", "dOw_"))]
        worst = _check(got, full, keys, cfg=cfg)
        _say(f"  weight gradients: worst rel err {worst[0]:.3e} ({worst[1]})")


def test_attention_block_graph_replay_is_bitwise(dev):
    """Graph replays of the block equal its eager run bitwise (no atomics in
    the core, fixed orders everywhere)."""
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    cfg = dataclasses.replace(get_config("gpt350m"), micro_batch=1, seq=512)
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, dev, attn_core=True)
    step.run_eager()
    want = step.results()
    step.capture()
    for _ in range(3):
        step.run()
        torch.cuda.synchronize()
        got = step.results()
        for k in want:
            np.testing.assert_array_equal(got[k], want[k], err_msg=k)


@pytest.mark.parametrize("shards,batch,seq,heads", [(2, 2, 512, 8), (4, 1, 1024, 4), (3, 2, 200, 2)])
def test_attention_core_of_several_shards_in_one_launch(dev, shards, batch, seq, heads):
    """tp_attention_fwd_shards / tp_attention_bwd_shards over shards side by
    side (each shard's [Q | K | V] block, its C heads, its lse rows) give the
    per-shard calls' C, lse and dQKV bit for bit, including a ragged
    sequence."""
    from tensor_transformer_layer_fwd_amd import _lib as L
    _say(f"attention core, {shards} shards in one launch: {batch} x {seq}, {heads} heads")
    g = torch.Generator(device=dev)
    g.manual_seed(1000 * shards + seq)
    T, hq, hc = batch * seq, 3 * heads * 64, heads * 64
    bf = dict(device=dev, dtype=torch.bfloat16)
    QKV = torch.randn(T, shards * hq, device=dev, generator=g).to(torch.bfloat16)
    dC = torch.randn(T, shards * hc, device=dev, generator=g).to(torch.bfloat16)
    C = torch.empty(T, shards * hc, **bf)
    dQKV = torch.empty(T, shards * hq, **bf)
    lse = torch.empty(batch, shards * heads, seq, device=dev)
    delta = torch.empty_like(lse)
    L.tp_attention_fwd(QKV, C, lse, batch, seq, heads, shards=shards)
    L.tp_attention_bwd(QKV, C, dC, lse, delta, dQKV, batch, seq, heads, shards=shards)
    for s in range(shards):
        q, c = slice(s * hq, (s + 1) * hq), slice(s * hc, (s + 1) * hc)
        Cs = torch.empty(T, hc, **bf)
        ls = torch.empty(batch, heads, seq, device=dev)
        dQs = torch.empty(T, hq, **bf)
        L.tp_attention_fwd(QKV[:, q], Cs, ls, batch, seq, heads)
        L.tp_attention_bwd(QKV[:, q], Cs, dC[:, c].contiguous(), ls, torch.empty_like(ls), dQs,
                           batch, seq, heads)
        torch.cuda.synchronize()
        assert torch.equal(C[:, c], Cs), f"C of shard {s}"
        assert torch.equal(lse[:, s * heads:(s + 1) * heads], ls), f"lse of shard {s}"
        assert torch.equal(dQKV[:, q], dQs), f"dQKV of shard {s}"
