"""Pins of the attention-core oracle (CPU only)."""
import math

import numpy as np
import pytest

from oracle.attention import attention_core_fwd, split_qkv


def _brute(QKV, batch, seq, heads, d, causal):
    """Pure-Python loops: exp and correctly rounded sums (math.fsum)."""
    rows = [list(map(float, r)) for r in np.asarray(QKV, dtype=np.float64)]
    C = [[0.0] * (heads * d) for _ in range(batch * seq)]
    lse = [[[0.0] * seq for _ in range(heads)] for _ in range(batch)]
    for b in range(batch):
        for h in range(heads):
            for qi in range(seq):
                qrow = rows[b * seq + qi][h * d:(h + 1) * d]
                keys = range(qi + 1) if causal else range(seq)
                sc = []
                for ki in keys:
                    krow = rows[b * seq + ki][heads * d + h * d:heads * d + (h + 1) * d]
                    sc.append(math.fsum(x * y for x, y in zip(qrow, krow)) / math.sqrt(d))
                mx = max(sc)
                w = [math.exp(x - mx) for x in sc]
                den = math.fsum(w)
                lse[b][h][qi] = mx + math.log(den)
                for j in range(d):
                    C[b * seq + qi][h * d + j] = math.fsum(
                        wk * rows[b * seq + ki][2 * heads * d + h * d + j]
                        for wk, ki in zip(w, keys)) / den
    return np.array(C), np.array(lse)


@pytest.mark.parametrize("causal", [True, False])
def test_brute_force_tiny(causal):
    rng = np.random.default_rng(5)
    batch, seq, heads, d = 2, 5, 2, 3
    QKV = rng.standard_normal((batch * seq, 3 * heads * d))
    C, lse = attention_core_fwd(QKV, batch, seq, heads, d, causal)
    Cb, lseb = _brute(QKV, batch, seq, heads, d, causal)
    np.testing.assert_allclose(C, Cb, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lseb, rtol=1e-13, atol=1e-14)


def test_zero_queries_give_prefix_means():
    """Q = 0: all scores 0, so causal attention is the mean of V over positions
    0..q and lse = log(q + 1)."""
    rng = np.random.default_rng(6)
    batch, seq, heads, d = 3, 7, 2, 4
    QKV = rng.standard_normal((batch * seq, 3 * heads * d))
    QKV[:, :heads * d] = 0.0
    C, lse = attention_core_fwd(QKV, batch, seq, heads, d)
    _, _, v = split_qkv(QKV, batch, seq, heads, d)
    mean = np.cumsum(v, axis=1) / np.arange(1, seq + 1)[None, :, None, None]
    np.testing.assert_allclose(C, mean.reshape(batch * seq, heads * d), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, seq + 1)), lse.shape),
                               rtol=1e-13)


def test_first_position_sees_only_itself():
    rng = np.random.default_rng(7)
    batch, seq, heads, d = 2, 6, 3, 8
    QKV = rng.standard_normal((batch * seq, 3 * heads * d)) * 3
    C, _ = attention_core_fwd(QKV, batch, seq, heads, d)
    _, _, v = split_qkv(QKV, batch, seq, heads, d)
    np.testing.assert_array_equal(C.reshape(batch, seq, heads, d)[:, 0], v[:, 0])


def test_one_hot_attention_picks_a_value_row():
    """Each query aligned with one earlier key at a large scale: the output is
    that key's value row (to within exp(-gap))."""
    batch, seq, heads, d = 1, 6, 1, 6
    rng = np.random.default_rng(8)
    QKV = np.zeros((seq, 3 * d))
    QKV[:, d:2 * d] = np.eye(seq, d) * 40.0      # key k = 40 e_k
    target = [0, 0, 1, 2, 1, 4]                  # query q looks at key target[q] <= q
    for qi, t in enumerate(target):
        QKV[qi, :d] = np.eye(d)[t] * 40.0
    QKV[:, 2 * d:] = rng.standard_normal((seq, d))
    C, _ = attention_core_fwd(QKV, batch, seq, heads, d)
    np.testing.assert_allclose(C, QKV[target, 2 * d:], rtol=0, atol=1e-12)


def test_last_row_is_unmasked_and_sequences_are_independent():
    rng = np.random.default_rng(9)
    batch, seq, heads, d = 4, 9, 2, 5
    QKV = rng.standard_normal((batch * seq, 3 * heads * d))
    Cc, lc = attention_core_fwd(QKV, batch, seq, heads, d, causal=True)
    Cn, ln = attention_core_fwd(QKV, batch, seq, heads, d, causal=False)
    last = np.arange(batch) * seq + seq - 1
    np.testing.assert_allclose(Cc[last], Cn[last], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lc[:, :, -1], ln[:, :, -1], rtol=1e-14)
    perm = np.array([2, 0, 3, 1])
    QKVp = QKV.reshape(batch, seq, -1)[perm].reshape(batch * seq, -1)
    Cp, lp = attention_core_fwd(QKVp, batch, seq, heads, d)
    np.testing.assert_array_equal(Cp.reshape(batch, seq, -1), Cc.reshape(batch, seq, -1)[perm])
    np.testing.assert_array_equal(lp, lc[perm])


def test_weights_are_normalised():
    """exp(score - lse) sums to one over the visible keys of every query."""
    rng = np.random.default_rng(10)
    batch, seq, heads, d = 2, 11, 3, 4
    QKV = rng.standard_normal((batch * seq, 3 * heads * d)) * 2
    _, lse = attention_core_fwd(QKV, batch, seq, heads, d)
    q, k, _ = split_qkv(QKV, batch, seq, heads, d)
    s = np.einsum("bqhd,bkhd->bhqk", q, k) / math.sqrt(d)
    w = np.exp(s - lse[..., None]) * np.tril(np.ones((seq, seq)))
    np.testing.assert_allclose(w.sum(-1), 1.0, rtol=1e-13)


from oracle.attention import attention_core_bwd  # noqa: E402


@pytest.mark.parametrize("causal", [True, False])
def test_backward_finite_differences(causal):
    """<dC, dC_dir> sensitivity: d/de L(QKV + e*E) with L = <G, C(QKV)> equals
    <dQKV, E>, checked by central differences in float64."""
    rng = np.random.default_rng(11)
    batch, seq, heads, d = 2, 6, 2, 4
    QKV = rng.standard_normal((batch * seq, 3 * heads * d))
    G = rng.standard_normal((batch * seq, heads * d))
    dQKV = attention_core_bwd(QKV, G, batch, seq, heads, d, causal)
    for trial in range(4):
        E = rng.standard_normal(QKV.shape)
        h = 1e-5
        lp = np.sum(G * attention_core_fwd(QKV + h * E, batch, seq, heads, d, causal)[0])
        lm = np.sum(G * attention_core_fwd(QKV - h * E, batch, seq, heads, d, causal)[0])
        assert abs((lp - lm) / (2 * h) - np.sum(dQKV * E)) <= 1e-7 * (1 + abs(np.sum(dQKV * E)))


def _brute_bwd(QKV, G, batch, seq, heads, d, causal):
    """Chain rule written out per element with pure-Python loops."""
    X = [list(map(float, r)) for r in np.asarray(QKV, dtype=np.float64)]
    Gl = [list(map(float, r)) for r in np.asarray(G, dtype=np.float64)]
    out = [[0.0] * (3 * heads * d) for _ in range(batch * seq)]
    sc = 1.0 / math.sqrt(d)
    for b in range(batch):
        for h in range(heads):
            Q = [X[b * seq + t][h * d:(h + 1) * d] for t in range(seq)]
            K = [X[b * seq + t][heads * d + h * d:heads * d + (h + 1) * d] for t in range(seq)]
            V = [X[b * seq + t][2 * heads * d + h * d:2 * heads * d + (h + 1) * d] for t in range(seq)]
            for qi in range(seq):
                keys = list(range(qi + 1)) if causal else list(range(seq))
                s = [math.fsum(a * c for a, c in zip(Q[qi], K[ki])) * sc for ki in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                den = math.fsum(w)
                pr = [x / den for x in w]
                g = Gl[b * seq + qi][h * d:(h + 1) * d]
                dp = [math.fsum(a * c for a, c in zip(g, V[ki])) for ki in keys]
                dot = math.fsum(a * c for a, c in zip(pr, dp))
                ds = [p_ * (x - dot) for p_, x in zip(pr, dp)]
                for j in range(d):
                    out[b * seq + qi][h * d + j] += math.fsum(
                        x * K[ki][j] for x, ki in zip(ds, keys)) * sc
                for x, p_, ki in zip(ds, pr, keys):
                    for j in range(d):
                        out[b * seq + ki][heads * d + h * d + j] += x * Q[qi][j] * sc
                        out[b * seq + ki][2 * heads * d + h * d + j] += p_ * g[j]
    return np.array(out)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_brute_force(causal):
    rng = np.random.default_rng(12)
    batch, seq, heads, d = 2, 5, 2, 3
    QKV = rng.standard_normal((batch * seq, 3 * heads * d))
    G = rng.standard_normal((batch * seq, heads * d))
    np.testing.assert_allclose(attention_core_bwd(QKV, G, batch, seq, heads, d, causal),
                               _brute_bwd(QKV, G, batch, seq, heads, d, causal),
                               rtol=1e-12, atol=1e-13)


def test_backward_special_cases():
    """Q = 0 (uniform causal weights): dV[k] = sum over q >= k of dC[q]/(q+1)
    and dK = 0 exactly. For any inputs each query's score gradient sums to
    zero over its keys (softmax is shift-invariant), so dK sums to zero over
    the keys of a sequence."""
    rng = np.random.default_rng(13)
    batch, seq, heads, d = 1, 7, 1, 4
    QKV = rng.standard_normal((seq, 3 * d))
    QKV[:, :d] = 0.0
    G = rng.standard_normal((seq, d))
    dQKV = attention_core_bwd(QKV, G, batch, seq, heads, d, True)
    w = 1.0 / np.arange(1, seq + 1)
    dv_ref = np.array([np.sum(G[k:] * w[k:, None], axis=0) for k in range(seq)])
    np.testing.assert_allclose(dQKV[:, 2 * d:], dv_ref, rtol=1e-13, atol=1e-14)
    # with Q = 0, dK = dS^T Q / sqrt(d) = 0 exactly
    np.testing.assert_array_equal(dQKV[:, d:2 * d], 0.0)
    # for general inputs, sum over keys of dK = (sum_k dS[q,k]) Q ... = 0
    QKV2 = rng.standard_normal((seq, 3 * d))
    dQKV2 = attention_core_bwd(QKV2, G, batch, seq, heads, d, True)
    np.testing.assert_allclose(dQKV2[:, d:2 * d].sum(axis=0), 0.0, atol=1e-12)


# --------------------------------------------------------------------------- #
# the attention block: projections with the core between them                  #
# --------------------------------------------------------------------------- #
from oracle.attention import tp_attn_block  # noqa: E402


def _block_inputs(rng, batch, seq, heads, d, h):
    T = batch * seq
    X = rng.standard_normal((T, h))
    W = rng.standard_normal((h, 3 * heads * d)) * 0.3
    Ow = rng.standard_normal((heads * d, h)) * 0.3
    dZa = rng.standard_normal((T, h))
    return X, W, Ow, dZa


@pytest.mark.parametrize("causal", [True, False])
def test_block_finite_differences(causal):
    """L = <dZa, Za(X, W, Ow)>: central differences along random directions
    in X, W and Ow equal <dXq, E>, <[dW_0 .. dW_p-1], E> and <[dOw_0; ..], E>."""
    rng = np.random.default_rng(21)
    batch, seq, heads, d, h, p = 2, 5, 4, 3, 7, 2
    X, W, Ow, dZa = _block_inputs(rng, batch, seq, heads, d, h)
    g = tp_attn_block(X, W, Ow, dZa, p, batch, seq, heads, d=d, causal=causal)
    dW = np.concatenate([g[f"dW_{i}"] for i in range(p)], axis=1)
    dOw = np.concatenate([g[f"dOw_{i}"] for i in range(p)], axis=0)

    def loss(X_, W_, Ow_):
        return np.sum(dZa * tp_attn_block(X_, W_, Ow_, dZa, p, batch, seq, heads, d=d,
                                          causal=causal)["Za"])

    eps = 1e-5
    for grad, which in ((g["dXq"], 0), (dW, 1), (dOw, 2)):
        for _ in range(3):
            args = [X, W, Ow]
            E = rng.standard_normal(args[which].shape)
            plus = list(args)
            minus = list(args)
            plus[which] = args[which] + eps * E
            minus[which] = args[which] - eps * E
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            an = np.sum(grad * E)
            assert abs(fd - an) <= 1e-7 * (1 + abs(an)), (which, fd, an)


def test_block_is_independent_of_the_tp_degree():
    """Heads do not interact, so the block over p = 1, 2, 4 shards gives the
    same sums when W's columns are laid out per shard as [Q | K | V] of that
    shard's heads (and Ow's rows as its heads' rows): this pins the head and
    shard indexing of the column and row splits."""
    rng = np.random.default_rng(22)
    batch, seq, heads, d, h = 2, 4, 4, 2, 5
    X, W1, Ow, dZa = _block_inputs(rng, batch, seq, heads, d, h)
    ref = tp_attn_block(X, W1, Ow, dZa, 1, batch, seq, heads, d=d)
    for p in (2, 4):
        H = heads // p
        # p = 1 layout: [Q heads 0..3 | K heads 0..3 | V heads 0..3]
        cols = []
        for i in range(p):
            for part in range(3):
                for j in range(i * H, (i + 1) * H):
                    cols.extend(range(part * heads * d + j * d, part * heads * d + (j + 1) * d))
        Wp = W1[:, cols]
        got = tp_attn_block(X, Wp, Ow, dZa, p, batch, seq, heads, d=d)
        np.testing.assert_allclose(got["Za"], ref["Za"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(got["dXq"], ref["dXq"], rtol=1e-12, atol=1e-12)
        dWp = np.concatenate([got[f"dW_{i}"] for i in range(p)], axis=1)
        np.testing.assert_allclose(dWp, ref["dW_0"][:, cols], rtol=1e-12, atol=1e-12)
        dOwp = np.concatenate([got[f"dOw_{i}"] for i in range(p)], axis=0)
        np.testing.assert_allclose(dOwp, ref["dOw_0"], rtol=1e-12, atol=1e-12)


def test_block_with_zero_queries_and_identity_values():
    """W with a zero Q block and a V block that copies the first d features of
    X per head: causal attention is then the running mean of those features,
    so Za = prefix-mean(X[:, :d] per head) Ow, written out directly."""
    rng = np.random.default_rng(23)
    batch, seq, heads, d, h, p = 2, 6, 2, 3, 4, 2
    X, W, Ow, dZa = _block_inputs(rng, batch, seq, heads, d, h)
    H = heads // p
    Q = 3 * H * d
    for i in range(p):
        blk = W[:, i * Q:(i + 1) * Q]
        blk[:, :H * d] = 0.0                       # Q of the shard's heads
        blk[:, 2 * H * d:] = 0.0                   # V of the shard's heads
        for j in range(H):
            for c in range(d):
                blk[c, 2 * H * d + j * d + c] = 1.0
    got = tp_attn_block(X, W, Ow, dZa, p, batch, seq, heads, d=d)
    xs = X[:, :d].reshape(batch, seq, d)
    mean = np.cumsum(xs, axis=1) / np.arange(1, seq + 1)[None, :, None]
    C = np.tile(mean.reshape(batch * seq, d), (1, heads))    # every head sees the same values
    np.testing.assert_allclose(got["Za"], C @ Ow, rtol=1e-12, atol=1e-12)


def test_block_equals_projections_around_the_core():
    """With C_i and dQKV_i taken from the core, the projection oracle
    (tp_attn_proj, which takes them as inputs) gives the block's outputs."""
    import oracle
    rng = np.random.default_rng(24)
    batch, seq, heads, d, h, p = 2, 5, 4, 2, 6, 2
    X, W, Ow, dZa = _block_inputs(rng, batch, seq, heads, d, h)
    g = tp_attn_block(X, W, Ow, dZa, p, batch, seq, heads, d=d)
    C = np.concatenate([g[f"C_{i}"] for i in range(p)], axis=1)
    dQKV = np.concatenate([g[f"dQKV_{i}"] for i in range(p)], axis=1)
    r = oracle.tp_attn_proj(X, W, C, Ow, dQKV, dZa, p)
    for k in r:
        np.testing.assert_allclose(g[k], r[k], rtol=1e-12, atol=1e-12)


def test_block_sampled_sequences_match_the_full_block():
    """The whole-sequence sample of the block equals those rows of the full block."""
    from oracle.sampled import attn_block_sampled
    rng = np.random.default_rng(25)
    batch, seq, heads, d, h, p = 4, 5, 2, 64, 8, 2
    X, W, Ow, dZa = _block_inputs(rng, batch, seq, heads, d, h)
    full = tp_attn_block(X, W, Ow, dZa, p, batch, seq, heads)
    seqs = [3, 1]
    rows = np.concatenate([np.arange(s * seq, (s + 1) * seq) for s in seqs])
    got = attn_block_sampled(X, W, Ow, dZa, p, batch, seq, heads, seqs)
    for k, v in got.items():
        ref = full[k][seqs] if k.startswith("lse_") else full[k][rows]
        np.testing.assert_allclose(v, ref, rtol=1e-12, atol=1e-13, err_msg=k)
    assert not any(k.startswith(("dW_", "dOw_")) for k in got)
