"""Pins of the CPU oracle to things other than itself (CPU only).

- hand-worked example with exact values (tests/golden/hand_worked_tp_mlp.json)
- brute force with exactly rounded sums and an independently written GeLU
- the column-split and row-split identities of the pages, and p-invariance
- GeLU closed forms, odd-part identity, asymptotes, library special case
- finite differences of the backward products, adjoint identities
- special cases that reduce the method to plain indexing
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from tp_inputs import get_config, make_inputs

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _lists(a):
    return np.asarray(a, np.float64).tolist()


# --------------------------------------------------------------------------- #
# Hand-worked example                                                          #
# --------------------------------------------------------------------------- #
def test_hand_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "hand_worked_tp_mlp.json")))
    f = lambda k: np.asarray(g[k], np.float64)  # noqa: E731
    out = oracle.tp_mlp(f("X"), f("A"), f("a"), f("B"), f("b"), f("dZ"), g["p"])
    exp = {k: np.asarray(v, np.float64) for k, v in g["expected"].items()}
    F = 4
    np.testing.assert_array_equal(np.concatenate([out["U_0"], out["U_1"]], 1), exp["U"])
    np.testing.assert_array_equal(np.concatenate([out["Y_0"], out["Y_1"]], 1), exp["Y"])
    np.testing.assert_array_equal(out["Zp_0"], exp["Zp_0"])
    np.testing.assert_array_equal(out["Zp_1"], exp["Zp_1"])
    np.testing.assert_array_equal(out["Z"], exp["Z"])
    np.testing.assert_array_equal(np.concatenate([out["dU_0"], out["dU_1"]], 1), exp["dU"])
    np.testing.assert_array_equal(np.concatenate([out["dB_0"], out["dB_1"]], 0), exp["dB"])
    np.testing.assert_array_equal(out["db"], exp["db"])
    np.testing.assert_array_equal(np.concatenate([out["dA_0"], out["dA_1"]], 1), exp["dA"])
    np.testing.assert_array_equal(np.concatenate([out["da_0"], out["da_1"]]), exp["da"])
    np.testing.assert_array_equal(out["dXp_0"], exp["dXp_0"])
    np.testing.assert_array_equal(out["dXp_1"], exp["dXp_1"])
    np.testing.assert_array_equal(out["dX"], exp["dX"])
    assert exp["U"].shape[1] == 2 * F


# --------------------------------------------------------------------------- #
# Brute force (exactly rounded sums, independent GeLU) on the tiny workload    #
# --------------------------------------------------------------------------- #
def test_brute_force_tiny_workload():
    cfg = get_config("tiny")
    inp = make_inputs(cfg)
    g = {k: v.f64() for k, v in inp.items()}
    ref = oracle.run_config(cfg, inp)
    bf = brute.mlp_step(_lists(g["X"]), _lists(g["A"]), _lists(g["a"]), _lists(g["B"]),
                        _lists(g["b"]), _lists(g["dZ"]), cfg.p)
    for k, v in bf.items():
        v = np.asarray(v)
        assert v.shape == ref[k].shape, k
        err = oracle.rel_fro(ref[k], v)
        assert err <= 1e-13, (k, err)
    # first-layer products of fp32 inputs are exact in float64 and fsum rounds
    # once: numpy's U may differ only by its own summation rounding
    np.testing.assert_allclose(ref["U_0"], bf["U_0"], rtol=1e-14, atol=1e-15)


def test_brute_force_random_nonzero_bias():
    rng = np.random.default_rng(11)
    T, h, p = 7, 3, 3
    X = rng.standard_normal((T, h))
    A = rng.standard_normal((h, 4 * h))
    a = rng.standard_normal(4 * h)
    B = rng.standard_normal((4 * h, h))
    b = rng.standard_normal(h)
    dZ = rng.standard_normal((T, h))
    ref = oracle.tp_mlp(X, A, a, B, b, dZ, p)
    bf = brute.mlp_step(_lists(X), _lists(A), _lists(a), _lists(B), _lists(b), _lists(dZ), p)
    for k, v in bf.items():
        assert oracle.rel_fro(ref[k], np.asarray(v)) <= 1e-13, k


# --------------------------------------------------------------------------- #
# Split identities of the pages                                                 #
# --------------------------------------------------------------------------- #
def _small_cfg_arrays(name, rows=None):
    cfg = get_config(name)
    inp = make_inputs(cfg)
    g = {k: v.f64() for k, v in inp.items()}
    if rows is not None:
        for k in ("X", "dZ", "C", "dQKV", "dZa"):
            if k in g:
                g[k] = g[k][:rows]
    return cfg, g


@pytest.mark.parametrize("name,rows", [("tiny", None), ("gpt2s", 256), ("gpt350m", 128)])
def test_column_and_row_split_identities(name, rows):
    cfg, g = _small_cfg_arrays(name, rows)
    sh = oracle.tp_mlp(g["X"], g["A"], g.get("a"), g["B"], g.get("b"), g["dZ"], cfg.p)
    un = oracle.mlp_unsharded(g["X"], g["A"], g.get("a"), g["B"], g.get("b"), g["dZ"])
    P = range(cfg.p)
    tol = 1e-12
    # column split: the concatenation of the shard outputs is the unsharded output
    assert oracle.rel_fro(np.concatenate([sh[f"U_{i}"] for i in P], 1), un["U"]) <= tol
    assert oracle.rel_fro(np.concatenate([sh[f"Y_{i}"] for i in P], 1), un["Y"]) <= tol
    assert oracle.rel_fro(np.concatenate([sh[f"dU_{i}"] for i in P], 1), un["dU"]) <= tol
    assert oracle.rel_fro(np.concatenate([sh[f"dA_{i}"] for i in P], 1), un["dA"]) <= tol
    if g.get("a") is not None:
        assert oracle.rel_fro(np.concatenate([sh[f"da_{i}"] for i in P]), un["da"]) <= tol
    # row split: stacked shard weight grads, summed partials
    assert oracle.rel_fro(np.concatenate([sh[f"dB_{i}"] for i in P], 0), un["dB"]) <= tol
    assert oracle.rel_fro(sh["Z"], un["Z"]) <= tol
    assert oracle.rel_fro(sh["dX"], un["dX"]) <= tol
    # every single partial is far from the sum when p > 1 (the sum is needed)
    assert oracle.rel_fro(sh["Zp_0"], un["Z"]) > 1e-3


def test_attention_split_identities():
    cfg, g = _small_cfg_arrays("attn", 128)
    sh = oracle.tp_attn_proj(g["X"], g["W"], g["C"], g["Ow"], g["dQKV"], g["dZa"], cfg.p)
    P = range(cfg.p)
    QKV = g["X"] @ g["W"]
    Za = g["C"] @ g["Ow"]
    assert oracle.rel_fro(np.concatenate([sh[f"QKV_{i}"] for i in P], 1), QKV) <= 1e-12
    assert oracle.rel_fro(sh["Za"], Za) <= 1e-12
    assert oracle.rel_fro(sh["dXq"], g["dQKV"] @ g["W"].T) <= 1e-12
    assert oracle.rel_fro(np.concatenate([sh[f"dW_{i}"] for i in P], 1), g["X"].T @ g["dQKV"]) <= 1e-12
    assert oracle.rel_fro(np.concatenate([sh[f"dC_{i}"] for i in P], 1), g["dZa"] @ g["Ow"].T) <= 1e-12
    assert oracle.rel_fro(np.concatenate([sh[f"dOw_{i}"] for i in P], 0), g["C"].T @ g["dZa"]) <= 1e-12


@pytest.mark.parametrize("p", [1, 2, 4, 8])
def test_p_invariance(p):
    """Every TP degree gives the same unsharded results (merging the shards of a
    checkpoint onto one device relies on this)."""
    rng = np.random.default_rng(5)
    T, h = 24, 8
    X, A, a = rng.standard_normal((T, h)), rng.standard_normal((h, 4 * h)), rng.standard_normal(4 * h)
    B, b, dZ = rng.standard_normal((4 * h, h)), rng.standard_normal(h), rng.standard_normal((T, h))
    base = oracle.tp_mlp(X, A, a, B, b, dZ, 1)
    sh = oracle.tp_mlp(X, A, a, B, b, dZ, p)
    for k in ("Z", "dX", "db"):
        assert oracle.rel_fro(sh[k], base[k]) <= 1e-12
    for k in ("U", "Y", "dU", "dA"):
        cat = np.concatenate([sh[f"{k}_{i}"] for i in range(p)], 1)
        assert oracle.rel_fro(cat, base[f"{k}_0"]) <= 1e-12
    cat = np.concatenate([sh[f"dB_{i}"] for i in range(p)], 0)
    assert oracle.rel_fro(cat, base["dB_0"]) <= 1e-12


# --------------------------------------------------------------------------- #
# GeLU                                                                         #
# --------------------------------------------------------------------------- #
def test_gelu_closed_forms():
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh_grad(0.0) == 0.5
    x = np.linspace(-8, 8, 2001)
    # the tanh factor is odd, so gelu(x) - gelu(-x) = x
    np.testing.assert_allclose(oracle.gelu_tanh(x) - oracle.gelu_tanh(-x), x, atol=1e-14)
    # asymptotes: gelu(x)/x -> 1 for x -> +inf, -> 0 for x -> -inf
    assert abs(oracle.gelu_tanh(30.0) / 30.0 - 1.0) < 1e-15
    assert abs(oracle.gelu_tanh(-30.0)) < 1e-15
    assert oracle.gelu_tanh_grad(30.0) == 1.0
    assert abs(oracle.gelu_tanh_grad(-30.0)) < 1e-15


def test_gelu_against_independent_forms():
    x = np.linspace(-10, 10, 4001)
    # logistic form, written independently in oracle/brute.py
    np.testing.assert_allclose(oracle.gelu_tanh(x), [brute.gelu(v) for v in x], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(oracle.gelu_tanh_grad(x), [brute.gelu_grad(v) for v in x], rtol=1e-12, atol=1e-14)
    # library special case: torch's tanh-approximate GeLU, float64 on the CPU
    t = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(x), t, rtol=1e-13, atol=1e-15)
    # the tanh form approximates the exact (erf) GeLU to about 5e-4 absolute
    erf = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in x])
    assert np.max(np.abs(oracle.gelu_tanh(x) - erf)) < 1e-3


def test_gelu_grad_is_derivative():
    x = np.linspace(-6, 6, 1201)
    eps = 1e-6
    fd = (oracle.gelu_tanh(x + eps) - oracle.gelu_tanh(x - eps)) / (2 * eps)
    np.testing.assert_allclose(oracle.gelu_tanh_grad(x), fd, rtol=1e-7, atol=1e-8)


# --------------------------------------------------------------------------- #
# Backward: finite differences and adjoint identities                          #
# --------------------------------------------------------------------------- #
def _fd_grad(loss, x, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        lp = loss()
        x[i] = old - eps
        lm = loss()
        x[i] = old
        g[i] = (lp - lm) / (2 * eps)
    return g


def test_mlp_backward_finite_differences():
    rng = np.random.default_rng(3)
    T, h, p = 6, 4, 2
    X, A, a = rng.standard_normal((T, h)), rng.standard_normal((h, 4 * h)) * 0.5, rng.standard_normal(4 * h) * 0.3
    B, b, dZ = rng.standard_normal((4 * h, h)), rng.standard_normal(h), rng.standard_normal((T, h))

    def loss():
        return float(np.sum(dZ * oracle.tp_mlp(X, A, a, B, b, dZ, p)["Z"]))

    out = oracle.tp_mlp(X, A, a, B, b, dZ, p)
    P = range(p)
    analytic = {
        "X": out["dX"],
        "A": np.concatenate([out[f"dA_{i}"] for i in P], 1),
        "a": np.concatenate([out[f"da_{i}"] for i in P]),
        "B": np.concatenate([out[f"dB_{i}"] for i in P], 0),
        "b": out["db"],
    }
    for name, arr in (("X", X), ("A", A), ("a", a), ("B", B), ("b", b)):
        fd = _fd_grad(loss, arr)
        np.testing.assert_allclose(analytic[name], fd, rtol=1e-6, atol=1e-7, err_msg=name)
    # dU is the gradient of the loss with respect to the pre-activation U
    U = np.concatenate([out[f"U_{i}"] for i in P], 1)
    dU = np.concatenate([out[f"dU_{i}"] for i in P], 1)

    def loss_u():
        return float(np.sum(dZ * (oracle.gelu_tanh(U) @ B + b)))

    np.testing.assert_allclose(dU, _fd_grad(loss_u, U), rtol=1e-6, atol=1e-7)


def test_attention_backward_finite_differences():
    rng = np.random.default_rng(4)
    T, h, p = 5, 4, 2
    X, W = rng.standard_normal((T, h)), rng.standard_normal((h, 3 * h))
    C, Ow = rng.standard_normal((T, h)), rng.standard_normal((h, h))
    dQKV, dZa = rng.standard_normal((T, 3 * h)), rng.standard_normal((T, h))

    def loss():
        o = oracle.tp_attn_proj(X, W, C, Ow, dQKV, dZa, p)
        qkv = np.concatenate([o[f"QKV_{i}"] for i in range(p)], 1)
        return float(np.sum(dZa * o["Za"]) + np.sum(dQKV * qkv))

    out = oracle.tp_attn_proj(X, W, C, Ow, dQKV, dZa, p)
    np.testing.assert_allclose(out["dXq"], _fd_grad(loss, X), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(np.concatenate([out[f"dW_{i}"] for i in range(p)], 1),
                               _fd_grad(loss, W), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(np.concatenate([out[f"dC_{i}"] for i in range(p)], 1),
                               _fd_grad(loss, C), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(np.concatenate([out[f"dOw_{i}"] for i in range(p)], 0),
                               _fd_grad(loss, Ow), rtol=1e-6, atol=1e-7)


def test_adjoint_identities():
    """<dOut, In W> = <dgrad(dOut, W), In> = <wgrad(In, dOut), W>."""
    rng = np.random.default_rng(9)
    In, W, dOut = rng.standard_normal((13, 5)), rng.standard_normal((5, 7)), rng.standard_normal((13, 7))
    fwd = np.sum(dOut * (In @ W))
    dIn = oracle.linear_bwd_dgrad(dOut, W)
    dW, dc = oracle.linear_bwd_wgrad(In, dOut)
    assert abs(np.sum(dIn * In) - fwd) <= 1e-12 * abs(fwd) + 1e-12
    assert abs(np.sum(dW * W) - fwd) <= 1e-12 * abs(fwd) + 1e-12
    # bias: <dOut, 1 c^T> = <colsum(dOut), c>
    c = rng.standard_normal(7)
    assert abs(np.sum(dOut * c[None, :]) - np.dot(dc, c)) <= 1e-12


# --------------------------------------------------------------------------- #
# Special cases                                                                #
# --------------------------------------------------------------------------- #
def test_special_cases():
    rng = np.random.default_rng(21)
    T, h, p = 9, 4, 2
    X, A, a = rng.standard_normal((T, h)), rng.standard_normal((h, 4 * h)), rng.standard_normal(4 * h)
    B, b, dZ = rng.standard_normal((4 * h, h)), rng.standard_normal(h), rng.standard_normal((T, h))
    # B = 0  =>  Z = b on every token, and dU = 0
    o = oracle.tp_mlp(X, A, a, np.zeros_like(B), b, dZ, p)
    np.testing.assert_array_equal(o["Z"], np.tile(b, (T, 1)))
    assert not np.any(o["dU_0"]) and not np.any(o["dU_1"])
    # X = 0  =>  U = a, Y = gelu(a), dA = 0
    o = oracle.tp_mlp(np.zeros_like(X), A, a, B, b, dZ, p)
    np.testing.assert_array_equal(np.concatenate([o["U_0"], o["U_1"]], 1), np.tile(a, (T, 1)))
    assert not np.any(o["dA_0"])
    # one-hot columns of A pick columns of X: U_i[:, j] = X[:, sel[j]]
    sel = rng.integers(0, h, 4 * h)
    onehot = np.zeros((h, 4 * h))
    onehot[sel, np.arange(4 * h)] = 1.0
    o = oracle.tp_mlp(X, onehot, None, B, None, dZ, p)
    np.testing.assert_array_equal(np.concatenate([o["U_0"], o["U_1"]], 1), X[:, sel])
    # identity output projection (pO = h): Za = C
    C = rng.standard_normal((T, h))
    o = oracle.tp_attn_proj(X, rng.standard_normal((h, 3 * h)), C, np.eye(h),
                            rng.standard_normal((T, 3 * h)), dZ, p)
    np.testing.assert_array_equal(o["Za"], C)


def test_rel_fro_and_sampled_dot():
    rng = np.random.default_rng(2)
    L, R = rng.standard_normal((11, 6)), rng.standard_normal((6, 9))
    full = L @ R
    rows, cols = rng.integers(0, 11, 20), rng.integers(0, 9, 20)
    np.testing.assert_allclose(oracle.sampled_dot(L, R, rows, cols), full[rows, cols], rtol=1e-13)
    # transposed operands
    np.testing.assert_allclose(oracle.sampled_dot(L.T.copy(), R, rows, cols, transpose_left=True),
                               full[rows, cols], rtol=1e-13)
    np.testing.assert_allclose(oracle.sampled_dot(L, R.T.copy(), rows, cols, transpose_right=True),
                               full[rows, cols], rtol=1e-13)
    assert oracle.rel_fro(full, full) == 0.0
    assert abs(oracle.rel_fro(full * 1.01, full) - 0.01) < 1e-12
