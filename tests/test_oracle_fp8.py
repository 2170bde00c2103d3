"""Pins of the FP8 oracle (oracle/fp8.py) against things other than itself:
PyTorch's CPU float8 types (decode of every code, encode of random values and
of every midpoint), a brute-force nearest search with ties to the even code,
exact integer arithmetic for the GEMM, closed forms of the scaling, and the
closed-form error of rounding to 3 or 2 significand bits."""
import numpy as np

import oracle
import pytest
import torch

from oracle import fp8 as F

TORCH = {F.E4M3: torch.float8_e4m3fn, F.E5M2: torch.float8_e5m2}
FMTS = [F.E4M3, F.E5M2]


def _torch_decode(codes, fmt):
    t = torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(TORCH[fmt])
    return t.to(torch.float64).numpy()


def _torch_encode(v32, fmt):
    return torch.from_numpy(np.asarray(v32, dtype=np.float32)).to(TORCH[fmt]).view(
        torch.uint8).numpy()


def _finite_table(fmt):
    codes = np.arange(256, dtype=np.uint8)
    vals = F.fp8_decode(codes, fmt)
    ok = np.isfinite(vals)
    return codes[ok], vals[ok]


@pytest.mark.parametrize("fmt", FMTS)
def test_decode_every_code_matches_torch(fmt):
    codes = np.arange(256, dtype=np.uint8)
    got, ref = F.fp8_decode(codes, fmt), _torch_decode(codes, fmt)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.nanmax(np.where(np.isinf(got), np.nan, got)) == F.fp8_max(fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_matches_torch_on_values_and_midpoints(fmt):
    rng = np.random.default_rng(5 + fmt)
    fmax = F.fp8_max(fmt)
    _, vals = _finite_table(fmt)
    pos = np.unique(vals[vals >= 0])
    mids = (pos[1:] + pos[:-1]) / 2          # exact in fp32: ties
    v = np.concatenate([pos, -pos, mids, -mids,
                        rng.uniform(-fmax, fmax, 20000),
                        rng.standard_normal(20000) * 1e-2,
                        np.ldexp(rng.uniform(-1, 1, 5000), -12)]).astype(np.float32)
    v = np.clip(v, -fmax, fmax)
    assert np.array_equal(F.fp8_encode(v.astype(np.float64), fmt), _torch_encode(v, fmt))


@pytest.mark.parametrize("fmt", FMTS)
def test_encode_is_nearest_with_ties_to_even(fmt):
    """Brute force: the code of the nearest finite value; of two equally
    near, the one with an even code."""
    rng = np.random.default_rng(11 + fmt)
    codes, vals = _finite_table(fmt)
    fmax = F.fp8_max(fmt)
    pos = np.unique(vals[vals > 0])
    v = np.concatenate([rng.uniform(-fmax, fmax, 3000), (pos[1:] + pos[:-1]) / 2,
                        rng.standard_normal(3000) * pos[3]])
    v = np.clip(v, -fmax, fmax)
    got = F.fp8_encode(v, fmt)
    for x, c in zip(v, got):
        d = np.abs(vals - x)
        cand = codes[d == d.min()]
        # the sign of a zero result follows x
        cand = [k for k in cand if (k & 0x80) == (0x80 if np.signbit(x) else 0)
                or F.fp8_decode(k, fmt) != 0]
        even = [k for k in cand if k % 2 == 0]
        want = even[0] if len(cand) > 1 else cand[0]
        assert c == want, (x, c, cand)


@pytest.mark.parametrize("fmt", FMTS)
def test_quantize_scaling(fmt):
    rng = np.random.default_rng(3)
    X = rng.standard_normal((37, 53)) * 3.0
    X[5, 7] = -np.max(np.abs(X)) * 1.5          # the amax element, negative
    q, s, sinv = F.quantize(X, fmt)
    fmax = F.fp8_max(fmt)
    assert F.fp8_decode(q[5, 7], fmt) == -fmax   # amax maps to -fmax exactly
    assert s == np.float32(fmax) / np.float32(np.abs(X[5, 7]))
    # scaling by a power of two leaves the codes and moves the factor
    q2, s2, sinv2 = F.quantize(X * 4.0, fmt)
    assert np.array_equal(q, q2) and s2 == s / 4 and sinv2 == sinv * 4
    # dequantised values are within half a quantum of X
    deq = F.fp8_decode(q, fmt) * float(sinv)
    rel = 2.0 ** -(4 if fmt == F.E4M3 else 3)     # half-ulp of the significand
    big = np.abs(X) > np.max(np.abs(X)) * 2.0 ** -6
    assert np.all(np.abs(deq - X)[big] <= rel * np.abs(X)[big] * 1.0001)
    # transpose gives the transposed codes; zeros give s = 1 and zero codes
    qt, _, _ = F.quantize(X, fmt, transpose=True)
    assert np.array_equal(qt, q.T)
    qz, sz, _ = F.quantize(np.zeros((4, 4)), fmt)
    assert sz == 1 and not qz.any()


@pytest.mark.parametrize("fa,fb", [(F.E4M3, F.E4M3), (F.E5M2, F.E4M3), (F.E4M3, F.E5M2)])
def test_gemm_exact_integer_arithmetic(fa, fb):
    """Every code value times 2^17 is an integer: the GEMM on those integers
    in Python's exact arithmetic, scaled back, equals the oracle exactly."""
    rng = np.random.default_rng(7)
    M, N, K = 5, 4, 70
    qa = rng.integers(0, 256, (M, K)).astype(np.uint8)
    qb = rng.integers(0, 256, (N, K)).astype(np.uint8)
    qa[np.isnan(F.fp8_decode(qa, fa)) | np.isinf(F.fp8_decode(qa, fa))] = 0x11
    qb[np.isnan(F.fp8_decode(qb, fb)) | np.isinf(F.fp8_decode(qb, fb))] = 0x22
    ia = [[int(F.fp8_decode(qa[m, k], fa) * 2 ** 17) for k in range(K)] for m in range(M)]
    ib = [[int(F.fp8_decode(qb[n, k], fb) * 2 ** 17) for k in range(K)] for n in range(N)]
    sa, sb = np.float32(0.375), np.float32(3.0)
    got = F.fp8_gemm(qa, qb, fa, fb, sa, sb)
    for m in range(M):
        for n in range(N):
            exact = sum(ia[m][k] * ib[n][k] for k in range(K))
            assert got[m, n] == exact / 2 ** 34 * 0.375 * 3.0


def test_linear_epilogues_closed_forms():
    rng = np.random.default_rng(9)
    qa, sa, ia = F.quantize(rng.standard_normal((6, 64)), F.E4M3)
    qb, sb, ib = F.quantize(rng.standard_normal((5, 64)), F.E4M3)
    C = F.fp8_gemm(qa, qb, 0, 0, ia, ib)
    assert np.array_equal(F.fp8_linear(qa, qb, 0, 0, ia, ib), C)
    # GeLU'(0) = 1/2
    assert np.allclose(F.fp8_linear(qa, qb, 0, 0, ia, ib, act="dgelu", U=np.zeros((6, 5))),
                       C / 2, rtol=0, atol=0)
    # a large positive bias makes GeLU the identity; U is the biased product
    Y, U = F.fp8_linear(qa, qb, 0, 0, ia, ib, bias=np.full(5, 50.0), act="gelu")
    assert np.allclose(U, C + 50.0) and np.allclose(Y, U, rtol=1e-12)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.integers(-6, 6, 50000),
                        [0.0, -0.0, 1.0, 65504.0, 1e-40]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.round_bf16(x), ref)


def rne_rel_rms(m):
    """RMS relative error of rounding to nearest with m stored significand
    bits, for values spread log-uniformly within a binade (as a Gaussian's
    are, over the few binades that hold most of its mass): the error is
    uniform on +-2^-m / 2 of the binade, so its RMS is 2^-m / sqrt(12) of it,
    and the value's significand 1 + f has density 1 / ((1 + f) ln 2), giving
    E[(1 + f)^-2] = (1/2 - 1/8) / ln 2."""
    return 2.0 ** -m / np.sqrt(12.0) * np.sqrt((0.5 - 0.125) / np.log(2.0))


@pytest.mark.parametrize("fmt,m", [(F.E4M3, 3), (F.E5M2, 2)])
def test_quantised_gemm_error_matches_the_rounding_closed_form(fmt, m):
    """Per-tensor current scaling then rounding to 3 (E4M3) or 2 (E5M2)
    significand bits: each element's relative error has the closed-form RMS
    above, and a product of two independently quantised Gaussian operands
    over a long K sums those errors in quadrature, sqrt(2) times it."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((256, 2048))
    w = rng.standard_normal((384, 2048))
    qx, _, ix = F.quantize(x, fmt)
    qw, _, iw = F.quantize(w, fmt)
    eps = rne_rel_rms(m)
    e_elem = oracle.rel_fro(F.fp8_decode(qx, fmt) * float(ix), x)
    assert 0.95 < e_elem / eps < 1.05, e_elem / eps
    e_gemm = oracle.rel_fro(F.fp8_gemm(qx, qw, fmt, fmt, ix, iw), x @ w.T)
    assert 0.95 < e_gemm / (np.sqrt(2.0) * eps) < 1.05, e_gemm / (np.sqrt(2.0) * eps)


@pytest.mark.parametrize("grad_fmt", [F.E4M3, F.E5M2])
def test_fp8_step_within_quantisation_error_of_exact_step(grad_fmt):
    """The FP8 step against the exact step, output by output, at the error
    the recipe predicts: activations and weights in E4M3 (eps4 per element),
    the gradients dZ and dU in grad_fmt (eps_g), errors of independent
    roundings adding in quadrature and carried forward by the products:

      U, Y   sqrt(2) eps4                        (X, A quantised)
      Zp, Z  sqrt(e_Y^2 + 2 eps4^2)              (Y's own error, Y and B quantised)
      dU, da sqrt(eps_g^2 + eps4^2)              (dZ and B quantised)
      dB     sqrt(e_Y^2 + eps4^2 + eps_g^2)      (Y carried and quantised, dZ quantised)
      dXp, dX, dA  sqrt(e_dU^2 + eps4^2 + eps_g^2)

    Each error must lie within [0.85, 1.2] of its prediction. E5M2 where the
    recipe has E4M3 doubles eps, and E4M3 where it has E5M2 halves eps_g, so
    either swap moves some output's error out of its band (by factors 0.65 to
    2); a transposed operand, a wrong shard or a misapplied scale gives errors
    of order one. db comes from the unquantised dZ and is exact."""
    exact, got = _fp8_step(grad_fmt)
    assert set(got) == set(exact)
    assert np.array_equal(got["db"], exact["db"])   # from the unquantised dZ
    assert _out_of_band(exact, got, grad_fmt) == []


def test_fp8_step_band_rejects_the_other_gradient_format():
    """The step run with one gradient format, held to the other format's
    prediction, leaves the band."""
    for run, claimed in ((F.E4M3, F.E5M2), (F.E5M2, F.E4M3)):
        exact, got = _fp8_step(run)
        assert len(_out_of_band(exact, got, claimed)) >= 5


def _fp8_step(grad_fmt):
    import dataclasses
    from tp_inputs import get_config, make_inputs
    cfg = dataclasses.replace(get_config("gpt2s"), micro_batch=1, seq=256, h=256)
    inputs = make_inputs(cfg)
    return oracle.run_config(cfg, inputs), F.run_config_fp8(cfg, inputs, grad_fmt)


def _out_of_band(exact, got, grad_fmt):
    """Outputs (other than db) whose error is outside [0.85, 1.2] x the
    prediction for this gradient format."""
    e4 = rne_rel_rms(3)
    eg = rne_rel_rms(3 if grad_fmt == F.E4M3 else 2)
    e_y = np.sqrt(2.0) * e4
    e_du = np.sqrt(eg ** 2 + e4 ** 2)
    pred = {"U": e_y, "Y": e_y, "Zp": np.sqrt(e_y ** 2 + 2 * e4 ** 2),
            "Z": np.sqrt(e_y ** 2 + 2 * e4 ** 2), "dU": e_du, "da": e_du,
            "dB": np.sqrt(e_y ** 2 + e4 ** 2 + eg ** 2),
            "dXp": np.sqrt(e_du ** 2 + e4 ** 2 + eg ** 2),
            "dX": np.sqrt(e_du ** 2 + e4 ** 2 + eg ** 2),
            "dA": np.sqrt(e_du ** 2 + e4 ** 2 + eg ** 2)}
    bad = []
    for k in exact:
        if k == "db":
            continue
        r = oracle.rel_fro(got[k], exact[k]) / pred[k.split("_")[0]]
        if not 0.85 < r < 1.2:
            bad.append((k, round(r, 3)))
    return bad
