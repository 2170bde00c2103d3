"""Pins of the FP8 oracle (oracle/fp8.py) against things other than itself:
PyTorch's CPU float8 types (decode of every code, encode of random values and
of every midpoint), a brute-force nearest search with ties to the even code,
exact integer arithmetic for the GEMM, and closed forms of the scaling."""
import numpy as np
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


@pytest.mark.parametrize("grad_fmt", [F.E4M3, F.E5M2])
def test_fp8_step_within_quantisation_error_of_exact_step(grad_fmt):
    """The FP8 step approximates the exact step: every output within the error
    that 3-bit (2-bit) significands allow (about 2^-4 (2^-3) per element,
    averaging down in the products), and visibly different from it (so the
    quantisation really took place). A transposed operand, a wrong shard or a
    misapplied scale gives errors of order one."""
    import dataclasses
    import oracle
    from tp_inputs import get_config, make_inputs
    cfg = dataclasses.replace(get_config("gpt2s"), micro_batch=1, seq=256, h=256)
    inputs = make_inputs(cfg)
    exact = oracle.run_config(cfg, inputs)
    got = F.run_config_fp8(cfg, inputs, grad_fmt)
    assert set(got) == set(exact)
    bound = 0.12 if grad_fmt == F.E5M2 else 0.08
    for k in exact:
        if k == "db":
            assert np.array_equal(got[k], exact[k])   # from the unquantised dZ
            continue
        e = oracle.rel_fro(got[k], exact[k])
        assert 1e-3 < e < bound, (k, e)
