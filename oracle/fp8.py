"""CPU oracle of the FP8 variant of the shard GEMMs (float64 arithmetic).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. It shares no code
with the HIP path and imports nothing from it.

Source: the "Megatron" page (zzmblog.top), "mixed-precision training": besides
FP16/BF16 the framework trains in FP8 on Hopper GPUs; the "Megatron-LM
quick-start" page (blog.gitcode.com), "performance optimisation", recommends
mixed precision such as FP8. The pages fix neither the format nor the scaling.
Readings:

  * formats: the OCP 8-bit floats E4M3 (exponent bias 7, 3 mantissa bits, no
    infinities, largest finite 448) and E5M2 (bias 15, 2 mantissa bits,
    largest finite 57344); subnormals included;
  * per-tensor current scaling: s = fmax / amax(X), computed in fp32
    (s = 1 when X is all zeros); a code is the nearest format value, ties to
    even, of the fp32 product fp32(x) * s clamped to [-fmax, fmax]. The
    quantised decision is taken in fp32, as on the device;
  * the dequantisation factor is 1/s in fp32;
  * an FP8 GEMM of codes qa [M, K] and qb [N, K] (both K-contiguous) is
    C = (sum_k dec(qa[m, k]) dec(qb[n, k])) * (1/sa) * (1/sb), followed by the
    same epilogues as the bf16 GEMMs (bias + GeLU saving U, GeLU' of a saved U,
    plain store).

Pins (tests/test_oracle_fp8.py): the decoder against PyTorch's CPU float8
types on every code; the encoder against PyTorch's conversion (random values,
every format value and every midpoint) and against a brute-force nearest
search over all finite values with ties to the even code; the scaling by the
amax element, power-of-two invariance and the half-quantum error bound; the
GEMM against exact integer arithmetic on scaled code values; the epilogues by
closed forms (GeLU'(0) = 1/2, GeLU the identity for large inputs).
"""
from __future__ import annotations

import numpy as np

from .oracle import gelu_tanh, gelu_tanh_grad

E4M3, E5M2 = 0, 1
_FMT = {E4M3: (4, 3, 7), E5M2: (5, 2, 15)}  # exponent bits, mantissa bits, bias


def fp8_max(fmt: int) -> float:
    """Largest finite value: 448 (E4M3, whose all-ones exponent still holds
    normal numbers except mantissa 111) or 57344 (E5M2, IEEE-like)."""
    return 448.0 if fmt == E4M3 else 57344.0


def fp8_decode(codes, fmt: int) -> np.ndarray:
    """Exact value of each 8-bit code (NaN codes decode to NaN, E5M2's
    infinity codes to +-inf)."""
    ebits, mbits, bias = _FMT[fmt]
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> mbits) & ((1 << ebits) - 1)
    m = (c & ((1 << mbits) - 1)).astype(np.float64)
    normal = np.ldexp(1.0 + m / (1 << mbits), e - bias)
    sub = np.ldexp(m / (1 << mbits), 1 - bias)
    v = sign * np.where(e == 0, sub, normal)
    if fmt == E4M3:
        v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    else:
        top = e == (1 << ebits) - 1
        v = np.where(top & (m == 0), sign * np.inf, v)
        v = np.where(top & (m != 0), np.nan, v)
    return v


def fp8_encode(v, fmt: int) -> np.ndarray:
    """Codes of values already in [-fmax, fmax]: round to the nearest format
    value, ties to even. Arithmetic form: with e the binade of |v| (at least
    the smallest normal binade), the quantum is 2^(e - mbits) and the rounded
    significand is rint(|v| / quantum) (numpy rounds half to even); a carry
    into the next binade is folded back into the exponent field."""
    ebits, mbits, bias = _FMT[fmt]
    x = np.asarray(v, dtype=np.float64)
    assert np.all(np.abs(x) <= fp8_max(fmt)), "fp8_encode: value out of range"
    a = np.abs(x)
    _, ex = np.frexp(a)                  # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, 1 - bias)     # binade, clamped to the subnormal one
    q = np.rint(np.ldexp(a, mbits - e))  # significand in quanta, 0 .. 2^(mbits+1)
    carry = q >= (1 << (mbits + 1))
    e = np.where(carry, e + 1, e)
    q = np.where(carry, q / 2, q).astype(np.int64)
    normal = q >= (1 << mbits)
    efield = np.where(normal, e + bias, 0)
    mfield = np.where(normal, q - (1 << mbits), q)
    code = (efield << mbits) | mfield
    code = np.where(np.signbit(x), code | 0x80, code)  # the sign of zero is kept
    return code.astype(np.uint8)


def quantize(X, fmt: int, transpose: bool = False):
    """Per-tensor current scaling of X (exact stored values). Returns the
    codes (of X, or of X^T when transpose), the fp32 scale s and the fp32
    dequantisation factor 1/s."""
    x32 = np.asarray(X, dtype=np.float64).astype(np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    fmax = np.float32(fp8_max(fmt))
    s = fmax / amax if amax > 0 else np.float32(1.0)
    s = np.float32(s)
    v = np.clip(x32 * s, -fmax, fmax)    # fp32 product, then clamp
    codes = fp8_encode(v.astype(np.float64), fmt)
    if transpose:
        codes = np.ascontiguousarray(codes.T)
    return codes, s, np.float32(np.float32(1.0) / s)


def fp8_gemm(qa, qb, fmt_a: int, fmt_b: int, sinv_a, sinv_b) -> np.ndarray:
    """C[M, N] = sum_k dec(qa[m, k]) dec(qb[n, k]) * sinv_a * sinv_b."""
    A = fp8_decode(qa, fmt_a)
    B = fp8_decode(qb, fmt_b)
    return (A @ B.T) * float(sinv_a) * float(sinv_b)


def fp8_linear(qa, qb, fmt_a, fmt_b, sinv_a, sinv_b, bias=None, act="none", U=None):
    """The GEMM and its epilogue.
    act == "gelu", U None: returns (Y, Upre) with Upre = C + bias, Y = GeLU(Upre);
    act == "dgelu": returns C * GeLU'(U) for a saved pre-activation U;
    otherwise C (+ bias)."""
    C = fp8_gemm(qa, qb, fmt_a, fmt_b, sinv_a, sinv_b)
    if act == "dgelu":
        return C * gelu_tanh_grad(np.asarray(U, dtype=np.float64))
    if bias is not None:
        C = C + np.asarray(bias, dtype=np.float64)[None, :]
    if act == "gelu":
        return gelu_tanh(C), C
    return C


def round_bf16(x) -> np.ndarray:
    """x rounded to fp32 (nearest even), then to bf16 (nearest even on the
    upper 16 bits): the storage of the recipe's bf16 intermediates."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def tp_mlp_fp8(X, A, a, B, b, dZ, p, shards=None, weights_are_shards=False, grad_fmt=E5M2):
    """One fwd+bwd step of the MLP shard with every product in FP8: weights and
    activations in E4M3, gradients in grad_fmt, each operand quantised from its
    stored value (inputs as given; U_i, Y_i, dU_i rounded to bf16, the storage
    precision of the bf16 path) with its own current scale, in the layout its
    product reads (K-contiguous). Bias gradients are column sums of the stored
    gradients. Outputs are named as in oracle.tp_mlp."""
    shards = tuple(range(p)) if shards is None else tuple(shards)
    g = grad_fmt
    X = np.asarray(X, np.float64)
    dZ = np.asarray(dZ, np.float64)
    qX, _, sX = quantize(X, E4M3)
    qXt, _, sXt = quantize(X, E4M3, transpose=True)
    qD, _, sD = quantize(dZ, g)
    qDt, _, sDt = quantize(dZ, g, transpose=True)
    out, Zp, dXp = {}, [], []
    F = np.asarray(A).shape[1] if weights_are_shards else np.asarray(A).shape[1] // p
    for i in shards:
        if weights_are_shards:
            A_i, B_i, a_i = A, B, a
        else:
            A_i, B_i = A[:, i * F:(i + 1) * F], B[i * F:(i + 1) * F]
            a_i = None if a is None else a[i * F:(i + 1) * F]
        qAt, _, sAt = quantize(A_i, E4M3, transpose=True)
        Y, U = fp8_linear(qX, qAt, E4M3, E4M3, sX, sAt, bias=a_i, act="gelu")
        U16, Y16 = round_bf16(U), round_bf16(Y)
        qY, _, sY = quantize(Y16, E4M3)
        qBt, _, sBt = quantize(B_i, E4M3, transpose=True)
        Zp_i = fp8_linear(qY, qBt, E4M3, E4M3, sY, sBt)
        qB, _, sB = quantize(B_i, E4M3)
        dU = fp8_linear(qD, qB, g, E4M3, sD, sB, act="dgelu", U=U16)
        dU16 = round_bf16(dU)
        qYt, _, sYt = quantize(Y16, E4M3, transpose=True)
        dB = fp8_linear(qYt, qDt, E4M3, g, sYt, sDt)
        qdU, _, sdU = quantize(dU16, g)
        qA, _, sA = quantize(A_i, E4M3)
        dXp_i = fp8_linear(qdU, qA, g, E4M3, sdU, sA)
        qdUt, _, sdUt = quantize(dU16, g, transpose=True)
        dA = fp8_linear(qXt, qdUt, E4M3, g, sXt, sdUt)
        out.update({f"U_{i}": U, f"Y_{i}": Y, f"Zp_{i}": Zp_i, f"dU_{i}": dU,
                    f"dB_{i}": dB, f"dA_{i}": dA, f"dXp_{i}": dXp_i})
        if a is not None:
            out[f"da_{i}"] = dU16.sum(axis=0)
        Zp.append(Zp_i)
        dXp.append(dXp_i)
    if b is not None:
        out["db"] = dZ.sum(axis=0)
    if len(shards) == p:
        Z = Zp[0].copy()
        for z in Zp[1:]:
            Z = Z + z
        out["Z"] = Z + (0.0 if b is None else np.asarray(b, np.float64)[None, :])
        dX = dXp[0].copy()
        for d in dXp[1:]:
            dX = dX + d
        out["dX"] = dX
    return out


def run_config_fp8(cfg, inputs, grad_fmt=E5M2) -> dict:
    """tp_mlp_fp8 on a workload's inputs (MLP workloads)."""
    g = {k: v.f64() for k, v in inputs.items()}
    return tp_mlp_fp8(g["X"], g["A"], g.get("a"), g["B"], g.get("b"), g["dZ"], cfg.p,
                      cfg.shards, weights_are_shards=not cfg.full_weights, grad_fmt=grad_fmt)
