// Device helpers shared by the kernels: bf16 conversion, GeLU (tanh form) and
// its derivative, the per-element epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace tpmlp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest with ties to even; a NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Two fp32 -> packed bf16 pair (lo = a, hi = b).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// GeLU, tanh form: 0.5 x (1 + tanh(s)), s = sqrt(2/pi) (x + 0.044715 x^3)
// (Hendrycks & Gimpel). Since (1 + tanh s)/2 is the logistic function of 2s,
// it is evaluated as x / (1 + exp(-2s)), which saturates cleanly at both ends.
constexpr float kSqrt2OverPi = 0.7978845608028654f;
constexpr float kGeluCubic = 0.044715f;

__device__ __forceinline__ float gelu_tanh(float x) {
  float s = kSqrt2OverPi * fmaf(kGeluCubic * x, x * x, x);
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * s));
}

// d/dx of gelu_tanh. With g = 1/(1 + exp(-2s)):
//   gelu'(x) = g + x * 2 g (1 - g) * s'(x),  s'(x) = sqrt(2/pi) (1 + 3 * 0.044715 x^2).
// For |x| >= 10, g is 0 or 1 to fp32 precision; x is clamped there so that the
// cubic cannot overflow (the result is then 0 or 1 up to ~1e-35).
__device__ __forceinline__ float gelu_tanh_grad(float x) {
  float xc = fminf(fmaxf(x, -10.0f), 10.0f);
  float x2 = xc * xc;
  float s = kSqrt2OverPi * fmaf(kGeluCubic * xc, x2, xc);
  float g = __builtin_amdgcn_rcpf(1.0f + __expf(-2.0f * s));
  float ds = kSqrt2OverPi * fmaf(3.0f * kGeluCubic, x2, 1.0f);
  float r = fmaf(2.0f * xc * ds, g * (1.0f - g), g);
  return (x != x) ? x : r;  // NaN in, NaN out
}

__device__ __forceinline__ float apply_act(int act, float x) {
  return act == ACT_GELU ? gelu_tanh(x) : x;
}

__device__ __forceinline__ float apply_act_grad(int act, float x) {
  return act == ACT_GELU ? gelu_tanh_grad(x) : 1.0f;
}

// Load element i of an array that is bf16 (is_bf16) or fp32.
__device__ __forceinline__ float load_elem(const void* p, int64_t i, int is_bf16) {
  return is_bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i])
                 : static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void store_elem(void* p, int64_t i, float v, int is_bf16) {
  if (is_bf16)
    static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
  else
    static_cast<float*>(p)[i] = v;
}

// The epilogue for one output element (row, col) of a GEMM with accumulator v.
// in_bf16: dtype of the operands, which is also the dtype of bias and U.
__device__ __forceinline__ void epilogue_elem(const GemmParams& p, int64_t row, int64_t col,
                                              float v, int in_bf16) {
  const int64_t o = row * p.ldc + col;
  if (p.epi == EPI_BIAS_ACT) {
    if (p.bias) v += load_elem(p.bias, col, in_bf16);
    if (p.c2) store_elem(p.c2, o, v, p.out_bf16);
    store_elem(p.c, o, apply_act(p.act, v), p.out_bf16);
  } else if (p.epi == EPI_DACT) {
    float u = load_elem(p.u, row * p.ldu + col, in_bf16);
    store_elem(p.c, o, v * apply_act_grad(p.act, u), p.out_bf16);
  } else {
    if (p.accumulate && !p.out_bf16) v += static_cast<const float*>(p.c)[o];
    store_elem(p.c, o, v, p.out_bf16);
  }
}

}  // namespace tpmlp
