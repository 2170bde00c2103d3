// Device helpers shared by the kernels: bf16 conversion, GeLU (tanh form) and
// its derivative, the per-element epilogue.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "internal.h"

namespace tpmlp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (lo = a, hi = b), round to nearest with ties to
// even, NaN stays NaN: one v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return static_cast<uint16_t>(pack_bf16x2(f, 0.0f) & 0xffffu);
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
// For |x| >= 1e4, g is exactly 0 or 1 in fp32, so g (1 - g) = 0 and the result
// is g; x is clamped there only so that x^2 stays finite (no 0 * inf).
__device__ __forceinline__ float gelu_tanh_grad(float x) {
  float xc = fminf(fmaxf(x, -1.0e4f), 1.0e4f);
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
    if (p.c2) store_elem(p.c2, row * p.ldc2 + col, v, p.out_bf16);
    store_elem(p.c, o, apply_act(p.act, v), p.out_bf16);
  } else if (p.epi == EPI_DACT) {
    float u = load_elem(p.u, row * p.ldu + col, in_bf16);
    if (p.c2) store_elem(p.c2, row * p.ldc2 + col, apply_act(p.act, u), p.out_bf16);
    store_elem(p.c, o, v * apply_act_grad(p.act, u), p.out_bf16);
  } else {
    if (p.accumulate && !p.out_bf16) v += static_cast<const float*>(p.c)[o];
    store_elem(p.c, o, v, p.out_bf16);
  }
}

// --------------------------------------------------------------------------
// Vector epilogue: 8 consecutive outputs (row, col .. col+7) of a bf16-operand
// GEMM, with 16-byte loads and stores. Valid when epilogue_vec_ok(p) holds and
// col is a multiple of 8 with col + 8 <= N.
// --------------------------------------------------------------------------
__device__ __forceinline__ bool aligned16(const void* ptr) {
  return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0;
}

__device__ __forceinline__ bool epilogue_vec_ok(const GemmParams& p) {
  return aligned16(p.c) && (p.ldc & 7) == 0 && (!p.c2 || (aligned16(p.c2) && (p.ldc2 & 7) == 0)) &&
         (!p.bias || aligned16(p.bias)) && (!p.u || (aligned16(p.u) && (p.ldu & 7) == 0));
}

typedef uint32_t ep_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load8_bf16(const void* base, int64_t off, float v[8]) {
  const ep_u32x4 w = *reinterpret_cast<const ep_u32x4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = __uint_as_float(w[q] << 16);
    v[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
  }
}

__device__ __forceinline__ void load8_f32(const void* base, int64_t off, float v[8]) {
  const float* s = static_cast<const float*>(base) + off;
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(s);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(s + 4);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[q] = a[q];
    v[q + 4] = b[q];
  }
}

__device__ __forceinline__ void store8(void* base, int64_t off, const float v[8], int is_bf16) {
  if (is_bf16) {
    *reinterpret_cast<ep_u32x4*>(static_cast<uint16_t*>(base) + off) =
        ep_u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])};
  } else {
    float* d = static_cast<float*>(base) + off;
    *reinterpret_cast<f32x4_t*>(d) = f32x4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4_t*>(d + 4) = f32x4_t{v[4], v[5], v[6], v[7]};
  }
}

__device__ __forceinline__ void epilogue_vec8(const GemmParams& p, int64_t row, int64_t col,
                                              float v[8]) {
  const int64_t o = row * p.ldc + col;
  if (p.epi == EPI_BIAS_ACT) {
    if (p.bias) {
      float b[8];
      load8_bf16(p.bias, col, b);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += b[q];
    }
    if (p.c2) store8(p.c2, row * p.ldc2 + col, v, p.out_bf16);
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = apply_act(p.act, v[q]);
    store8(p.c, o, v, p.out_bf16);
  } else if (p.epi == EPI_DACT) {
    float u[8];
    load8_bf16(p.u, row * p.ldu + col, u);
    if (p.c2) {
      float y[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) y[q] = apply_act(p.act, u[q]);
      store8(p.c2, row * p.ldc2 + col, y, p.out_bf16);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] *= apply_act_grad(p.act, u[q]);
    store8(p.c, o, v, p.out_bf16);
  } else {
    if (p.accumulate && !p.out_bf16) {
      float c[8];
      load8_f32(p.c, o, c);
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] += c[q];
    }
    store8(p.c, o, v, p.out_bf16);
  }
}

// Compile-time loop: f(std::integral_constant<int, i>) for i = I0 .. END-1.
template <int I0, int END>
struct Unroll {
  template <class F>
  __device__ __forceinline__ static void run(F&& f) {
    f(std::integral_constant<int, I0>{});
    Unroll<I0 + 1, END>::run(f);
  }
};
template <int END>
struct Unroll<END, END> {
  template <class F>
  __device__ __forceinline__ static void run(F&&) {}
};

}  // namespace tpmlp
