// Column-sum (bias-gradient) and split-K fix-up work units shared by the
// standalone kernels and the launches they ride along with: pass 1 runs in
// spare blocks of the weight-gradient GEMM, pass 2 and the fix-up in spare
// blocks of the fix-up launch or of the next layer's paired backward launch.
// Each unit is the same arithmetic in every launch, so the result does not
// depend on which launch carried it.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace tpmlp {

// Pass 1, vector path (N a multiple of 8, 16-byte aligned rows): unit (cb,
// chunk) covers 256 columns of rows [chunk*kColsumRows, +kColsumRows); thread
// (cv, rl) of the first 256 threads loads 8 columns (16 bytes of bf16, or 32
// of fp32) of rows rl, rl+8, .., all loads independent, and the 8 row lanes
// are added in order through LDS (part: 8 x 256 floats). Every thread of the
// block must call it (it synchronises the block twice).
__device__ __forceinline__ void colsum_vec_unit(const ColsumParams& p, int cb, int chunk,
                                                int nchunks, float (*part)[256]) {
  const int tid = threadIdx.x;
  if (tid < 256) {
    const int cv = tid & 31, rl = tid >> 5;
    const int64_t c0 = static_cast<int64_t>(cb) * 256 + cv * 8;
    const int64_t t0 = static_cast<int64_t>(chunk) * kColsumRows;
    float s[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) s[q] = 0.0f;
    if (c0 < p.N) {
#pragma unroll
      for (int j = 0; j < kColsumRows / 8; ++j) {
        const int64_t t = t0 + rl + 8 * j;
        if (t < p.T) {
          float v[8];
          if (p.src_bf16)
            load8_bf16(p.src, t * p.ld + c0, v);
          else
            load8_f32(p.src, t * p.ld + c0, v);
#pragma unroll
          for (int q = 0; q < 8; ++q) s[q] += v[q];
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) part[rl][cv * 8 + q] = s[q];
  }
  __syncthreads();
  if (tid < 256) {
    const int64_t cc = static_cast<int64_t>(cb) * 256 + tid;
    if (cc < p.N) {
      float v = part[0][tid];
#pragma unroll
      for (int r = 1; r < 8; ++r) v += part[r][tid];
      if (nchunks == 1)
        p.dbias[cc] = p.accumulate ? p.dbias[cc] + v : v;
      else
        p.ws[static_cast<int64_t>(chunk) * p.N + cc] = v;
    }
  }
  __syncthreads();  // part is reused by the next unit
}

// Pass 2: dbias[c] (+)= sum over chunks for the 64 columns of unit bx. Each
// column's chunks are split over 4 threads (chunks i, i+4, ...; loads
// independent) whose sums are added in order (part: 4 x 64 floats). Called by
// the first 256 threads of a block and all of them synchronise.
__device__ __forceinline__ void colsum_pass2_unit(const ColsumParams& p, int bx, int nchunks,
                                                  float (*part)[64]) {
  const int tid = threadIdx.x;
  if (tid < 256) {
    const int cl = tid & 63, pr = tid >> 6;
    const int64_t c = static_cast<int64_t>(bx) * 64 + cl;
    float s = 0.0f;
    if (c < p.N) {
#pragma unroll 16
      for (int i = pr; i < nchunks; i += 4) s += p.ws[static_cast<int64_t>(i) * p.N + c];
    }
    part[pr][cl] = s;
  }
  __syncthreads();
  if (tid < 64) {
    const int64_t c = static_cast<int64_t>(bx) * 64 + tid;
    if (c < p.N) {
      const float v = ((part[0][tid] + part[1][tid]) + part[2][tid]) + part[3][tid];
      p.dbias[c] = p.accumulate ? p.dbias[c] + v : v;
    }
  }
}

// Split-K fix-up, vector path (fp32 C, N and ldc multiples of 4, C and the
// partials 16-byte aligned): C (+)= the K slices' partials summed in slice
// order, four columns per thread. Thread `first` of `nthreads` takes every
// nthreads-th group of four.
__device__ __forceinline__ void splitk_fixup_vec4_unit(const GemmParams& p, int64_t first,
                                                       int64_t nthreads) {
  const int64_t nq = p.N >> 2;
  const int64_t total = p.M * nq;
  const int64_t slice = p.M * p.N;
  for (int64_t e = first; e < total; e += nthreads) {
    const int64_t row = e / nq, col = (e - row * nq) << 2;
    const float* w = p.ws + row * p.N + col;
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(w);
    for (int z = 1; z < p.splitk; ++z) v += *reinterpret_cast<const f32x4_t*>(w + z * slice);
    float* c = static_cast<float*>(p.c) + row * p.ldc + col;
    if (p.accumulate) v += *reinterpret_cast<const f32x4_t*>(c);
    *reinterpret_cast<f32x4_t*>(c) = v;
  }
}

}  // namespace tpmlp
