// FP8 quantisation with per-tensor current scaling: s = fmax / amax(X) in fp32,
// codes = nearest E4M3 / E5M2 value (ties to even) of clamp(x * s, +-fmax),
// and the dequantisation factor 1/s written to device memory, so a step never
// waits on the host. Two launches, both deterministic (a maximum does not
// depend on order): per-block maxima of |x|, then a cast in which every block
// first reduces those maxima itself. The cast writes X's codes in X's layout,
// or X^T's (through a 64x64 LDS tile) for operands the FP8 GEMM needs
// K-contiguous.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace tpmlp {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float fp8_fmax(int fmt) { return fmt == 0 ? 448.0f : 57344.0f; }

// 8 consecutive elements of row `row` from column c0 (bf16 or fp32); elements
// at or past `cols` read as 0.
__device__ __forceinline__ void load8_any(const Fp8QuantParams& p, int64_t row, int64_t c0,
                                          float v[8]) {
  const int64_t off = row * p.ld_x + c0;
  if (p.vec_in && c0 + 8 <= p.cols) {
    if (p.x_bf16) load8_bf16(p.x, off, v);
    else load8_f32(p.x, off, v);
    return;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e)
    v[e] = c0 + e < p.cols ? load_elem(p.x, off + e, p.x_bf16) : 0.0f;
}

__device__ __forceinline__ float block_max(float m, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; ++w) m = fmaxf(m, red[w]);
  __syncthreads();
  return m;
}

// Per-block maxima of |x|: block `block` of the tensor's `nblocks`.
__device__ __forceinline__ void fp8_amax_block(const Fp8QuantParams& p, int block, int nblocks) {
  __shared__ float red[kThreads / 64];
  const int64_t ucols = (p.cols + 7) / 8, units = p.rows * ucols;
  float m = 0.0f;
  for (int64_t u = static_cast<int64_t>(block) * kThreads + threadIdx.x; u < units;
       u += static_cast<int64_t>(nblocks) * kThreads) {
    const int64_t row = u / ucols, c0 = (u - row * ucols) * 8;
    float v[8];
    load8_any(p, row, c0, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  }
  m = block_max(m, red);
  if (threadIdx.x == 0) p.partial[block] = m;
}

__global__ __launch_bounds__(kThreads) void fp8_amax_kernel(Fp8QuantParams p) {
  fp8_amax_block(p, blockIdx.x, gridDim.x);
}

// Four codes of v[0..3] packed little-endian (v[0] in the low byte).
__device__ __forceinline__ uint32_t cvt4(const float* v, float s, float fmax, int fmt) {
  float c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) c[e] = fminf(fmaxf(v[e] * s, -fmax), fmax);
  int w;
  if (fmt == 0) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c[0], c[1], 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c[2], c[3], w, true);
  }
  return static_cast<uint32_t>(w);
}

// amax from the per-block maxima, the scale, and (block 0) 1/s to memory
__device__ __forceinline__ float fp8_scale(const Fp8QuantParams& p, float* red, int block) {
  float m = 0.0f;
  for (int i = threadIdx.x; i < p.nblk; i += kThreads) m = fmaxf(m, p.partial[i]);
  m = block_max(m, red);
  const float s = m > 0.0f ? fp8_fmax(p.fmt) / m : 1.0f;
  if (block == 0 && threadIdx.x == 0) p.scale_inv[0] = 1.0f / s;
  return s;
}

__global__ __launch_bounds__(kThreads) void fp8_cast_kernel(Fp8QuantParams p) {
  __shared__ float red[kThreads / 64];
  const float s = fp8_scale(p, red, blockIdx.x), fmax = fp8_fmax(p.fmt);
  const int64_t ucols = (p.cols + 7) / 8, units = p.rows * ucols;
  for (int64_t u = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; u < units;
       u += static_cast<int64_t>(gridDim.x) * kThreads) {
    const int64_t row = u / ucols, c0 = (u - row * ucols) * 8;
    float v[8];
    load8_any(p, row, c0, v);
    const uint32_t lo = cvt4(v, s, fmax, p.fmt), hi = cvt4(v + 4, s, fmax, p.fmt);
    uint8_t* q = p.q + row * p.ld_q + c0;
    if (p.vec_out && c0 + 8 <= p.cols) {
      *reinterpret_cast<uint2*>(q) = uint2{lo, hi};
    } else {
      for (int e = 0; e < 8 && c0 + e < p.cols; ++e)
        q[e] = static_cast<uint8_t>((e < 4 ? lo >> (8 * e) : hi >> (8 * (e - 4))) & 0xff);
    }
  }
}

// Transposed cast: Q[c, r] = code(X[r, c]) through 64x64 tiles. Load: thread t
// converts row t/4, columns 16*(t%4) .. +15 of the tile and writes the 16 codes
// to LDS row-major; store: thread t gathers column t/4, rows 16*(t%4) .. +15 and
// writes them as one 16-byte row piece of Q.
constexpr int kTT = 64;
constexpr int kTStride = 80;  // bytes per LDS row: 16-byte aligned, rows spread over banks

// Block `block` of the tensor's `nblocks`.
__device__ __forceinline__ void fp8_cast_t_block(const Fp8QuantParams& p, int block, int nblocks) {
  __shared__ float red[kThreads / 64];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kTT * kTStride];
  const float s = fp8_scale(p, red, block), fmax = fp8_fmax(p.fmt);
  const int64_t tr = (p.rows + kTT - 1) / kTT, tc = (p.cols + kTT - 1) / kTT;
  const int t = threadIdx.x, lr = t / 4, lc = 16 * (t % 4);
  for (int64_t b = block; b < tr * tc; b += nblocks) {
    const int64_t r0 = (b / tc) * kTT, c0 = (b % tc) * kTT;
    const int64_t row = r0 + lr;
    float v[16];
    if (row < p.rows) {
      load8_any(p, row, c0 + lc, v);
      load8_any(p, row, c0 + lc + 8, v + 8);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = 0.0f;
    }
    uint4 w;
    w.x = cvt4(v, s, fmax, p.fmt);
    w.y = cvt4(v + 4, s, fmax, p.fmt);
    w.z = cvt4(v + 8, s, fmax, p.fmt);
    w.w = cvt4(v + 12, s, fmax, p.fmt);
    *reinterpret_cast<uint4*>(tile + lr * kTStride + lc) = w;
    if (p.q_rows && row < p.rows) {  // the codes of X itself, from the same read
      const int64_t c = c0 + lc;
      uint8_t* qr = p.q_rows + row * p.ld_q_rows + c;
      if (p.vec_rows && c + 16 <= p.cols) {
        *reinterpret_cast<uint4*>(qr) = w;
      } else {
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        for (int e = 0; e < 16 && c + e < p.cols; ++e)
          qr[e] = static_cast<uint8_t>((ww[e / 4] >> (8 * (e % 4))) & 0xff);
      }
    }
    __syncthreads();
    // output row c = c0 + lr of Q, entries r0 + lc .. r0 + lc + 15
    const int64_t qrow = c0 + lr, qc = r0 + lc;
    if (qrow < p.cols) {
      uint32_t o[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t x = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) x |= static_cast<uint32_t>(tile[(lc + 4 * g + e) * kTStride + lr]) << (8 * e);
        o[g] = x;
      }
      uint8_t* q = p.q + qrow * p.ld_q + qc;
      if (p.vec_out && qc + 16 <= p.rows) {
        *reinterpret_cast<uint4*>(q) = uint4{o[0], o[1], o[2], o[3]};
      } else {
        for (int e = 0; e < 16 && qc + e < p.rows; ++e)
          q[e] = static_cast<uint8_t>((o[e / 4] >> (8 * (e % 4))) & 0xff);
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void fp8_cast_t_kernel(Fp8QuantParams p) {
  fp8_cast_t_block(p, blockIdx.x, gridDim.x);
}

// Several tensors in one launch: tensor i owns blocks first[i] .. first[i+1]-1.
__device__ __forceinline__ int fp8_multi_tensor(const Fp8MultiParams& m) {
  int i = 0;
  while (i + 1 < m.n && static_cast<int>(blockIdx.x) >= m.first[i + 1]) ++i;
  return i;
}

__global__ __launch_bounds__(kThreads) void fp8_amax_multi_kernel(Fp8MultiParams m) {
  const int i = fp8_multi_tensor(m);
  const Fp8QuantParams p = m.t[i];
  fp8_amax_block(p, blockIdx.x - m.first[i], m.first[i + 1] - m.first[i]);
}

__global__ __launch_bounds__(kThreads) void fp8_cast_t_multi_kernel(Fp8MultiParams m) {
  const int i = fp8_multi_tensor(m);
  const Fp8QuantParams p = m.t[i];
  fp8_cast_t_block(p, blockIdx.x - m.first[i], m.first[i + 1] - m.first[i]);
}

}  // namespace

int fp8_amax_blocks(int64_t rows, int64_t cols) {
  const int64_t units = rows * ((cols + 7) / 8);
  const int64_t b = (units + kThreads - 1) / kThreads;
  return static_cast<int>(b < kFp8AmaxBlocks ? b : kFp8AmaxBlocks);
}

namespace {
unsigned cast_t_blocks(const Fp8QuantParams& p) {
  const int64_t tiles = ((p.rows + kTT - 1) / kTT) * ((p.cols + kTT - 1) / kTT);
  return static_cast<unsigned>(tiles < 4096 ? tiles : 4096);
}
}  // namespace

hipError_t launch_fp8_quantize(Fp8QuantParams p, hipStream_t s) {
  p.nblk = fp8_amax_blocks(p.rows, p.cols);
  hipLaunchKernelGGL(fp8_amax_kernel, dim3(p.nblk), dim3(kThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_fp8_cast(p, s);
}

hipError_t launch_fp8_cast(Fp8QuantParams p, hipStream_t s) {
  if (p.transpose) {
    hipLaunchKernelGGL(fp8_cast_t_kernel, dim3(cast_t_blocks(p)), dim3(kThreads), 0, s, p);
  } else {
    const int64_t units = p.rows * ((p.cols + 7) / 8);
    const int64_t b = (units + kThreads - 1) / kThreads;
    const unsigned g = static_cast<unsigned>(b < 8192 ? b : 8192);
    hipLaunchKernelGGL(fp8_cast_kernel, dim3(g), dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_quantize_multi(const Fp8QuantParams* ps, int n, hipStream_t s) {
  if (n < 1 || n > kFp8MaxMulti) return hipErrorInvalidValue;
  Fp8MultiParams m{};
  m.n = n;
  for (int i = 0; i < n; ++i) {
    m.t[i] = ps[i];
    if (!m.t[i].transpose) return hipErrorInvalidValue;
    m.t[i].nblk = fp8_amax_blocks(m.t[i].rows, m.t[i].cols);
    m.first[i + 1] = m.first[i] + m.t[i].nblk;
  }
  hipLaunchKernelGGL(fp8_amax_multi_kernel, dim3(m.first[n]), dim3(kThreads), 0, s, m);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  for (int i = 0; i < n; ++i) m.first[i + 1] = m.first[i] + static_cast<int>(cast_t_blocks(m.t[i]));
  hipLaunchKernelGGL(fp8_cast_t_multi_kernel, dim3(m.first[n]), dim3(kThreads), 0, s, m);
  return hipGetLastError();
}

}  // namespace tpmlp
