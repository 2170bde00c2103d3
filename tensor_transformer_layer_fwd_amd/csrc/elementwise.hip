// HBM-bound passes of the shard step:
//   - split-K fix-up: sum the fp32 K-slice partials in slice order, apply the
//     epilogue (used by the wgrad GEMM when its output has too few tiles);
//   - column sums (bias gradients), two deterministic passes;
//   - the sum over shards that stands in for the All-Reduce;
//   - a standalone bias + activation pass.
#include <hip/hip_runtime.h>

#include "colsum_device.h"
#include "device_common.h"
#include "internal.h"

namespace tpmlp {
namespace {

__global__ __launch_bounds__(256) void splitk_fixup_kernel(GemmParams p) {
  const int64_t total = p.M * p.N;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += stride) {
    float v = 0.0f;
    for (int z = 0; z < p.splitk; ++z) v += p.ws[z * total + e];
    const int64_t row = e / p.N, col = e - row * p.N;
    epilogue_elem(p, row, col, v, 1);
  }
}

// Vector fix-up of fp32 weight gradients: four columns per thread, the K-slice
// partials summed in slice order, then accumulated into C if requested.
__global__ __launch_bounds__(256) void splitk_fixup_vec4_kernel(GemmParams p) {
  splitk_fixup_vec4_unit(p, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x,
                         static_cast<int64_t>(gridDim.x) * blockDim.x);
}

// Column sums (bias gradients) in two deterministic passes over chunks of
// kColsumRows rows.
// Pass 1, general path: block (cb, chunk) sums its rows of 128 columns.
// Thread (cx, ry) owns columns 2cx, 2cx+1 and rows ry, ry+4, ...; the four
// row-groups are then added in order through LDS.
__global__ __launch_bounds__(256) void colsum_pass1_kernel(ColsumParams p, int nchunks) {
  __shared__ float part[4][128];
  const int cx = threadIdx.x & 63, ry = threadIdx.x >> 6;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 128 + cx * 2;
  const int64_t t0 = static_cast<int64_t>(blockIdx.y) * kColsumRows;
  const int64_t t1 = min(p.T, t0 + kColsumRows);
  float s0 = 0.0f, s1 = 0.0f;
  for (int64_t t = t0 + ry; t < t1; t += 4) {
    const int64_t o = t * p.ld + c;
    if (c < p.N) s0 += load_elem(p.src, o, p.src_bf16);
    if (c + 1 < p.N) s1 += load_elem(p.src, o + 1, p.src_bf16);
  }
  part[ry][cx * 2] = s0;
  part[ry][cx * 2 + 1] = s1;
  __syncthreads();
  if (threadIdx.x < 128) {
    const int64_t cc = static_cast<int64_t>(blockIdx.x) * 128 + threadIdx.x;
    if (cc < p.N) {
      float v = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) +
                part[3][threadIdx.x];
      if (nchunks == 1) {
        p.dbias[cc] = p.accumulate ? p.dbias[cc] + v : v;
      } else {
        p.ws[static_cast<int64_t>(blockIdx.y) * p.N + cc] = v;
      }
    }
  }
}

// Pass 1, vector path: one unit (column block, row chunk) per block.
__global__ __launch_bounds__(256) void colsum_vec_pass1_kernel(ColsumParams p, int nchunks) {
  __shared__ float part[8][256];
  colsum_vec_unit(p, blockIdx.x, blockIdx.y, nchunks, part);
}

// Pass 2: one unit of 64 columns per block.
__global__ __launch_bounds__(256) void colsum_pass2_kernel(ColsumParams p, int nchunks) {
  __shared__ float part[4][64];
  colsum_pass2_unit(p, blockIdx.x, nchunks, part);
}

// Split-K fix-up (vector path) and column-sum pass 2 in one launch: blocks
// below nfix run the fix-up, the rest one pass-2 unit each.
__global__ __launch_bounds__(256) void splitk_fixup_colsum_kernel(GemmParams p, int nfix,
                                                                  int nchunks) {
  __shared__ float part[4][64];
  if (static_cast<int>(blockIdx.x) >= nfix) {
    colsum_pass2_unit(p.cs, blockIdx.x - nfix, nchunks, part);
    return;
  }
  splitk_fixup_vec4_unit(p, static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x,
                         static_cast<int64_t>(nfix) * blockDim.x);
}

// out = ((parts[0] + parts[1]) + ...) + bias, rounded once. Vector path: four
// consecutive columns per thread.
__global__ __launch_bounds__(256) void reduce_vec4_kernel(ReduceParams p) {
  const int64_t nq = p.N >> 2;
  const int64_t total = p.T * nq;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += stride) {
    const int64_t t = e / nq, c = (e - t * nq) << 2;
    const int64_t ip = t * p.ldp + c;
    float4 s = *reinterpret_cast<const float4*>(p.parts[0] + ip);
    for (int i = 1; i < p.p; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(p.parts[i] + ip);
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    if (p.bias) {
      const int bb = p.out_bf16;
      s.x += load_elem(p.bias, c, bb);
      s.y += load_elem(p.bias, c + 1, bb);
      s.z += load_elem(p.bias, c + 2, bb);
      s.w += load_elem(p.bias, c + 3, bb);
    }
    const int64_t io = t * p.ldo + c;
    if (p.out_bf16) {
      uint2 o;
      o.x = pack_bf16x2(s.x, s.y);
      o.y = pack_bf16x2(s.z, s.w);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + io) = o;
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p.out) + io) = s;
    }
  }
}

// Eight consecutive columns per thread: two 16-byte loads per partial in
// flight and one 16-byte bf16 store (or two fp32 ones), with 32-bit index
// arithmetic (the host checks T * N / 8 < 2^31). Same summation order as the
// four-column path: partials in shard order, then the bias.
__global__ __launch_bounds__(256) void reduce_vec8_kernel(ReduceParams p) {
  const uint32_t no = static_cast<uint32_t>(p.N >> 3);
  const uint32_t total = static_cast<uint32_t>(p.T) * no;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const uint32_t t = e / no, c = (e - t * no) << 3;
    const int64_t ip = static_cast<int64_t>(t) * p.ldp + c;
    float s[8];
    load8_f32(p.parts[0], ip, s);
    for (int i = 1; i < p.p; ++i) {
      float v[8];
      load8_f32(p.parts[i], ip, v);
#pragma unroll
      for (int q = 0; q < 8; ++q) s[q] += v[q];
    }
    if (p.bias) {
      float b[8];
      if (p.out_bf16) load8_bf16(p.bias, c, b);
      else load8_f32(p.bias, c, b);
#pragma unroll
      for (int q = 0; q < 8; ++q) s[q] += b[q];
    }
    store8(p.out, static_cast<int64_t>(t) * p.ldo + c, s, p.out_bf16);
  }
}

__global__ __launch_bounds__(256) void reduce_scalar_kernel(ReduceParams p) {
  const int64_t total = p.T * p.N;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += stride) {
    const int64_t t = e / p.N, c = e - t * p.N;
    float s = p.parts[0][t * p.ldp + c];
    for (int i = 1; i < p.p; ++i) s += p.parts[i][t * p.ldp + c];
    if (p.bias) s += load_elem(p.bias, c, p.out_bf16);
    store_elem(p.out, t * p.ldo + c, s, p.out_bf16);
  }
}

__global__ __launch_bounds__(256) void bias_act_kernel(BiasActParams p) {
  const int64_t total = p.T * p.N;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += stride) {
    const int64_t t = e / p.N, c = e - t * p.N;
    float u = p.u_f32 ? static_cast<const float*>(p.u)[t * p.ldu + c]
                      : load_elem(p.u, t * p.ldu + c, p.in_bf16);
    if (p.bias) u += load_elem(p.bias, c, p.in_bf16);
    store_elem(p.y, t * p.ldy + c, apply_act(p.act, u), p.out_bf16);
  }
}

// Vector path of bias_act: fp32 or bf16 U, bf16 Y, eight columns per thread
// (two 16-byte loads of fp32 U or one of bf16 U, one 16-byte store), 32-bit
// index arithmetic.
__global__ __launch_bounds__(256) void bias_act_vec8_kernel(BiasActParams p) {
  const uint32_t no = static_cast<uint32_t>(p.N >> 3);
  const uint32_t total = static_cast<uint32_t>(p.T) * no;
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t e = blockIdx.x * blockDim.x + threadIdx.x; e < total; e += stride) {
    const uint32_t t = e / no, c = (e - t * no) << 3;
    float u[8];
    if (p.u_f32) load8_f32(p.u, static_cast<int64_t>(t) * p.ldu + c, u);
    else load8_bf16(p.u, static_cast<int64_t>(t) * p.ldu + c, u);
    if (p.bias) {
      float b[8];
      if (p.in_bf16) load8_bf16(p.bias, c, b);
      else load8_f32(p.bias, c, b);
#pragma unroll
      for (int q = 0; q < 8; ++q) u[q] += b[q];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) u[q] = apply_act(p.act, u[q]);
    store8(p.y, static_cast<int64_t>(t) * p.ldy + c, u, 1);
  }
}

// Vector path of bias_act: fp32 U, bf16 Y, four columns per thread.
__global__ __launch_bounds__(256) void bias_act_vec4_kernel(BiasActParams p) {
  const int64_t nq = p.N >> 2;
  const int64_t total = p.T * nq;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += stride) {
    const int64_t t = e / nq, c = (e - t * nq) << 2;
    float4 u = *reinterpret_cast<const float4*>(static_cast<const float*>(p.u) + t * p.ldu + c);
    if (p.bias) {
      u.x += load_elem(p.bias, c, p.in_bf16);
      u.y += load_elem(p.bias, c + 1, p.in_bf16);
      u.z += load_elem(p.bias, c + 2, p.in_bf16);
      u.w += load_elem(p.bias, c + 3, p.in_bf16);
    }
    uint2 o;
    o.x = pack_bf16x2(apply_act(p.act, u.x), apply_act(p.act, u.y));
    o.y = pack_bf16x2(apply_act(p.act, u.z), apply_act(p.act, u.w));
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + t * p.ldy + c) = o;
  }
}

unsigned grid_for(int64_t work, int per_block) {
  int64_t g = (work + per_block - 1) / per_block;
  const int64_t cap = 256 * 16;  // enough workgroups to cover every CU many times
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return static_cast<unsigned>(g);
}

}  // namespace

size_t colsum_workspace_bytes(int64_t T, int64_t N) {
  const int64_t nchunks = (T + kColsumRows - 1) / kColsumRows;
  return nchunks > 1 ? static_cast<size_t>(nchunks * N) * sizeof(float) : 0;
}

bool splitk_fixup_vec_ok(const GemmParams& p) {
  return !p.out_bf16 && p.epi == EPI_STORE && p.N % 4 == 0 && p.ldc % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(p.c) & 15) == 0 &&
         (reinterpret_cast<uintptr_t>(p.ws) & 15) == 0;
}

hipError_t launch_splitk_fixup(const GemmParams& p, hipStream_t s) {
  const bool vec = splitk_fixup_vec_ok(p);
  // column sums carried by the GEMM launch: pass 2 rides along here
  const bool pass2 = p.cs_blocks > 0 && p.cs_nchunks > 1;
  if (vec && pass2) {
    const unsigned nfix = grid_for(p.M * p.N / 4, 256);
    const unsigned ncs = static_cast<unsigned>((p.cs.N + 63) / 64);
    hipLaunchKernelGGL(splitk_fixup_colsum_kernel, dim3(nfix + ncs), dim3(256), 0, s, p,
                       static_cast<int>(nfix), p.cs_nchunks);
    return hipGetLastError();
  }
  if (vec)
    hipLaunchKernelGGL(splitk_fixup_vec4_kernel, dim3(grid_for(p.M * p.N / 4, 256)), dim3(256), 0,
                       s, p);
  else
    hipLaunchKernelGGL(splitk_fixup_kernel, dim3(grid_for(p.M * p.N, 256)), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !pass2) return e;
  return launch_colsum_pass2(p.cs, p.cs_nchunks, s);
}

int64_t colsum_chunks(const ColsumParams& p) { return (p.T + kColsumRows - 1) / kColsumRows; }

bool colsum_vec_ok(const ColsumParams& p) {
  return p.N % 8 == 0 && p.ld % 8 == 0 && (reinterpret_cast<uintptr_t>(p.src) & 15) == 0;
}

hipError_t launch_colsum_pass2(const ColsumParams& p, int nchunks, hipStream_t s) {
  hipLaunchKernelGGL(colsum_pass2_kernel, dim3(static_cast<unsigned>((p.N + 63) / 64)), dim3(256),
                     0, s, p, nchunks);
  return hipGetLastError();
}

hipError_t launch_colsum(const ColsumParams& p, hipStream_t s) {
  const int64_t nchunks = colsum_chunks(p);
  if (nchunks > 65535) return hipErrorInvalidConfiguration;
  const bool vec = colsum_vec_ok(p);
  if (vec)
    hipLaunchKernelGGL(colsum_vec_pass1_kernel,
                       dim3(static_cast<unsigned>((p.N + 255) / 256), static_cast<unsigned>(nchunks)),
                       dim3(256), 0, s, p, static_cast<int>(nchunks));
  else
    hipLaunchKernelGGL(colsum_pass1_kernel,
                       dim3(static_cast<unsigned>((p.N + 127) / 128), static_cast<unsigned>(nchunks)),
                       dim3(256), 0, s, p, static_cast<int>(nchunks));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || nchunks == 1) return e;
  return launch_colsum_pass2(p, static_cast<int>(nchunks), s);
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t s) {
  auto a16 = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  bool vec8 = p.N % 8 == 0 && p.ldp % 4 == 0 && p.ldo % 8 == 0 && a16(p.out) &&
              (!p.bias || a16(p.bias)) && p.T * (p.N / 8) < (int64_t(1) << 31);
  for (int i = 0; i < p.p; ++i) vec8 = vec8 && a16(p.parts[i]);
  if (vec8) {
    hipLaunchKernelGGL(reduce_vec8_kernel, dim3(grid_for(p.T * (p.N / 8), 256)), dim3(256), 0,
                       s, p);
    return hipGetLastError();
  }
  bool vec = (p.N % 4 == 0) && (p.ldp % 4 == 0) && (p.ldo % 4 == 0);
  for (int i = 0; i < p.p; ++i) vec = vec && (reinterpret_cast<uintptr_t>(p.parts[i]) % 16 == 0);
  vec = vec && (reinterpret_cast<uintptr_t>(p.out) % (p.out_bf16 ? 8 : 16) == 0);
  if (vec)
    hipLaunchKernelGGL(reduce_vec4_kernel, dim3(grid_for(p.T * (p.N / 4), 256)), dim3(256), 0,
                       s, p);
  else
    hipLaunchKernelGGL(reduce_scalar_kernel, dim3(grid_for(p.T * p.N, 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bias_act(const BiasActParams& p, hipStream_t s) {
  auto a16 = [](const void* q) { return reinterpret_cast<uintptr_t>(q) % 16 == 0; };
  // rows of U start 16-byte aligned: 4 fp32 or 8 bf16 elements
  if ((p.u_f32 || p.in_bf16) && p.out_bf16 && p.N % 8 == 0 && p.ldu % (p.u_f32 ? 4 : 8) == 0 &&
      p.ldy % 8 == 0 && a16(p.u) && a16(p.y) && (!p.bias || a16(p.bias)) &&
      p.T * (p.N / 8) < (int64_t(1) << 31)) {
    hipLaunchKernelGGL(bias_act_vec8_kernel, dim3(grid_for(p.T * (p.N / 8), 256)), dim3(256), 0,
                       s, p);
    return hipGetLastError();
  }
  const bool vec = p.u_f32 && p.out_bf16 && (p.N % 4 == 0) && (p.ldu % 4 == 0) &&
                   (p.ldy % 4 == 0) && (reinterpret_cast<uintptr_t>(p.u) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(p.y) % 8 == 0);
  if (vec)
    hipLaunchKernelGGL(bias_act_vec4_kernel, dim3(grid_for(p.T * (p.N / 4), 256)), dim3(256), 0,
                       s, p);
  else
    hipLaunchKernelGGL(bias_act_kernel, dim3(grid_for(p.T * p.N, 256)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace tpmlp
