// fp32 GEMM for the fp32 shard workloads (small shapes; exactness over speed):
// C[M,N] = op(A)[M,K] op(B)[K,N] with the same fused epilogues as the bf16
// path. 64x64 output tile per workgroup, 4x4 outputs per thread, K staged
// through LDS in steps of 16. Any layout, stride and shape is handled with
// bounds checks; products accumulate with fmaf in K order.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace tpmlp {
namespace {

constexpr int TM = 64, TN = 64, TK = 16;

__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmParams p) {
  __shared__ float As[TK][TM + 1];
  __shared__ float Bs[TK][TN + 1];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int64_t m0 = static_cast<int64_t>(blockIdx.y) * TM;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * TN;
  const float* __restrict__ A = static_cast<const float*>(p.a);
  const float* __restrict__ B = static_cast<const float*>(p.b);
  const int64_t sam = p.a_kcontig ? p.lda : 1, sak = p.a_kcontig ? 1 : p.lda;
  const int64_t sbn = p.b_kcontig ? p.ldb : 1, sbk = p.b_kcontig ? 1 : p.ldb;

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int64_t k0 = 0; k0 < p.K; k0 += TK) {
    for (int e = tid; e < TK * TM; e += 256) {
      const int kk = e / TM, mm = e % TM;
      const int64_t gk = k0 + kk, gm = m0 + mm, gn = n0 + mm;
      As[kk][mm] = (gk < p.K && gm < p.M) ? A[gm * sam + gk * sak] : 0.0f;
      Bs[kk][mm] = (gk < p.K && gn < p.N) ? B[gn * sbn + gk * sbk] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t row = m0 + ty * 4 + i, col = n0 + tx * 4 + j;
      if (row < p.M && col < p.N) epilogue_elem(p, row, col, acc[i][j], 0);
    }
}

}  // namespace

hipError_t launch_gemm_f32(const GemmParams& p, hipStream_t s) {
  const int64_t gx = (p.N + TN - 1) / TN, gy = (p.M + TM - 1) / TM;
  if (gy > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(static_cast<unsigned>(gx), static_cast<unsigned>(gy)),
                     dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace tpmlp
