// Device pieces shared by the persistent row launches of the fused steps
// (mlp_step.hip, proj_step.hip): each XCD drains its own ticket queue of units
// over its own token rows; a unit waits for per-row-block counts of the units
// it reads, which their producers raise once their stores are complete.
#pragma once
#include <hip/hip_runtime.h>

#include "colsum_device.h"  // load8_f32, load8_bf16, store8
#include "gemm_tile.h"

namespace tpmlp {
namespace {

constexpr int kRows = 128;  // token rows of the smaller unit

__device__ __forceinline__ int xcc_id() {
  int v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(v));
  return v;
}

__device__ __forceinline__ unsigned load_count(const unsigned* c) {
  return __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread: returns once *c >= target (or the poll budget is spent, which
// sets the error word). Thread 0 polls; the block synchronises after.
__device__ __forceinline__ void wait_count(const unsigned* c, unsigned target, long long spin,
                                           unsigned* err) {
  if (threadIdx.x == 0) {
    unsigned v = load_count(c);
    for (long long n = spin; v < target && n > 0; --n) {
      __builtin_amdgcn_s_sleep(2);
      v = load_count(c);
    }
    if (v < target) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
}

// Every thread: after this block's stores are complete, count it done.
__device__ __forceinline__ void signal_count(unsigned* c) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every thread: the next ticket of queue q, broadcast through the pool.
__device__ __forceinline__ unsigned next_ticket(unsigned* q, uint8_t* pool) {
  __syncthreads();  // every wave is done with the pool
  unsigned* slot = reinterpret_cast<unsigned*>(pool);
  if (threadIdx.x == 0) *slot = __hip_atomic_fetch_add(q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const unsigned t = *slot;
  __syncthreads();  // read by all before the pool is reused
  return t;
}

// Every thread: the last block of the launch (by the done count at `done`)
// sets the words [from, to) of the counters, and the done count, back to 0.
__device__ __forceinline__ void finish_launch(unsigned* ctr, int64_t done, int64_t from,
                                              int64_t to) {
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned d = __hip_atomic_fetch_add(ctr + done, 1u, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_AGENT);
    if (d == gridDim.x - 1) {
      for (int64_t w = from; w < to; ++w)
        if (w != done) __hip_atomic_store(ctr + w, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(ctr + done, 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// out[row] = ((parts[0][row] + parts[1][row]) + ...) + bias, rounded once to
// bf16, for the kSumRows rows from row0: eight columns per item, each thread
// issuing the loads of all its items (up to kSumItems) before adding.
constexpr int kSumRows = 16;
constexpr int kSumItems = 4;
__device__ void rows_sum_unit(const float* parts, int64_t shard_stride, int p, int64_t ldp,
                              const void* bias, void* out, int64_t ldo, int64_t row0, int64_t N) {
  const int nv = static_cast<int>(N >> 3);
  const int items = kSumRows * nv;
  for (int base = 0; base < items; base += kSumItems * blockDim.x) {
    float sum[kSumItems][8];
#pragma unroll
    for (int k = 0; k < kSumItems; ++k) {
      const int e = base + k * blockDim.x + threadIdx.x;
      if (e < items) load8_f32(parts, (row0 + e / nv) * ldp + ((e % nv) << 3), sum[k]);
    }
    for (int i = 1; i < p; ++i) {
      float v[kSumItems][8];
#pragma unroll
      for (int k = 0; k < kSumItems; ++k) {
        const int e = base + k * blockDim.x + threadIdx.x;
        if (e < items)
          load8_f32(parts + i * shard_stride, (row0 + e / nv) * ldp + ((e % nv) << 3), v[k]);
      }
#pragma unroll
      for (int k = 0; k < kSumItems; ++k)
#pragma unroll
        for (int q = 0; q < 8; ++q) sum[k][q] += v[k][q];
    }
#pragma unroll
    for (int k = 0; k < kSumItems; ++k) {
      const int e = base + k * blockDim.x + threadIdx.x;
      if (e >= items) continue;
      const int64_t c = (e % nv) << 3;
      if (bias) {
        float b[8];
        load8_bf16(bias, c, b);
#pragma unroll
        for (int q = 0; q < 8; ++q) sum[k][q] += b[q];
      }
      store8(out, (row0 + e / nv) * ldo + c, sum[k], 1);
    }
  }
}

__device__ __forceinline__ const uint16_t* bf(const void* q) {
  return static_cast<const uint16_t*>(q);
}
__device__ __forceinline__ uint16_t* bfw(void* q) { return static_cast<uint16_t*>(q); }

// Tile configuration: RB token rows per unit (the row block), TN output
// columns, WM x WN waves; K-tile and stages of the products with an
// N-contiguous weight (NN: the forwards) and with two K-contiguous operands
// (NT: the data gradients); the LDS pool and blocks per CU it leaves room for.
template <int RB_, int TN_, int WM_, int WN_, int BKN_, int SN_, int BKT_, int ST_, int POOL_,
          int MINB_>
struct RowsCfg {
  static constexpr int RB = RB_, TN = TN_, WM = WM_, WN = WN_, BKN = BKN_, SN = SN_;
  static constexpr int BKT = BKT_, ST = ST_, POOL = POOL_, MINB = MINB_;
  static constexpr int THREADS = WM * WN * 64;
};
// 128 x 128 tiles, four waves, two blocks per CU
using RowsSmall = RowsCfg<128, 128, 2, 2, 32, 4, 64, 2, 80 * 1024, 2>;
// 256 x 128 tiles, eight waves of 64 x 64, one block per CU: two thirds of
// the operand bytes per flop of the 128 x 128 tile; three 64-wide K-tiles in
// flight (144 KiB of LDS)
using RowsLarge = RowsCfg<256, 128, 4, 2, 64, 3, 64, 3, 144 * 1024, 1>;

// One GEMM tile of a unit. (Inlined: as a function of its own every call
// saved and restored most of a wave's registers through scratch memory.)
template <int BM, int BN, int WM, int WN, int BK, int S, bool AK, bool BKC, int EK, int POOL>
__device__ __forceinline__ void unit_tile(const GemmParams& g, int64_t m0, int64_t n0,
                                                   int nk) {
  gemm_pipe_tile<BM, BN, WM, WN, BK, S, AK, BKC, EK, 0, POOL>(g, m0, n0, 0, 0, nk);
}

}  // namespace
}  // namespace tpmlp
