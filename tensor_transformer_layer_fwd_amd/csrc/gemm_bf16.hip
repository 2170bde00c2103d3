// bf16 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fp32
// accumulation, with the fused epilogues of the tensor-parallel shard:
//   forward  (NN): C = X W              + bias, activation, pre-activation saved
//   dgrad    (NT): C = dOut W^T         * act'(U)
//   wgrad    (TN): C = In^T dOut        (+= for accumulation, split-K partials)
//
// Work decomposition. A workgroup owns a BM x BN output tile and walks K in
// steps of 64. Both operand tiles are staged through LDS in the layout the
// matrix cores read: one 128-byte row of 64 K-values per output row / column,
// so every lane fetches its 8 consecutive K-values with one 16-byte LDS read.
// An operand that is contiguous along K in HBM (activations in NN/NT, the
// weight in NT) is copied as 16-byte vectors. An operand contiguous along M or
// N (the weight in NN, both operands in TN) is loaded as 16-byte vectors along
// M/N from KB consecutive K rows, transposed in registers (KB x 8 -> 8 x KB)
// and written as KB-element runs, so HBM reads stay fully coalesced.
// The 16-byte chunks of each LDS row are XOR-swizzled with (r ^ r>>3) & 7 so
// that 8 (or 16) lanes reading the same K-chunk of consecutive rows hit
// distinct banks.
// Two LDS stages: the next K-tile is fetched into registers while the matrix
// cores consume the current stage, then stored to the other stage; one barrier
// per K-step.
// Tile order: workgroups are dealt to the 8 XCDs round-robin, so block ids are
// remapped to give each XCD a contiguous range of tiles, and tiles are walked
// in groups of 8 tile-rows so that neighbours share operand tiles in L2.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace tpmlp {
namespace {

constexpr int KT = 64;  // K-tile (elements), one 128-byte LDS row

// Staging registers are native vectors (not HIP's union-based uint4), so the
// optimiser keeps them in VGPRs.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * KT + (((chunk ^ row ^ (row >> 3)) & 7) << 3);
}

// ---------------------------------------------------------------------------
// Operand tile loaders. An operand tile is ROWS (M or N) x KT (K) in LDS.
// ---------------------------------------------------------------------------

// Operand contiguous along K in HBM: element (r, k) at base[r*ld + k].
template <int ROWS, int NT, bool CHECK>
struct LoadKContig {
  static constexpr int NV = ROWS * (KT / 8) / NT;  // 16-byte vectors per thread
  static_assert(NV >= 1 && NV * NT == ROWS * (KT / 8), "tile/threads mismatch");
  u32x4 v[NV];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld,
                                       int64_t r0, int64_t rows_total, int64_t k0,
                                       int64_t kend, bool vec_ok, int tid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = tid + i * NT;
      const int r = idx >> 3, ch = idx & 7;
      const int64_t gr = r0 + r, gk = k0 + ch * 8;
      if (!CHECK) {
        v[i] = *reinterpret_cast<const u32x4*>(base + gr * ld + gk);
      } else if (gr < rows_total && gk + 8 <= kend && vec_ok) {
        v[i] = *reinterpret_cast<const u32x4*>(base + gr * ld + gk);
      } else {
        uint32_t e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j)
          e[j] = (gr < rows_total && gk + j < kend) ? base[gr * ld + gk + j] : 0u;
        v[i] = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                     e[6] | (e[7] << 16)};
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int idx = tid + i * NT;
      const int r = idx >> 3, ch = idx & 7;
      *reinterpret_cast<u32x4*>(lds + swz(r, ch)) = v[i];
    }
  }
};

// 16-bit element q (a compile-time constant after unrolling) of a u32x4.
__device__ __forceinline__ uint32_t elem16(const u32x4& v, int q) {
  const uint32_t w = v[q >> 1];
  return (q & 1) ? (w >> 16) : (w & 0xffffu);
}

// Operand contiguous along M/N in HBM: element (r, k) at base[k*ld + r].
// Each thread owns NB blocks of KB (K) x 8 (M/N) elements.
template <int ROWS, int NT, bool CHECK>
struct LoadMNContig {
  static constexpr int EPT = ROWS * KT / NT;                 // elements per thread
  static constexpr int KB = EPT / 8 >= 8 ? 8 : EPT / 8;      // K-rows per block
  static constexpr int NB = EPT / (8 * KB);                  // blocks per thread
  static constexpr int RB = ROWS / 8;                        // 8-wide blocks along M/N
  static_assert(KB == 2 || KB == 4 || KB == 8, "unsupported K block");
  static_assert(NB >= 1 && NB * KB * 8 * NT == ROWS * KT, "tile/threads mismatch");
  u32x4 v[NB][KB];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ base, int64_t ld,
                                       int64_t r0, int64_t rows_total, int64_t k0,
                                       int64_t kend, bool vec_ok, int tid) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int idx = tid + b * NT;
      const int rb = idx % RB, kb = idx / RB;
      const int64_t gr = r0 + rb * 8;
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        const int64_t gk = k0 + kb * KB + j;
        if (!CHECK) {
          v[b][j] = *reinterpret_cast<const u32x4*>(base + gk * ld + gr);
        } else if (gk < kend && gr + 8 <= rows_total && vec_ok) {
          v[b][j] = *reinterpret_cast<const u32x4*>(base + gk * ld + gr);
        } else {
          uint32_t e[8];
#pragma unroll
          for (int q = 0; q < 8; ++q)
            e[q] = (gk < kend && gr + q < rows_total) ? base[gk * ld + gr + q] : 0u;
          v[b][j] = u32x4{e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16),
                          e[6] | (e[7] << 16)};
        }
      }
    }
  }

  // Transpose each KB x 8 block to 8 runs of KB K-values and write them.
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int idx = tid + b * NT;
      const int rb = idx % RB, kb = idx / RB;
      const int kk = kb * KB;  // first K within the tile
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int r = rb * 8 + q;
        uint16_t* dst = lds + swz(r, kk >> 3) + (kk & 7);
        if constexpr (KB == 8) {
          *reinterpret_cast<u32x4*>(dst) =
              u32x4{elem16(v[b][0], q) | (elem16(v[b][1], q) << 16),
                    elem16(v[b][2], q) | (elem16(v[b][3], q) << 16),
                    elem16(v[b][4], q) | (elem16(v[b][5], q) << 16),
                    elem16(v[b][6], q) | (elem16(v[b][7], q) << 16)};
        } else if constexpr (KB == 4) {
          *reinterpret_cast<u32x2*>(dst) =
              u32x2{elem16(v[b][0], q) | (elem16(v[b][1], q) << 16),
                    elem16(v[b][2], q) | (elem16(v[b][3], q) << 16)};
        } else {
          *reinterpret_cast<uint32_t*>(dst) = elem16(v[b][0], q) | (elem16(v[b][1], q) << 16);
        }
      }
    }
  }
};

// Calls f(std::integral_constant<int, I>) for I = I0 .. END-1, so that the
// body indexes register arrays with compile-time constants only.
template <int I0, int END>
struct StaticFor {
  template <class F>
  __device__ __forceinline__ static void run(F&& f) {
    f(std::integral_constant<int, I0>{});
    StaticFor<I0 + 1, END>::run(f);
  }
};
template <int END>
struct StaticFor<END, END> {
  template <class F>
  __device__ __forceinline__ static void run(F&&) {}
};

template <bool KCONTIG, int ROWS, int NT, bool CHECK>
using Loader = typename std::conditional<KCONTIG, LoadKContig<ROWS, NT, CHECK>,
                                         LoadMNContig<ROWS, NT, CHECK>>::type;

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, bool AK, bool BKC, bool CHECK>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_kernel(GemmParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile
  constexpr int FM = WTM / 32, FN = WTN / 32;  // 32x32 fragments per wave
  static_assert(FM >= 1 && FN >= 1 && FM * 32 * WM == BM && FN * 32 * WN == BN, "tile");

  __shared__ __attribute__((aligned(16))) uint16_t smem[2][(BM + BN) * KT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- tile of this workgroup
  const int tiles_m = static_cast<int>((p.M + BM - 1) / BM);
  const int tiles_n = static_cast<int>((p.N + BN - 1) / BN);
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  const int X = p.xcds;  // blocks go round-robin over the XCDs
  if (X > 1 && ntiles % X == 0) bid = (bid % X) * (ntiles / X) + bid / X;
  constexpr int G = 8;
  const int group = bid / (G * tiles_n);
  const int first_m = group * G;
  const int gs = min(tiles_m - first_m, G);
  const int in_group = bid - group * G * tiles_n;
  const int tm = first_m + in_group % gs;
  const int tn = in_group / gs;
  const int64_t m0 = static_cast<int64_t>(tm) * BM;
  const int64_t n0 = static_cast<int64_t>(tn) * BN;

  // ---- K range of this split
  const int z = blockIdx.y;
  const int64_t kbeg = static_cast<int64_t>(z) * p.k_chunk;
  const int64_t kend = min(p.K, kbeg + p.k_chunk);
  const int nk = static_cast<int>((kend - kbeg + KT - 1) / KT);

  const uint16_t* __restrict__ A = static_cast<const uint16_t*>(p.a);
  const uint16_t* __restrict__ B = static_cast<const uint16_t*>(p.b);
  const bool a_vec = ((reinterpret_cast<uintptr_t>(A) & 15) == 0) && ((p.lda & 7) == 0);
  const bool b_vec = ((reinterpret_cast<uintptr_t>(B) & 15) == 0) && ((p.ldb & 7) == 0);

  Loader<AK, BM, NT, CHECK> la;
  Loader<BKC, BN, NT, CHECK> lb;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  if (nk > 0) {
    la.load(A, p.lda, m0, p.M, kbeg, kend, a_vec, tid);
    lb.load(B, p.ldb, n0, p.N, kbeg, kend, b_vec, tid);
    la.store(&smem[0][0], tid);
    lb.store(&smem[0][BM * KT], tid);
  }
  __syncthreads();

  const int frow = lane & 31;   // row (A) / column (B) within a 32-wide fragment
  const int fkc = lane >> 5;    // which 8-element K chunk of the 16 per MFMA

  for (int it = 0; it < nk; ++it) {
    const int cur = it & 1;
    if (it + 1 < nk) {
      const int64_t kn = kbeg + static_cast<int64_t>(it + 1) * KT;
      la.load(A, p.lda, m0, p.M, kn, kend, a_vec, tid);
      lb.load(B, p.ldb, n0, p.N, kn, kend, b_vec, tid);
    }
    const uint16_t* sa = &smem[cur][0];
    const uint16_t* sb = &smem[cur][BM * KT];
#pragma unroll
    for (int ks = 0; ks < KT / 16; ++ks) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(sa + swz(wm * WTM + i * 32 + frow, ks * 2 + fkc));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(sb + swz(wn * WTN + j * 32 + frow, ks * 2 + fkc));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (it + 1 < nk) {
      la.store(&smem[cur ^ 1][0], tid);
      lb.store(&smem[cur ^ 1][BM * KT], tid);
    }
    __syncthreads();
  }

  // ---- epilogue through LDS. Each wave owns 32 x EP floats of the (now free)
  // operand LDS. For every 32-row band i of its wave tile it writes the
  // accumulators there in the 32x32 MFMA layout (lane holds column lane & 31;
  // register r holds row 8*(r/4) + 4*(lane/32) + r%4), then reads them back as
  // 8 consecutive columns per lane and finishes them with 16-byte accesses.
  constexpr int EP = WTN + 4;       // padded row pitch (floats)
  constexpr int LPR = WTN / 8;      // lanes per tile row on the way out
  constexpr int RPP = 64 / LPR;     // tile rows per pass
  static_assert(WM * WN * 32 * EP * 4 <= sizeof(smem), "epilogue LDS");
  static_assert(32 % RPP == 0, "rows per pass");
  float* ep = reinterpret_cast<float*>(&smem[0][0]) + wave * 32 * EP;
  const int er = lane / LPR, ec = (lane % LPR) * 8;
  const bool split = p.splitk > 1;
  float* ws = split ? p.ws + static_cast<int64_t>(z) * p.M * p.N : nullptr;
  const bool out_vec =
      split ? ((reinterpret_cast<uintptr_t>(p.ws) & 15) == 0 && (p.N & 7) == 0)
            : epilogue_vec_ok(p);
  StaticFor<0, FM>::run([&](auto band) {
    constexpr int i = decltype(band)::value;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ep[((r >> 2) * 8 + 4 * (lane >> 5) + (r & 3)) * EP + j * 32 + (lane & 31)] = acc[i][j][r];
    __syncthreads();
#pragma unroll
    for (int pass = 0; pass < 32 / RPP; ++pass) {
      const int lr = pass * RPP + er;
      const float* src = ep + lr * EP + ec;
      float v[8];
      const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(src);
      const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(src + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = lo[q];
        v[q + 4] = hi[q];
      }
      const int64_t row = m0 + wm * WTM + i * 32 + lr;
      const int64_t col = n0 + wn * WTN + ec;
      const bool full = !CHECK || (row < p.M && col + 8 <= p.N);
      if (split) {
        if (full && out_vec) {
          float* d = ws + row * p.N + col;
          *reinterpret_cast<f32x4_t*>(d) = lo;
          *reinterpret_cast<f32x4_t*>(d + 4) = hi;
        } else if (row < p.M) {
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if (col + q < p.N) ws[row * p.N + col + q] = v[q];
        }
      } else if (full && out_vec) {
        epilogue_vec8(p, row, col, v);
      } else if (row < p.M) {
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (col + q < p.N) epilogue_elem(p, row, col + q, v[q], 1);
      }
    }
    __syncthreads();
  });
}

// ---------------------------------------------------------------------------
// Launch
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, bool AK, bool BKC>
hipError_t launch_cfg(const GemmParams& p, const SplitPlan& plan, hipStream_t s) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(plan.splitk));
  dim3 block(WM * WN * 64);
  const bool a_vec = (reinterpret_cast<uintptr_t>(p.a) & 15) == 0 && (p.lda & 7) == 0;
  const bool b_vec = (reinterpret_cast<uintptr_t>(p.b) & 15) == 0 && (p.ldb & 7) == 0;
  const bool fast = p.M % BM == 0 && p.N % BN == 0 && p.K % KT == 0 &&
                    plan.k_chunk % KT == 0 && a_vec && b_vec;
  if (fast)
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, AK, BKC, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, AK, BKC, true>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <bool AK, bool BKC>
hipError_t launch_layout(const GemmParams& p, const SplitPlan& plan, hipStream_t s) {
  return launch_cfg<128, 128, 2, 2, AK, BKC>(p, plan, s);
}

}  // namespace

hipError_t launch_gemm_bf16_general(const GemmParams& p, const SplitPlan& plan, hipStream_t s) {
  if (p.a_kcontig && !p.b_kcontig) return launch_layout<true, false>(p, plan, s);    // NN
  if (p.a_kcontig && p.b_kcontig) return launch_layout<true, true>(p, plan, s);      // NT
  if (!p.a_kcontig && !p.b_kcontig) return launch_layout<false, false>(p, plan, s);  // TN
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
