// Pipelined bf16 / FP8 GEMM launches for tile-aligned shapes on gfx950: one
// output tile per block (gemm_tile.h), the paired backward launches of a
// layer's two gradients, and the host-side dispatch by tile and epilogue.
#include <hip/hip_runtime.h>

#include "gemm_tile.h"
#include "step_queue.h"  // rows_sum_unit

namespace tpmlp {
namespace {

template <int BM, int BN, int WM, int WN, int BK, int S, bool AK, bool BKC, int EK, int F8 = 0>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_pipe_kernel(GemmParams p) {
  gemm_pipe_block<BM, BN, WM, WN, BK, S, AK, BKC, EK, F8>(p, static_cast<int>(blockIdx.x));
}

// The backward of one linear layer in one launch: the weight gradient (TN,
// fp32, tile W = BMW x BNW with BKW-wide K-tiles in SW stages; K slices and
// column-sum units as in its own launch) in blocks 0 .. nblk_w-1, then the
// data gradient (NT, tile D, epilogue EKD). Both products keep their stages
// in one LDS pool sized for the larger, so the launch needs no more LDS than
// its larger product alone. The last nfix_r + ncs_r blocks finish an earlier
// weight gradient pr on the CUs the data gradient leaves while the weight
// gradient's longer blocks still run: its split-K fix-up (vector path), then
// its column-sum pass-2 units.
template <int BMW, int BNW, int BKW, int SW, int BMD, int BND, int BKD, int SD, int EKD>
__global__ __launch_bounds__(256) void gemm_bwd_pair_kernel(GemmParams pw, GemmParams pd,
                                                            int nblk_w, int nblk_d,
                                                            GemmParams pr, int nfix_r, int ncs_r,
                                                            ColsumParams c2, int c2_nchunks) {
  constexpr int PW = SW * (BMW + BNW) * BKW * 2, PD = SD * (BMD + BND) * BKD * 2;
  constexpr int POOL = PW > PD ? PW : PD;
  const int b = static_cast<int>(blockIdx.x);
  if (b < nblk_w) {
    gemm_pipe_block<BMW, BNW, 2, 2, BKW, SW, false, false, kEpiF32, 0, POOL>(pw, b);
  } else if (b < nblk_w + nblk_d) {
    gemm_pipe_block<BMD, BND, 2, 2, BKD, SD, true, true, EKD, 0, POOL>(pd, b - nblk_w);
  } else {
    const int r = b - nblk_w - nblk_d;
    if (r < nfix_r) {
      splitk_fixup_vec4_unit(pr, static_cast<int64_t>(r) * blockDim.x + threadIdx.x,
                             static_cast<int64_t>(nfix_r) * blockDim.x);
    } else {
      float(*part)[64] = reinterpret_cast<float(*)[64]>(pool_buf<POOL>());
      if (r < nfix_r + ncs_r) colsum_pass2_unit(pr.cs, r - nfix_r, pr.cs_nchunks, part);
      else colsum_pass2_unit(c2, r - nfix_r - ncs_r, c2_nchunks, part);
    }
  }
}

// Two weight gradients in one launch (TN, fp32, 128 x 128 tiles with 32-wide
// K-tiles in four stages): the tiles run over all of K (product 0's, then
// product 1's), then each product's column-sum pass-1 units (gemm_pipe_block
// runs those for block indices past its tiles), then the K slices of the
// split tiles, then the units of an optional row sum. Where each product
// alone fills only part of the CUs, one launch puts both products' tiles on
// them at once; where the tiles leave a remainder over the CUs, slicing the
// remaining tiles along K spreads them over every CU instead of doubling the
// work of a few. The row-sum units read and write memory only: they take the
// CUs' second block slots, which the slices leave early, while the tiles'
// matrix work runs beside them.
constexpr int kWg = 128;  // tile rows and columns

// K slice c of the split tiles: tile whole + c / sk, slice c % sk, into its
// compact partial. The operands start at the tile's origin, so the tile body
// runs at (0, 0) and its split-K epilogue stores rows of 128.
__device__ __forceinline__ void wgrad_slice(const GemmParams& p0, const GemmParams& p1, int nt0,
                                            const WgradSplit& sp, int c) {
  const int t = sp.whole + c / sp.sk, kz = c % sp.sk;
  const GemmParams& p = t < nt0 ? p0 : p1;
  int64_t m0, n0;
  tile_origin<kWg, kWg>(p, t < nt0 ? t : t - nt0, &m0, &n0);
  GemmParams q = p;
  q.a = static_cast<const uint16_t*>(p.a) + m0;  // In [T, k]: its columns m0 ..
  q.b = static_cast<const uint16_t*>(p.b) + n0;  // dOut [T, n]: its columns n0 ..
  q.M = q.N = kWg;
  q.splitk = sp.sk;
  q.ws = sp.part + static_cast<int64_t>(c) * kWg * kWg;
  const int64_t kc = p.K / sp.sk;
  gemm_pipe_tile<128, 128, 2, 2, 32, 4, false, false, kEpiF32>(q, 0, 0, 0, kz * kc,
                                                              static_cast<int>(kc / 32));
}

__global__ __launch_bounds__(256) void gemm_wgrad2_kernel(GemmParams p0, GemmParams p1, int nt0,
                                                          int nt1, WgradSplit sp, int nsl,
                                                          RowSumParams rs) {
  const int b = static_cast<int>(blockIdx.x);
  const int ncs = p0.cs_blocks + p1.cs_blocks;
  if (b < sp.whole) {
    if (b < nt0) gemm_pipe_block<128, 128, 2, 2, 32, 4, false, false, kEpiF32>(p0, b);
    else gemm_pipe_block<128, 128, 2, 2, 32, 4, false, false, kEpiF32>(p1, b - nt0);
  } else if (b < sp.whole + ncs) {
    const int r = b - sp.whole;
    if (r < p0.cs_blocks) gemm_pipe_block<128, 128, 2, 2, 32, 4, false, false, kEpiF32>(p0, nt0 + r);
    else gemm_pipe_block<128, 128, 2, 2, 32, 4, false, false, kEpiF32>(p1, nt1 + r - p0.cs_blocks);
  } else if (b < sp.whole + ncs + nsl) {
    wgrad_slice(p0, p1, nt0, sp, b - sp.whole - ncs);
  } else {
    const int64_t row0 = static_cast<int64_t>(b - sp.whole - ncs - nsl) * kSumRows;
    rows_sum_unit(rs.parts, rs.rows * rs.N, rs.p, rs.N, nullptr, rs.out, rs.ld_out, row0, rs.N);
  }
}

// After the weight gradients: blocks below nfix add the K slices of 8 rows of
// a split tile, in slice order, into the tile's output (one float4 per thread,
// every slice's load issued before the adds); the others run pass 2 of the
// column sums, product 0's 64-column units (u0 of them), then product 1's.
constexpr int kFinRows = 8;   // rows of a split tile per fix-up block
constexpr int kMaxSlices = 16;
__global__ __launch_bounds__(256) void wgrad2_finish_kernel(GemmParams p0, GemmParams p1, int nt0,
                                                            WgradSplit sp, int nfix, int u0,
                                                            int n0, int n1) {
  const int b = static_cast<int>(blockIdx.x);
  if (b >= nfix) {
    __shared__ float part[4][64];
    if (b - nfix < u0) colsum_pass2_unit(p0.cs, b - nfix, n0, part);
    else colsum_pass2_unit(p1.cs, b - nfix - u0, n1, part);
    return;
  }
  constexpr int C = kWg, PER = kWg / kFinRows;  // row groups of a tile
  static_assert(kFinRows * C == 4 * 256, "one float4 per thread");
  const int e = b / PER, grp = b % PER;
  const int t = sp.whole + e;
  const GemmParams& p = t < nt0 ? p0 : p1;
  int64_t m0, n0t;
  tile_origin<kWg, kWg>(p, t < nt0 ? t : t - nt0, &m0, &n0t);
  const int idx = grp * kFinRows * C + static_cast<int>(threadIdx.x) * 4;  // within the tile
  const float* src = sp.part + static_cast<int64_t>(e) * sp.sk * C * C + idx;
  f32x4_t v[kMaxSlices];
#pragma unroll
  for (int z = 0; z < kMaxSlices; ++z)
    if (z < sp.sk) v[z] = *reinterpret_cast<const f32x4_t*>(src + static_cast<int64_t>(z) * C * C);
  f32x4_t acc = v[0];
#pragma unroll
  for (int z = 1; z < kMaxSlices; ++z)
    if (z < sp.sk) acc += v[z];
  float* dst = static_cast<float*>(p.c) + (m0 + idx / C) * p.ldc + n0t + idx % C;
  *reinterpret_cast<f32x4_t*>(dst) = acc;
}

// The same for the 8-wave 256x192 tile in both products (64-wide K-tiles, two
// stages), which share their stage arrays.
template <int EKD>
__global__ __launch_bounds__(512) void gemm_bwd_pair256_kernel(GemmParams pw, GemmParams pd,
                                                               int nblk_w, int nblk_d,
                                                               GemmParams pr, int nfix_r,
                                                               int ncs_r, ColsumParams c2,
                                                               int c2_nchunks) {
  const int b = static_cast<int>(blockIdx.x);
  if (b < nblk_w) {
    gemm_pipe_block<256, 192, 4, 2, 64, 2, false, false, kEpiF32>(pw, b);
  } else if (b < nblk_w + nblk_d) {
    gemm_pipe_block<256, 192, 4, 2, 64, 2, true, true, EKD>(pd, b - nblk_w);
  } else {
    const int r = b - nblk_w - nblk_d;
    if (r < nfix_r) {
      splitk_fixup_vec4_unit(pr, static_cast<int64_t>(r) * blockDim.x + threadIdx.x,
                             static_cast<int64_t>(nfix_r) * blockDim.x);
    } else {
      constexpr int SB = (256 + 192) * 64 * 2;
      float(*part)[64] = reinterpret_cast<float(*)[64]>(stage_buf<0, SB>());
      if (r < nfix_r + ncs_r) colsum_pass2_unit(pr.cs, r - nfix_r, pr.cs_nchunks, part);
      else colsum_pass2_unit(c2, r - nfix_r - ncs_r, c2_nchunks, part);
    }
  }
}

// Epilogue kinds instantiated per layout (bf16) or operand formats (FP8):
// bf16 NN carries fc1's bias + GeLU, NT the dgrads, TN the weight gradients;
// FP8 E4M3 x E4M3 every kind, E5M2 x E4M3 (data gradients) the dgrad kinds,
// E4M3 x E5M2 (weight gradients) the fp32 store.
template <bool AK, bool BKC, int F8>
constexpr bool epi_instantiated(int ek) {
  if constexpr (F8 == 0) {
    return ek == kEpiF32 || (ek == kEpiBF16 && AK) || (ek == kEpiBiasGelu && AK && !BKC) ||
           (ek == kEpiDGelu && AK && BKC);
  } else {
    return F8 == 1 || ek == kEpiF32 || (F8 == 2 && (ek == kEpiBF16 || ek == kEpiDGelu));
  }
}

template <int BM, int BN, int WM, int WN, int BK, int S, bool AK, bool BKC, int F8 = 0>
hipError_t launch_pipe_cfg(const GemmParams& p, int splitk, int ek, hipStream_t s) {
  const int64_t tiles = (p.M / BM) * (p.N / BN);
  const dim3 grid(static_cast<unsigned>(tiles * splitk));
  const dim3 block(WM * WN * 64);
  switch (ek) {
    case kEpiF32:
      // column-sum blocks (if any) come last in dispatch order
      hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, BK, S, AK, BKC, kEpiF32, F8>),
                         dim3(grid.x + p.cs_blocks), block, 0, s, p);
      break;
    case kEpiBF16:
      if constexpr (epi_instantiated<AK, BKC, F8>(kEpiBF16))
        hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, BK, S, AK, BKC, kEpiBF16, F8>),
                           grid, block, 0, s, p);
      else
        return hipErrorInvalidValue;
      break;
    case kEpiBiasGelu:
      if constexpr (epi_instantiated<AK, BKC, F8>(kEpiBiasGelu))
        hipLaunchKernelGGL(
            (gemm_bf16_pipe_kernel<BM, BN, WM, WN, BK, S, AK, BKC, kEpiBiasGelu, F8>), grid,
            block, 0, s, p);
      else
        return hipErrorInvalidValue;
      break;
    case kEpiDGelu:
      if constexpr (epi_instantiated<AK, BKC, F8>(kEpiDGelu))
        hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, BK, S, AK, BKC, kEpiDGelu, F8>),
                           grid, block, 0, s, p);
      else
        return hipErrorInvalidValue;
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Tile configurations. A 32-wide K-tile of a K-contiguous operand is copied
// as 64-byte row pieces, half a 128-byte line each, which the vector memory
// path moves at about two thirds of its rate for whole lines. With both
// operands K-contiguous the 128-row tiles therefore take 64-wide K-tiles
// (three stages fit in LDS), and the 256x192 tile takes them in every layout,
// double-buffered (two 56 KiB stages): measured faster than four 32-wide
// stages even where both operands are M/N-contiguous, as it halves the
// block synchronisations per K.
template <bool AK, bool BKC>
hipError_t launch_pipe_layout(const GemmParams& p, const SplitPlan& plan, int ek, hipStream_t s) {
  constexpr bool kNT = AK && BKC;
  switch (plan.tile) {
    case kPipe256x256:
      return launch_pipe_cfg<256, 256, 2, 4, 32, 4, AK, BKC>(p, plan.splitk, ek, s);
    case kPipe256x128:
      return launch_pipe_cfg<256, 128, 2, 2, 32, 4, AK, BKC>(p, plan.splitk, ek, s);
    case kPipe128x256:
      return launch_pipe_cfg<128, 256, 2, 4, kNT ? 64 : 32, kNT ? 3 : 4, AK, BKC>(p, plan.splitk, ek,
                                                                                 s);
    case kPipe128x128:
      return launch_pipe_cfg<128, 128, 2, 2, kNT ? 64 : 32, kNT ? 3 : 4, AK, BKC>(p, plan.splitk, ek,
                                                                                 s);
    case kPipe256x192:
      return launch_pipe_cfg<256, 192, 4, 2, 64, 2, AK, BKC>(p, plan.splitk, ek, s);
    case kPipe128x192:
      return launch_pipe_cfg<128, 192, 2, 2, kNT ? 64 : 32, kNT ? 3 : 4, AK, BKC>(p, plan.splitk, ek,
                                                                                 s);
    default:
      return hipErrorInvalidValue;
  }
}

// FP8 tiles: 128-code (one line) K-tiles; three stages where they fit in LDS.
template <int F8>
hipError_t launch_fp8_tile(const GemmParams& p, const SplitPlan& plan, int ek, hipStream_t s) {
  switch (plan.tile) {
    case kPipe128x256:
      return launch_pipe_cfg<128, 256, 2, 4, 128, 3, true, true, F8>(p, plan.splitk, ek, s);
    case kPipe128x128:
      return launch_pipe_cfg<128, 128, 2, 2, 128, 3, true, true, F8>(p, plan.splitk, ek, s);
    case kPipe256x192:
      return launch_pipe_cfg<256, 192, 4, 2, 128, 2, true, true, F8>(p, plan.splitk, ek, s);
    case kPipe128x192:
      return launch_pipe_cfg<128, 192, 2, 2, 128, 3, true, true, F8>(p, plan.splitk, ek, s);
    default:
      return hipErrorInvalidValue;
  }
}

// Epilogue of an FP8 product; kEpiNone when the pipelined kernel cannot run it
// (there is no general FP8 kernel: the API rejects such calls).
int fp8_epilogue_kind(const GemmParams& p) {
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (p.splitk > 1)
    return (p.epi == EPI_STORE && a16(p.ws) && p.N % 8 == 0) ? kEpiF32 : kEpiNone;
  if (!a16(p.c) || p.ldc % 8) return kEpiNone;
  switch (p.epi) {
    case EPI_STORE:
      if (p.accumulate) return kEpiNone;
      return p.out_bf16 ? kEpiBF16 : kEpiF32;
    case EPI_BIAS_ACT:
      if (p.act == ACT_NONE && !p.bias && !p.c2) return p.out_bf16 ? kEpiBF16 : kEpiF32;
      if (p.act == ACT_GELU && p.out_bf16 && p.c2 && a16(p.c2) && p.ldc2 % 8 == 0 &&
          (!p.bias || a16(p.bias)))
        return kEpiBiasGelu;
      return kEpiNone;
    case EPI_DACT:
      if (p.act == ACT_GELU && p.out_bf16 && p.u && a16(p.u) && p.ldu % 8 == 0 &&
          (!p.c2 || (a16(p.c2) && p.ldc2 % 8 == 0)))
        return kEpiDGelu;
      return kEpiNone;
    default:
      return kEpiNone;
  }
}

// Blocks of a product on tile BM x BN (plus its column-sum units).
template <int BM, int BN>
int pair_blocks(const GemmParams& p) {
  return static_cast<int>((p.M / BM) * (p.N / BN) * p.splitk) + p.cs_blocks;
}

template <int BMW, int BNW, int BKW, int SW, int BMD, int BND, int BKD, int SD>
hipError_t launch_pair_cfg(const GemmParams& pw, const GemmParams& pd, int ekd,
                           const PairRider& rd, hipStream_t s) {
  const int nblk_w = pair_blocks<BMW, BNW>(pw);
  const int nblk_d = static_cast<int>((pd.M / BMD) * (pd.N / BND));
  const GemmParams pr = rd.p ? *rd.p : GemmParams{};
  const int nfix = rd.p ? rd.nfix : 0, ncs = rd.p ? rd.ncs : 0;
  const dim3 grid(static_cast<unsigned>(nblk_w + nblk_d + nfix + ncs + rd.ncs2)), block(256);
  switch (ekd) {
    case kEpiF32:
      hipLaunchKernelGGL((gemm_bwd_pair_kernel<BMW, BNW, BKW, SW, BMD, BND, BKD, SD, kEpiF32>),
                         grid, block, 0, s, pw, pd, nblk_w, nblk_d, pr, nfix, ncs,
                         rd.cs2, rd.cs2_nchunks);
      break;
    case kEpiBF16:
      hipLaunchKernelGGL((gemm_bwd_pair_kernel<BMW, BNW, BKW, SW, BMD, BND, BKD, SD, kEpiBF16>),
                         grid, block, 0, s, pw, pd, nblk_w, nblk_d, pr, nfix, ncs,
                         rd.cs2, rd.cs2_nchunks);
      break;
    case kEpiDGelu:
      hipLaunchKernelGGL((gemm_bwd_pair_kernel<BMW, BNW, BKW, SW, BMD, BND, BKD, SD, kEpiDGelu>),
                         grid, block, 0, s, pw, pd, nblk_w, nblk_d, pr, nfix, ncs,
                         rd.cs2, rd.cs2_nchunks);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_pair256(const GemmParams& pw, const GemmParams& pd, int ekd, const PairRider& rd,
                          hipStream_t s) {
  const int nblk_w = pair_blocks<256, 192>(pw);
  const int nblk_d = static_cast<int>((pd.M / 256) * (pd.N / 192));
  const GemmParams pr = rd.p ? *rd.p : GemmParams{};
  const int nfix = rd.p ? rd.nfix : 0, ncs = rd.p ? rd.ncs : 0;
  const dim3 grid(static_cast<unsigned>(nblk_w + nblk_d + nfix + ncs + rd.ncs2)), block(512);
  switch (ekd) {
    case kEpiF32:
      hipLaunchKernelGGL((gemm_bwd_pair256_kernel<kEpiF32>), grid, block, 0, s, pw, pd, nblk_w,
                         nblk_d, pr, nfix, ncs, rd.cs2, rd.cs2_nchunks);
      break;
    case kEpiBF16:
      hipLaunchKernelGGL((gemm_bwd_pair256_kernel<kEpiBF16>), grid, block, 0, s, pw, pd, nblk_w,
                         nblk_d, pr, nfix, ncs, rd.cs2, rd.cs2_nchunks);
      break;
    case kEpiDGelu:
      hipLaunchKernelGGL((gemm_bwd_pair256_kernel<kEpiDGelu>), grid, block, 0, s, pw, pd, nblk_w,
                         nblk_d, pr, nfix, ncs, rd.cs2, rd.cs2_nchunks);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_wgrad2(const GemmParams& a, const GemmParams& b, const WgradSplit& sp,
                              const RowSumParams* rs, hipStream_t s) {
  GemmParams p0 = a, p1 = b;
  p0.xcds = p1.xcds = device_shape().xcds;
  for (const GemmParams* q : {&p0, &p1})
    if (q->splitk != 1 || q->M % 128 || q->N % 128 || q->K % 32) return hipErrorInvalidValue;
  const int64_t nt0 = (p0.M / 128) * (p0.N / 128), nt1 = (p1.M / 128) * (p1.N / 128);
  if (sp.sk < 0 || sp.sk > kMaxSlices || sp.whole < 0 || sp.whole > nt0 + nt1 || (sp.sk == 0 && sp.whole != nt0 + nt1) ||
      (sp.sk > 0 && (!sp.part || p0.K != p1.K || p0.K % (32LL * sp.sk))))
    return hipErrorInvalidValue;
  const int64_t nsl = sp.sk > 0 ? (nt0 + nt1 - sp.whole) * sp.sk : 0;
  RowSumParams r{};
  if (rs) {
    r = *rs;
    auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    if (!r.parts || !r.out || !a16(r.parts) || !a16(r.out) || r.p < 1 || r.p > kMaxPartials || r.rows < 0 ||
        r.rows % kSumRows || r.N < 8 || r.N % 8 || r.ld_out < r.N || r.ld_out % 8)
      return hipErrorInvalidValue;
  }
  const int64_t nsum = r.rows / kSumRows;
  const int64_t grid = sp.whole + nsl + p0.cs_blocks + p1.cs_blocks + nsum;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(gemm_wgrad2_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, p0, p1,
                     static_cast<int>(nt0), static_cast<int>(nt1), sp, static_cast<int>(nsl), r);
  return hipGetLastError();
}

hipError_t launch_wgrad2_finish(const GemmParams& a, const GemmParams& b, const WgradSplit& sp,
                                int n0, int n1, hipStream_t s) {
  GemmParams p0 = a, p1 = b;
  p0.xcds = p1.xcds = device_shape().xcds;
  const int64_t nt0 = (p0.M / 128) * (p0.N / 128), nt1 = (p1.M / 128) * (p1.N / 128);
  if (sp.sk > kMaxSlices) return hipErrorInvalidValue;
  const int64_t nfix = sp.sk > 0 ? (kWg / kFinRows) * (nt0 + nt1 - sp.whole) : 0;
  const int64_t u0 = n0 > 1 ? (p0.cs.N + 63) / 64 : 0, u1 = n1 > 1 ? (p1.cs.N + 63) / 64 : 0;
  const int64_t grid = nfix + u0 + u1;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(wgrad2_finish_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, s, p0,
                     p1, static_cast<int>(nt0), sp, static_cast<int>(nfix), static_cast<int>(u0),
                     n0, n1);
  return hipGetLastError();
}

hipError_t launch_gemm_bwd_pair(const GemmParams& pw0, const GemmParams& pd0, int kind, int ekd,
                                const PairRider& rider, hipStream_t s) {
  GemmParams pw = pw0, pd = pd0;
  pw.xcds = pd.xcds = device_shape().xcds;
  switch (kind) {
    case kPairSame128x128:
      return launch_pair_cfg<128, 128, 64, 3, 128, 128, 64, 3>(pw, pd, ekd, rider, s);
    case kPairW128x128D128x192:
      return launch_pair_cfg<128, 128, 32, 4, 128, 192, 64, 3>(pw, pd, ekd, rider, s);
    case kPairSame256x192:
      return launch_pair256(pw, pd, ekd, rider, s);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_fp8(const GemmParams& p0, const SplitPlan& plan, hipStream_t s) {
  GemmParams p = p0;
  p.xcds = device_shape().xcds;
  const int ek = fp8_epilogue_kind(p);
  if (ek == kEpiNone) return hipErrorInvalidValue;
  switch (p.f8) {
    case 1:
      return launch_fp8_tile<1>(p, plan, ek, s);
    case 2:
      return launch_fp8_tile<2>(p, plan, ek, s);
    case 3:
      return launch_fp8_tile<3>(p, plan, ek, s);
    default:
      return hipErrorInvalidValue;
  }
}

int fp8_pipe_epilogue(const GemmParams& p) { return fp8_epilogue_kind(p); }

int pipe_epilogue_kind(const GemmParams& p) {
  auto a16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  if (p.splitk > 1) {
    return (p.epi == EPI_STORE && a16(p.ws) && p.N % 8 == 0) ? kEpiF32 : kEpiNone;
  }
  if (!a16(p.c) || p.ldc % 8) return kEpiNone;
  switch (p.epi) {
    case EPI_STORE:
      if (p.accumulate) return kEpiNone;
      if (!p.out_bf16) return kEpiF32;
      return p.a_kcontig ? kEpiBF16 : kEpiNone;
    case EPI_BIAS_ACT:
      // with no activation, no bias and no saved pre-activation it is a plain store
      if (p.act == ACT_NONE && !p.bias && !p.c2 && p.out_bf16 && p.a_kcontig) return kEpiBF16;
      if (p.act == ACT_GELU && p.out_bf16 && p.c2 && a16(p.c2) && p.ldc2 % 8 == 0 &&
          (!p.bias || a16(p.bias)) &&
          p.a_kcontig && !p.b_kcontig)
        return kEpiBiasGelu;
      return kEpiNone;
    case EPI_DACT:
      if (p.act == ACT_GELU && p.out_bf16 && p.u && a16(p.u) && p.ldu % 8 == 0 && p.a_kcontig &&
          p.b_kcontig && (!p.c2 || (a16(p.c2) && p.ldc2 % 8 == 0)))
        return kEpiDGelu;
      return kEpiNone;
    default:
      return kEpiNone;
  }
}

hipError_t launch_gemm_bf16_pipe(const GemmParams& p, const SplitPlan& plan, int ek,
                                 hipStream_t s) {
  if (p.a_kcontig && !p.b_kcontig) return launch_pipe_layout<true, false>(p, plan, ek, s);   // NN
  if (p.a_kcontig && p.b_kcontig) return launch_pipe_layout<true, true>(p, plan, ek, s);     // NT
  if (!p.a_kcontig && !p.b_kcontig) return launch_pipe_layout<false, false>(p, plan, ek, s); // TN
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
