// Pipelined bf16 GEMM for tile-aligned shapes on gfx950: operand tiles go from
// HBM straight into LDS (global_load_lds_dwordx4, no VGPR staging) through a
// ring of S stages, so S-1 K-tiles are in flight while the matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation) consume the current one.
//
// LDS layouts, each in the orientation the operand has in HBM:
//   K-contiguous operand (activations in NN/NT, the weight in NT):
//     ROWS x BK, one BK*2-byte row per output row; its 16-byte chunks are
//     XOR-swizzled by row so that the 16-byte fragment reads of 16 consecutive
//     rows at one K offset fall in distinct banks.
//   M/N-contiguous operand (the weight in NN, both operands in TN):
//     BK x ROWS, one ROWS*2-byte row per K; 16-byte chunks are XOR-swizzled by
//     4*(k mod 4). Fragments are read with ds_read_b64_tr_b16, which hands each
//     lane four consecutive K-values of its own column: within a 16-lane group,
//     lane i receives element i%4 of the 8-byte words read by lanes i/4,
//     i/4+4, i/4+8 and i/4+12. Two such reads give the 8 K-values of a
//     32x32x16 operand, in the same order a 16-byte read gives them for the
//     K-contiguous operand.
// A copy instruction writes 64 lanes x 16 bytes to a contiguous 1 KiB window of
// LDS; the swizzle is realised by choosing which global chunk each lane fetches.
//
// Each stage is a separate __shared__ object so the compiler can tell the
// stages apart and does not wait for copies into other stages before reading
// one. The steady-state loop issues one K-tile per step with no conditionals;
// the last steps run in a guarded tail with conservative waits.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace tpmlp {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

template <int J, int BYTES>
__device__ __forceinline__ uint8_t* stage_buf() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[BYTES];
  return buf;
}

__device__ __forceinline__ void copy16_to_lds(const uint16_t* g, uint8_t* lds) {
  // address-space casts (global = 1, LDS = 3) need C-style casts
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14;
// expcnt and lgkmcnt left at their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 32-bit LDS byte address of a pointer into a __shared__ buffer.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

// Wait for this wave's outstanding LDS reads; the fragments pass through the
// statement so that no instruction reading them is scheduled before the wait.
template <int NF>
__device__ __forceinline__ void lds_fence(bf16x8_t (&f)[NF]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < NF; ++i) asm volatile("" : "+v"(f[i]));
}

__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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

// ---------------------------------------------------------------------------
// Operand tiles
// ---------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (BK == 64) return (r ^ (r >> 3)) & 7;
  else return (r >> 2) & 3;
}

template <bool KC, int ROWS, int BK, int NW>
struct Operand {
  static constexpr int BYTES = ROWS * BK * 2;
  static constexpr int NI = BYTES / 1024 / NW;  // copy instructions per wave per tile
  static_assert(NI >= 1 && NI * 1024 * NW == BYTES, "tile / waves mismatch");
  static_assert(KC || ROWS % 128 == 0, "M/N-contiguous tiles need 16-chunk rows");
  static_assert(BK == 32 || BK == 64, "K tile");

  const uint16_t* ptr[NI];
  int64_t adv;  // elements between consecutive K-tiles

  // Tile origin (row r0 of M/N, k0 of K); ld = row stride of the operand in HBM.
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int64_t r0, int64_t k0,
                                       int wave, int lane) {
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      const int byte = (wave * NI + q) * 1024 + lane * 16;
      if constexpr (KC) {
        const int r = byte / (BK * 2);
        const int c = ((byte % (BK * 2)) >> 4) ^ kswz<BK>(r);
        ptr[q] = base + (r0 + r) * ld + k0 + c * 8;
      } else {
        const int k = byte / (ROWS * 2);
        const int c = ((byte % (ROWS * 2)) >> 4) ^ (4 * (k & 3));
        ptr[q] = base + (k0 + k) * ld + r0 + c * 8;
      }
    }
    adv = KC ? BK : BK * ld;
  }

  // Copy the next K-tile into the stage at lds (this operand's part of it).
  __device__ __forceinline__ void issue(uint8_t* lds, int wave) {
#pragma unroll
    for (int q = 0; q < NI; ++q) {
      copy16_to_lds(ptr[q], lds + (wave * NI + q) * 1024);
      ptr[q] += adv;
    }
  }

  // 32x32x16 fragment: rows (M or N) R0 .. R0+31, K = 16*ks .. 16*ks+15.
  // K-contiguous operand: one 16-byte read. M/N-contiguous operand: two
  // transposed 8-byte reads. Both are issued as inline assembly, so the
  // compiler neither waits for unrelated copies in flight before them nor
  // knows when their data arrives: a fragment is valid only after lds_fence().
  __device__ __forceinline__ static bf16x8_t frag(const uint8_t* lds, int R0, int ks, int lane) {
    bf16x8_t f;
    if constexpr (KC) {
      const int r = R0 + (lane & 31);
      const int c = ks * 2 + (lane >> 5);
      const uint32_t a = lds_addr(lds) + r * (BK * 2) + ((c ^ kswz<BK>(r)) << 4);
      asm volatile("ds_read_b128 %0, %1" : "=v"(f) : "v"(a));
    } else {
      const int g = lane >> 4, s = lane & 15;
      const int mn = R0 + 16 * (g & 1) + 4 * (s & 3);
      const int kb = ks * 16 + 8 * (g >> 1) + (s >> 2);
      const int sw = 4 * (s >> 2);  // 4 * (k & 3)
      const uint32_t a0 = lds_addr(lds) + kb * (ROWS * 2) + (((mn >> 3) ^ sw) << 4) + (mn & 7) * 2;
      const uint32_t a1 = a0 + 4 * (ROWS * 2);
      s16x4_t lo, hi;
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(a0));
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(hi) : "v"(a1));
      f = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    return f;
  }
};

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int BK, int S, bool AK, bool BKC>
__global__ __launch_bounds__(WM* WN * 64) void gemm_bf16_pipe_kernel(GemmParams p) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM * 32 * WM == BM && FN * 32 * WN == BN, "tile");
  static_assert(S >= 3 && S <= 4, "stages");
  using OA = Operand<AK, BM, BK, NW>;
  using OB = Operand<BKC, BN, BK, NW>;
  constexpr int SB = OA::BYTES + OB::BYTES;  // bytes per stage
  constexpr int NIT = OA::NI + OB::NI;       // copies per wave per K-tile

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // ---- output tile (same XCD-aware order as the general kernel)
  const int tiles_m = static_cast<int>(p.M / BM);
  const int tiles_n = static_cast<int>(p.N / BN);
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  constexpr int G = 8;
  const int group = bid / (G * tiles_n);
  const int first_m = group * G;
  const int gs = min(tiles_m - first_m, G);
  const int in_group = bid - group * G * tiles_n;
  const int64_t m0 = static_cast<int64_t>(first_m + in_group % gs) * BM;
  const int64_t n0 = static_cast<int64_t>(in_group / gs) * BN;

  const int z = blockIdx.y;
  const int64_t kbeg = static_cast<int64_t>(z) * p.k_chunk;
  const int nk = static_cast<int>((min(p.K, kbeg + p.k_chunk) - kbeg) / BK);

  OA oa;
  OB ob;
  oa.init(static_cast<const uint16_t*>(p.a), p.lda, m0, kbeg, wave, lane);
  ob.init(static_cast<const uint16_t*>(p.b), p.ldb, n0, kbeg, wave, lane);

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  auto issue = [&](auto stage_c) {
    constexpr int J = decltype(stage_c)::value;
    uint8_t* st = stage_buf<J, SB>();
    oa.issue(st, wave);
    ob.issue(st + OA::BYTES, wave);
  };
  // One K-tile from one stage. Fragments of K-step ks+1 are read while the
  // matrix cores work on K-step ks.
  auto compute = [&](auto stage_c) {
    constexpr int J = decltype(stage_c)::value;
    const uint8_t* sa = stage_buf<J, SB>();
    const uint8_t* sb = sa + OA::BYTES;
    bf16x8_t f[2][FM + FN];
    auto read = [&](int ks, bf16x8_t(&d)[FM + FN]) {
#pragma unroll
      for (int i = 0; i < FM; ++i) d[i] = OA::frag(sa, wm * WTM + i * 32, ks, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) d[FM + j] = OB::frag(sb, wn * WTN + j * 32, ks, lane);
    };
    read(0, f[0]);
    lds_fence(f[0]);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) read(ks + 1, f[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks & 1][i], f[ks & 1][FM + j],
                                                              acc[i][j], 0, 0, 0);
      if (ks + 1 < BK / 16) lds_fence(f[(ks + 1) & 1]);
    }
  };

  // ---- prologue: K-tiles 0 .. S-2 into stages 0 .. S-2
  Unroll<0, S - 1>::run([&](auto jc) {
    if (decltype(jc)::value < nk) issue(jc);
  });

  // ---- steady state: every step also prefetches K-tile it+S-1
  int it0 = 0;
  for (; it0 + 2 * S - 1 <= nk; it0 += S) {
    Unroll<0, S>::run([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      wait_vmcnt<(S - 2) * NIT>();
      block_sync();
      issue(std::integral_constant<int, (J + S - 1) % S>{});
      compute(jc);
    });
  }
  // ---- tail
  for (; it0 < nk; it0 += S) {
    Unroll<0, S>::run([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      const int it = it0 + J;
      if (it < nk) {
        const int after = min(S - 2, nk - 1 - it);  // K-tiles issued after this one
        if (after >= 2) wait_vmcnt<2 * NIT>();
        else if (after == 1) wait_vmcnt<NIT>();
        else wait_vmcnt<0>();
        block_sync();
        if (it + S - 1 < nk) issue(std::integral_constant<int, (J + S - 1) % S>{});
        compute(jc);
      }
    });
  }
  wait_vmcnt<0>();
  block_sync();

  // ---- epilogue through LDS (per-wave regions inside the stage buffers)
  constexpr int EP = WTN + 4;
  constexpr int REGION = 32 * EP * 4;
  constexpr int WPS = SB / REGION;  // wave regions per stage
  static_assert(WPS >= 1 && WPS * S >= NW, "epilogue LDS");
  constexpr int VPR = WTN / 8;      // 8-column vectors per tile row
  static_assert((32 * VPR) % 64 == 0, "epilogue passes");
  const int ws_idx = wave / WPS;
  uint8_t* base = ws_idx == 0 ? stage_buf<0, SB>()
                : ws_idx == 1 ? stage_buf<1, SB>()
                : ws_idx == 2 ? stage_buf<2, SB>()
                              : stage_buf<(S > 3 ? 3 : 2), SB>();
  float* ep = reinterpret_cast<float*>(base + (wave % WPS) * REGION);
  const bool split = p.splitk > 1;
  float* wsz = split ? p.ws + static_cast<int64_t>(z) * p.M * p.N : nullptr;
  const bool out_vec = split ? ((reinterpret_cast<uintptr_t>(p.ws) & 15) == 0 && (p.N & 7) == 0)
                             : epilogue_vec_ok(p);
  Unroll<0, FM>::run([&](auto band) {
    constexpr int i = decltype(band)::value;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ep[((r >> 2) * 8 + 4 * (lane >> 5) + (r & 3)) * EP + j * 32 + (lane & 31)] = acc[i][j][r];
    block_sync();
#pragma unroll
    for (int pass = 0; pass < 32 * VPR / 64; ++pass) {
      const int v = pass * 64 + lane;
      const int lr = v / VPR, ec = (v % VPR) * 8;
      const float* src = ep + lr * EP + ec;
      const f32x4_t lo = *reinterpret_cast<const f32x4_t*>(src);
      const f32x4_t hi = *reinterpret_cast<const f32x4_t*>(src + 4);
      float vals[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        vals[q] = lo[q];
        vals[q + 4] = hi[q];
      }
      const int64_t row = m0 + wm * WTM + i * 32 + lr;
      const int64_t col = n0 + wn * WTN + ec;
      if (split) {
        if (out_vec) {
          float* d = wsz + row * p.N + col;
          *reinterpret_cast<f32x4_t*>(d) = lo;
          *reinterpret_cast<f32x4_t*>(d + 4) = hi;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) wsz[row * p.N + col + q] = vals[q];
        }
      } else if (out_vec) {
        epilogue_vec8(p, row, col, vals);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) epilogue_elem(p, row, col + q, vals[q], 1);
      }
    }
    block_sync();
  });
}

template <int BM, int BN, int WM, int WN, int BK, int S, bool AK, bool BKC>
hipError_t launch_pipe_cfg(const GemmParams& p, int splitk, hipStream_t s) {
  const int64_t tiles = (p.M / BM) * (p.N / BN);
  hipLaunchKernelGGL((gemm_bf16_pipe_kernel<BM, BN, WM, WN, BK, S, AK, BKC>),
                     dim3(static_cast<unsigned>(tiles), static_cast<unsigned>(splitk)),
                     dim3(WM * WN * 64), 0, s, p);
  return hipGetLastError();
}

template <bool AK, bool BKC>
hipError_t launch_pipe_layout(const GemmParams& p, const SplitPlan& plan, hipStream_t s) {
  switch (plan.tile) {
    case kPipe256x256:
      return launch_pipe_cfg<256, 256, 2, 2, 32, 4, AK, BKC>(p, plan.splitk, s);
    case kPipe256x128:
      return launch_pipe_cfg<256, 128, 2, 2, 32, 4, AK, BKC>(p, plan.splitk, s);
    case kPipe128x256:
      return launch_pipe_cfg<128, 256, 2, 2, 32, 4, AK, BKC>(p, plan.splitk, s);
    case kPipe128x128:
      return launch_pipe_cfg<128, 128, 2, 2, 32, 4, AK, BKC>(p, plan.splitk, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gemm_bf16_pipe(const GemmParams& p, const SplitPlan& plan, hipStream_t s) {
  if (p.a_kcontig && !p.b_kcontig) return launch_pipe_layout<true, false>(p, plan, s);    // NN
  if (p.a_kcontig && p.b_kcontig) return launch_pipe_layout<true, true>(p, plan, s);      // NT
  if (!p.a_kcontig && !p.b_kcontig) return launch_pipe_layout<false, false>(p, plan, s);  // TN
  return hipErrorInvalidValue;
}

}  // namespace tpmlp
