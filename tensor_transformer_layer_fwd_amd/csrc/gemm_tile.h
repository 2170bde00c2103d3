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
//     4*(k mod 4) (ROWS = 128, 256) or rotated by 4*((k/2) mod 2) (ROWS = 192,
//     whose 384-byte rows already put odd K rows half a bank cycle apart), so
//     that the four K rows one transposed read touches hit disjoint banks.
//     Fragments are read with ds_read_b64_tr_b16, which hands each
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
// one. The block synchronises once per K-tile, just before the matrix cores
// start on the tile's last 16-wide K step: by then every wave holds that
// step's fragments in registers, so the tile's own stage can be refilled with
// K-tile t+S at once, and the first fragments of K-tile t+1 are read while the
// last MFMAs of tile t run. A wave therefore never waits on LDS between
// K-tiles, and all S stages are in flight. The steady-state loop has no
// conditionals; the last steps run in a guarded tail with conservative waits.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "colsum_device.h"
#include "device_common.h"
#include "internal.h"

namespace tpmlp {
namespace {

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));

template <int J, int BYTES>
__device__ __forceinline__ uint8_t* stage_buf() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[BYTES];
  return buf;
}

// One LDS array for a launch whose blocks run products of different tiles:
// stage J of a product with stage size SB at byte J * SB (multiples of 1 KiB).
template <int BYTES>
__device__ __forceinline__ uint8_t* pool_buf() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[BYTES];
  return buf;
}

// Stage J: its own array (POOL = 0), or inside a pool of POOL bytes.
template <int J, int SB, int POOL>
__device__ __forceinline__ uint8_t* stage_ptr() {
  if constexpr (POOL == 0) {
    return stage_buf<J, SB>();
  } else {
    static_assert((J + 1) * SB <= POOL && SB % 1024 == 0, "pool");
    return pool_buf<POOL>() + J * SB;
  }
}

__device__ __forceinline__ void copy16_to_lds(const void* g, uint8_t* lds) {
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
template <typename FT, int NF>
__device__ __forceinline__ void lds_fence(FT (&f)[NF]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < NF; ++i) asm volatile("" : "+v"(f[i]));
}
__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Operand tiles
// ---------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ int kswz(int r) {
  if constexpr (BK == 64) return (r ^ (r >> 3)) & 7;
  else return (r >> 2) & 3;
}

// M/N-contiguous tiles: physical 16-byte chunk of logical chunk c in K row k,
// and the inverse map.
template <int ROWS>
__device__ __forceinline__ int mn_phys(int k, int c) {
  if constexpr (ROWS % 128 == 0) return c ^ (4 * (k & 3));
  else return (c + 4 * ((k >> 1) & 1)) % (ROWS / 8);
}
template <int ROWS>
__device__ __forceinline__ int mn_logical(int k, int pc) {
  if constexpr (ROWS % 128 == 0) return pc ^ (4 * (k & 3));
  else return (pc + ROWS / 8 - 4 * ((k >> 1) & 1)) % (ROWS / 8);
}

template <bool KC, int ROWS, int BK, int NW>
struct Operand {
  static constexpr int BYTES = ROWS * BK * 2;
  // A copy instruction fills one 1 KiB window of the tile. Window q*NW + w is
  // copied by wave w; when the windows do not divide evenly among the waves,
  // the first EXTRA waves copy one more.
  static constexpr int NWIN = BYTES / 1024;
  static constexpr int NB = NWIN / NW;
  static constexpr int EXTRA = NWIN % NW;
  static_assert(NB >= 1 && NWIN * 1024 == BYTES, "tile / waves mismatch");
  static_assert(KC || ROWS % 128 == 0 || ROWS == 192, "M/N-contiguous tile rows");
  static_assert(BK == 32 || BK == 64, "K tile");

  const uint16_t* ptr[NB + (EXTRA > 0)];
  int64_t adv;  // elements between consecutive K-tiles

  // Tile origin (row r0 of M/N, k0 of K); ld = row stride of the operand in HBM.
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int64_t r0, int64_t k0,
                                       int wave, int lane) {
#pragma unroll
    for (int q = 0; q < NB + (EXTRA > 0); ++q) {
      // a wave without an extra window points its extra copy at window 0 (never issued)
      const int win = q < NB ? q * NW + wave : (wave < EXTRA ? NB * NW + wave : 0);
      const int byte = win * 1024 + lane * 16;
      if constexpr (KC) {
        const int r = byte / (BK * 2);
        const int c = ((byte % (BK * 2)) >> 4) ^ kswz<BK>(r);
        ptr[q] = base + (r0 + r) * ld + k0 + c * 8;
      } else {
        const int k = byte / (ROWS * 2);
        const int c = mn_logical<ROWS>(k, (byte % (ROWS * 2)) >> 4);
        ptr[q] = base + (k0 + k) * ld + r0 + c * 8;
      }
    }
    adv = KC ? BK : BK * ld;
  }

  // Copy the next K-tile into the stage at lds (this operand's part of it):
  // the windows every wave copies, and the extra one of waves below EXTRA
  // (`extra` must be wave-uniform).
  __device__ __forceinline__ void issue(uint8_t* lds, int wave) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      copy16_to_lds(ptr[q], lds + (q * NW + wave) * 1024);
      ptr[q] += adv;
    }
  }
  __device__ __forceinline__ void issue_extra(uint8_t* lds, int wave, bool extra) {
    if constexpr (EXTRA > 0) {
      if (extra) copy16_to_lds(ptr[NB], lds + (NB * NW + wave) * 1024);
      ptr[NB] += adv;
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
      // K rows kb and kb+4 share the chunk permutation
      const uint32_t a0 =
          lds_addr(lds) + kb * (ROWS * 2) + (mn_phys<ROWS>(kb, mn >> 3) << 4) + (mn & 7) * 2;
      const uint32_t a1 = a0 + 4 * (ROWS * 2);
      s16x4_t lo, hi;
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(lo) : "v"(a0));
      asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(hi) : "v"(a1));
      f = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    return f;
  }
};

// FP8 operand, K-contiguous codes: a K-tile is 128 codes, one 128-byte line
// per row, swizzled like the 64-wide bf16 K-tile (same bytes per row). A
// v_mfma_f32_32x32x64_f8f6f4 operand is 32 bytes per lane: row R0 + lane%32,
// K bytes 64*ks + 32*(lane/32) .. +31, read as two 16-byte chunks. Which K a
// byte position feeds inside the instruction does not matter: A and B use the
// same positions, and a dot product is invariant under a common permutation
// of K.
template <int ROWS, int NW>
struct OperandF8 {
  static constexpr int BK = 128;
  static constexpr int BYTES = ROWS * BK;
  static constexpr int NWIN = BYTES / 1024;
  static constexpr int NB = NWIN / NW;
  static constexpr int EXTRA = NWIN % NW;
  static_assert(NB >= 1 && NWIN * 1024 == BYTES, "tile / waves mismatch");

  const uint8_t* ptr[NB + (EXTRA > 0)];

  __device__ __forceinline__ void init(const uint8_t* base, int64_t ld, int64_t r0, int64_t k0,
                                       int wave, int lane) {
#pragma unroll
    for (int q = 0; q < NB + (EXTRA > 0); ++q) {
      const int win = q < NB ? q * NW + wave : (wave < EXTRA ? NB * NW + wave : 0);
      const int byte = win * 1024 + lane * 16;
      const int r = byte / BK;
      const int c = ((byte % BK) >> 4) ^ kswz<64>(r);
      ptr[q] = base + (r0 + r) * ld + k0 + c * 16;
    }
  }
  __device__ __forceinline__ void issue(uint8_t* lds, int wave) {
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      copy16_to_lds(ptr[q], lds + (q * NW + wave) * 1024);
      ptr[q] += BK;
    }
  }
  __device__ __forceinline__ void issue_extra(uint8_t* lds, int wave, bool extra) {
    if constexpr (EXTRA > 0) {
      if (extra) copy16_to_lds(ptr[NB], lds + (NB * NW + wave) * 1024);
      ptr[NB] += BK;
    }
  }
  __device__ __forceinline__ static i32x8_t frag(const uint8_t* lds, int R0, int ks, int lane) {
    const int r = R0 + (lane & 31);
    const int c = 4 * ks + 2 * (lane >> 5);
    const uint32_t row = lds_addr(lds) + r * BK;
    const uint32_t a0 = row + ((c ^ kswz<64>(r)) << 4), a1 = row + (((c + 1) ^ kswz<64>(r)) << 4);
    i32x4_t lo, hi;
    asm volatile("ds_read_b128 %0, %1" : "=v"(lo) : "v"(a0));
    asm volatile("ds_read_b128 %0, %1" : "=v"(hi) : "v"(a1));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
};

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------
// Rows of a tile group when each XCD takes c consecutive tiles of the grouped
// column-major order. A run of c tiles is a g x (c/g) rectangle when g divides
// c and tiles_m and c divides g * tiles_n; the rectangle reads g*BM + (c/g)*BN
// operand rows per K step into the XCD's L2. The default of 8 rows is kept
// unless a rectangle reads at most 4/5 of what 8 rows (and ceil(c/8) columns)
// read: that happens for small grids, such as 9 weight-gradient tiles per XCD
// (3 x 3 instead of a column of 8 and one more tile).
__device__ __forceinline__ int xcd_group_rows(int c, int tiles_m, int tiles_n, int BM, int BN) {
  const int base = 8 * BM + ((c + 7) / 8) * BN;
  int best = 8, cost = base;
  for (int g = 8; g >= 1; --g) {
    if (c % g != 0 || tiles_m % g != 0 || (g * tiles_n) % c != 0) continue;
    const int w = g * BM + (c / g) * BN;
    if (w < cost) {
      cost = w;
      best = g;
    }
  }
  return 5 * cost <= 4 * base ? best : 8;
}

// Origin (m0, n0) of output tile `bid` of a product's grid of BM x BN tiles.
// Blocks go round-robin over the XCDs, so each XCD takes a run of consecutive
// tiles of a grouped column-major order (groups of xcd_group_rows rows).
template <int BM, int BN>
__device__ __forceinline__ void tile_origin(const GemmParams& p, int bid, int64_t* m0,
                                            int64_t* n0) {
  const int tiles_m = static_cast<int>(p.M / BM);
  const int tiles_n = static_cast<int>(p.N / BN);
  const int ntiles = tiles_m * tiles_n;
  int G = 8;
  const int X = p.xcds;
  if (X > 1 && ntiles % X == 0) {
    bid = (bid % X) * (ntiles / X) + bid / X;
    G = xcd_group_rows(ntiles / X, tiles_m, tiles_n, BM, BN);
  }
  const int group = bid / (G * tiles_n);
  const int first_m = group * G;
  const int gs = min(tiles_m - first_m, G);
  const int in_group = bid - group * G * tiles_n;
  *m0 = static_cast<int64_t>(first_m + in_group % gs) * BM;
  *n0 = static_cast<int64_t>(in_group / gs) * BN;
}

// F8 = 0: bf16 operands; F8 = 1 + fmt_a + 2 * fmt_b: FP8 codes (both operands
// K-contiguous, BK = 128 codes), fmt 0 = E4M3, 1 = E5M2.
// One output tile of a product: rows m0 .. m0+BM-1, columns n0 .. n0+BN-1,
// over nk K-tiles from kbeg (K slice z for the split-K partials). Every thread
// of the block calls it; it leaves the LDS pool free (the block synchronised)
// only after its epilogue's last LDS access, so a caller that reuses the pool
// synchronises first.
template <int BM, int BN, int WM, int WN, int BK, int S, bool AK, bool BKC, int EK, int F8 = 0,
          int POOL = 0>
__device__ __forceinline__ void gemm_pipe_tile(const GemmParams& p, const int64_t m0,
                                               const int64_t n0, const int z, const int64_t kbeg,
                                               const int nk) {
  constexpr int NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  static_assert(FM * 32 * WM == BM && FN * 32 * WN == BN, "tile");
  static_assert(S >= 2 && S <= 8, "stages");
  static_assert(F8 == 0 || (AK && BKC && BK == 128), "FP8: K-contiguous operands, 128-code K-tiles");
  using OA = std::conditional_t<(F8 > 0), OperandF8<BM, NW>, Operand<AK, BM, BK, NW>>;
  using OB = std::conditional_t<(F8 > 0), OperandF8<BN, NW>, Operand<BKC, BN, BK, NW>>;
  using FragT = std::conditional_t<(F8 > 0), i32x8_t, bf16x8_t>;
  constexpr int SB = OA::BYTES + OB::BYTES;  // bytes per stage
  // copies per wave per K-tile: NIT, plus one for each operand with an extra
  // window for this wave
  constexpr int NIT = OA::NB + OB::NB;
  static_assert(OA::EXTRA == 0 || OB::EXTRA == 0, "extra windows in one operand only");
  static_assert(POOL == 0 || S * SB <= POOL, "stages exceed the LDS pool");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int wm = wave / WN, wn = wave % WN;

  OA oa;
  OB ob;
  if constexpr (F8 > 0) {
    oa.init(static_cast<const uint8_t*>(p.a), p.lda, m0, kbeg, wave, lane);
    ob.init(static_cast<const uint8_t*>(p.b), p.ldb, n0, kbeg, wave, lane);
  } else {
    oa.init(static_cast<const uint16_t*>(p.a), p.lda, m0, kbeg, wave, lane);
    ob.init(static_cast<const uint16_t*>(p.b), p.ldb, n0, kbeg, wave, lane);
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  constexpr int NX = OA::EXTRA + OB::EXTRA;  // waves 0..NX-1 copy NIT+1 windows per K-tile
  const bool xw = wave < NX;
  auto issue = [&](auto stage_c) {
    constexpr int J = decltype(stage_c)::value;
    uint8_t* st = stage_ptr<J, SB, POOL>();
    oa.issue(st, wave);
    ob.issue(st + OA::BYTES, wave);
  };
  auto issue_extra = [&](auto stage_c) {
    constexpr int J = decltype(stage_c)::value;
    uint8_t* st = stage_ptr<J, SB, POOL>();
    oa.issue_extra(st, wave, xw);
    ob.issue_extra(st + OA::BYTES, wave, xw);
  };
  // Wait until at most T K-tiles of this wave's copies are in flight.
  auto wait_tiles = [&](auto tiles_c) {
    constexpr int T = decltype(tiles_c)::value;
    if constexpr (NX == 0) {
      wait_vmcnt<T * NIT>();
    } else {
      if (xw) wait_vmcnt<T*(NIT + 1)>();
      else wait_vmcnt<T * NIT>();
    }
  };
  auto wait_after = [&](int after) {  // 0 <= after < S
    Unroll<0, S>::run([&](auto c) {
      if (after == decltype(c)::value) wait_tiles(c);
    });
  };
  constexpr int KS = F8 > 0 ? BK / 64 : BK / 16;  // MFMA K steps per K-tile
  FragT f[2][FM + FN];         // fragments of K step ks live in f[ks & 1]
  auto read = [&](auto stage_c, int ks, FragT(&d)[FM + FN]) {
    constexpr int J = decltype(stage_c)::value;
    const uint8_t* sa = stage_ptr<J, SB, POOL>();
    const uint8_t* sb = sa + OA::BYTES;
#pragma unroll
    for (int i = 0; i < FM; ++i) d[i] = OA::frag(sa, wm * WTM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) d[FM + j] = OB::frag(sb, wn * WTN + j * 32, ks, lane);
  };
  auto mfma = [&](const FragT(&d)[FM + FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (F8 > 0) {
          // operand formats are immediates; scales 0 select the unscaled instruction
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              d[i], d[FM + j], acc[i][j], (F8 - 1) & 1, (F8 - 1) >> 1, 0, 0, 0, 0);
        } else {
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(d[i], d[FM + j], acc[i][j], 0, 0, 0);
        }
      }
  };
  // One K-tile from stage J; its first fragments are already in f[0]. Before
  // the last K step, sync() synchronises the block (and issues the uneven
  // extra window copies into stage J); then the first fragments of the next
  // K-tile (stage J+1) are read and refill() reloads the rest of stage J while
  // the last MFMAs run. Scheduling barriers keep each K step in the order:
  // fragment reads for the next step, the MFMAs (with the tile copies of the
  // last step spread between them), the wait for the reads. Left alone, the
  // compiler sinks the reads to the end of the MFMAs, where their latency
  // shows, and bunches the copies.
  auto tile = [&](auto stage_c, auto&& sync, auto&& refill, bool has_next) {
    constexpr int J = decltype(stage_c)::value;
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      read(stage_c, ks + 1, f[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
      mfma(f[ks & 1]);
      __builtin_amdgcn_sched_barrier(0);
      lds_fence(f[(ks + 1) & 1]);
    }
    if (has_next) {
      sync();
      read(std::integral_constant<int, (J + 1) % S>{}, 0, f[0]);
    }
    __builtin_amdgcn_sched_barrier(0);
    refill();
    mfma(f[(KS - 1) & 1]);
#pragma unroll
    for (int q = 0; q < NIT; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // one copy
    }
    __builtin_amdgcn_sched_barrier(0);
    if (has_next) lds_fence(f[0]);
  };

  // ---- prologue: K-tiles 0 .. S-1 into all stages, first fragments of tile 0
  Unroll<0, S>::run([&](auto jc) {
    if (decltype(jc)::value < nk) {
      issue(jc);
      issue_extra(jc);
    }
  });
  wait_after(min(S - 1, nk - 1));
  block_sync();
  read(std::integral_constant<int, 0>{}, 0, f[0]);
  lds_fence(f[0]);

  // ---- steady state: K-tile t refills its own stage with K-tile t+S
  int it0 = 0;
  for (; it0 + 2 * S <= nk; it0 += S) {
    Unroll<0, S>::run([&](auto jc) {
      tile(
          jc,
          [&] {
            wait_tiles(std::integral_constant<int, S - 2>{});
            block_sync();
            issue_extra(jc);
          },
          [&] { issue(jc); }, true);
    });
  }
  // ---- tail
  for (; it0 < nk; it0 += S) {
    Unroll<0, S>::run([&](auto jc) {
      const int t = it0 + decltype(jc)::value;
      if (t < nk) {
        tile(
            jc,
            [&] {
              wait_after(min(S - 2, nk - 2 - t));  // K-tiles issued after tile t+1
              block_sync();
              if (t + S < nk) issue_extra(jc);
            },
            [&] {
              if (t + S < nk) issue(jc);
            },
            t + 1 < nk);
      }
    });
  }
  wait_vmcnt<0>();
  block_sync();
  if constexpr (F8 > 0) {  // dequantisation: 1/sa * 1/sb
    const float sc = p.sa_inv[0] * p.sb_inv[0];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] *= sc;
  }

  // ---- epilogue through LDS (per-wave regions inside the stage buffers).
  // For each 32-row band of its wave tile a wave writes the accumulators to
  // LDS in the 32x32 MFMA layout (lane holds column lane & 31; register r holds
  // row 8*(r/4) + 4*(lane/32) + r%4) and reads them back as 8 consecutive
  // columns per lane, which it finishes with 16-byte stores. The wave tile's
  // columns go in chunks of up to 64: a 64-wide chunk is 8 lanes wide and 8
  // rows deep per pass, a 32-wide one 4 lanes wide and 16 rows deep. A lane's
  // columns are the same in every band, so the bias is loaded once; the saved
  // pre-activation U of band i+1 is loaded before the stores of band i (on
  // gfx9 loads and stores share one counter: a load issued after stores could
  // only be waited for together with them).
  constexpr int EP = WTN + 4;
  constexpr int REGION = 32 * EP * 4;
  constexpr int WPS = SB / REGION;  // wave regions per stage
  static_assert(WPS >= 1 && WPS * S >= NW, "epilogue LDS");
  constexpr int NCH = (WTN + 63) / 64;  // column chunks
  constexpr int NPB = WTN / 16;         // passes per band, all chunks
  const int ws_idx = wave / WPS;
  uint8_t* base = stage_ptr<0, SB, POOL>();
  Unroll<1, S>::run([&](auto c) {
    if (ws_idx == decltype(c)::value) base = stage_ptr<decltype(c)::value, SB, POOL>();
  });
  const float* ep = reinterpret_cast<const float*>(base + (wave % WPS) * REGION);
  const int64_t col0 = n0 + wn * WTN;
  const int64_t rowt = m0 + wm * WTM;
  // chunk C = P / 4 of pass P: width, lanes per row, rows per pass, lane offsets
  auto chunk_w = [](int C) { return WTN - 64 * C < 64 ? WTN - 64 * C : 64; };
  // fp32 output: C, or this K slice's partial sums (row stride N) when split
  constexpr bool F32OUT = EK == kEpiF32;
  float* const cf = EK == kEpiF32 ? (p.splitk > 1 ? p.ws + static_cast<int64_t>(z) * p.M * p.N
                                                  : static_cast<float*>(p.c))
                                  : nullptr;
  const int64_t ldc = (EK == kEpiF32 && p.splitk > 1) ? p.N : p.ldc;

  float amax_run = 0.0f;  // largest |stored value| of this lane (amax epilogues)
  float bias8[NCH][8];
#pragma unroll
  for (int C = 0; C < NCH; ++C) {
#pragma unroll
    for (int q = 0; q < 8; ++q) bias8[C][q] = 0.0f;
    const int vpr = chunk_w(C) / 8;
    if (EK == kEpiBiasGelu && p.bias) load8_bf16(p.bias, col0 + 64 * C + (lane % vpr) * 8, bias8[C]);
  }
  u32x4_t upre[2][NPB];
  const uint16_t* Ug = static_cast<const uint16_t*>(p.u);
  auto load_u = [&](int i, u32x4_t(&d)[NPB]) {
#pragma unroll
    for (int P = 0; P < NPB; ++P) {
      const int C = P >> 2, ps = P & 3;
      const int vpr = chunk_w(C) / 8, rpp = 64 / vpr;
      const int64_t row = rowt + i * 32 + lane / vpr + ps * rpp;
      d[P] = *reinterpret_cast<const u32x4_t*>(Ug + row * p.ldu + col0 + 64 * C + (lane % vpr) * 8);
    }
  };
  if (EK == kEpiDGelu) load_u(0, upre[0]);

  // This wave's LDS region is written and read only by this wave, and LDS
  // executes one wave's operations in order, so no barrier is needed between
  // the bands. The LDS accesses are inline assembly: the compiler would
  // otherwise guard them against the earlier copies into the same buffers with
  // a full vector-memory wait, which also waits for the stores of the previous
  // pass.
  // Column sums of the stored (bf16) outputs of the GeLU-derivative epilogue
  // when cs_part is set: each lane adds its 8 columns of each chunk over the
  // rows it stores, in band and pass order (a lane's columns are the same in
  // every band and pass); the block then adds the lanes' sums in a fixed order.
  constexpr bool CSUM = EK == kEpiDGelu;
  float colacc[NCH][8];
#pragma unroll
  for (int C = 0; C < NCH; ++C)
#pragma unroll
    for (int q = 0; q < 8; ++q) colacc[C][q] = 0.0f;
  const uint32_t ep_lds = lds_addr(reinterpret_cast<const uint8_t*>(ep));
  const uint32_t ep_w = ep_lds + (4 * (lane >> 5) * EP + (lane & 31)) * 4;
  Unroll<0, FM>::run([&](auto band) {
    constexpr int i = decltype(band)::value;
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t a = ep_w + (((r >> 2) * 8 + (r & 3)) * EP + j * 32) * 4;
        asm volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(acc[i][j][r]) : "memory");
      }
    if (EK == kEpiDGelu && i + 1 < FM) load_u(i + 1, upre[(i + 1) & 1]);
#pragma unroll
    for (int P = 0; P < NPB; ++P) {
      const int C = P >> 2, ps = P & 3;
      const int vpr = chunk_w(C) / 8, rpp = 64 / vpr;
      const int lr = lane / vpr + ps * rpp, ec = 64 * C + (lane % vpr) * 8;
      const uint32_t a = ep_lds + (lr * EP + ec) * 4;
      f32x4_t lo, hi;
      asm volatile("ds_read_b128 %0, %1" : "=v"(lo) : "v"(a) : "memory");
      asm volatile("ds_read_b128 %0, %1" : "=v"(hi) : "v"(a + 16) : "memory");
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(lo), "+v"(hi)::"memory");
      const int64_t row = rowt + i * 32 + lr;
      const int64_t col = col0 + ec;
      if constexpr (F32OUT) {
        float* d = cf + row * ldc + col;
        *reinterpret_cast<f32x4_t*>(d) = lo;
        *reinterpret_cast<f32x4_t*>(d + 4) = hi;
      } else {
        float v[8];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = lo[q];
          v[q + 4] = hi[q];
        }
        const int64_t o = row * p.ldc + col;
        if constexpr (EK == kEpiBiasGelu) {
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] += bias8[C][q];
          store8(p.c2, row * p.ldc2 + col, v, 1);
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            v[q] = gelu_tanh(v[q]);
            amax_run = fmaxf(amax_run, fabsf(v[q]));
          }
        } else if constexpr (EK == kEpiDGelu) {
          const u32x4_t w = upre[i & 1][P];
          float u[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            u[2 * q] = __uint_as_float(w[q] << 16);
            u[2 * q + 1] = __uint_as_float(w[q] & 0xffff0000u);
          }
          if (p.c2) {  // recompute of the activation from the saved U
            float y[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) y[q] = gelu_tanh(u[q]);
            store8(p.c2, row * p.ldc2 + col, y, 1);
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            v[q] *= gelu_tanh_grad(u[q]);
            amax_run = fmaxf(amax_run, fabsf(v[q]));
          }
          const u32x4_t wv{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
          *reinterpret_cast<u32x4_t*>(static_cast<uint16_t*>(p.c) + o) = wv;
          if (p.cs_part) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              colacc[C][2 * q] += __uint_as_float(wv[q] << 16);
              colacc[C][2 * q + 1] += __uint_as_float(wv[q] & 0xffff0000u);
            }
          }
        }
        if constexpr (EK != kEpiDGelu) store8(p.c, o, v, 1);
      }
    }
  });
  if constexpr (EK == kEpiBiasGelu || EK == kEpiDGelu) {
    if (p.amax) {
      // the wave's largest |value| as stored: rounding to bf16 is monotonic
      // and symmetric, so that is the bf16 rounding of the largest |v|
      float m = amax_run;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      if (lane == 0) {
        const int64_t tile = (m0 / BM) * (p.N / BN) + n0 / BN;
        p.amax[tile * NW + wave] = __uint_as_float((pack_bf16x2(m, 0.0f) & 0xffffu) << 16);
      }
    }
  }
  if constexpr (CSUM) {
    if (p.cs_part) {
      // row lanes of each wave row's sums in LDS: [WM][16][BN] floats
      constexpr int RL = 16;
      static_assert(WM * RL * BN * 4 <= SB, "LDS for the column sums");
      block_sync();  // every wave is done with its epilogue region
      float* cb = reinterpret_cast<float*>(stage_ptr<0, SB, POOL>());
#pragma unroll
      for (int C = 0; C < NCH; ++C) {
        const int vpr = chunk_w(C) / 8;
        const int cc = wn * WTN + 64 * C + (lane % vpr) * 8;
#pragma unroll
        for (int q = 0; q < 8; ++q) cb[(wm * RL + lane / vpr) * BN + cc + q] = colacc[C][q];
      }
      block_sync();
      for (int c = tid; c < BN; c += NW * 64) {
        const int rpp = 64 / (chunk_w((c % WTN) / 64) / 8);  // row lanes of c's chunk
        float v = 0.0f;
        for (int w = 0; w < WM; ++w)
          for (int r = 0; r < rpp; ++r) v += cb[(w * RL + r) * BN + c];
        p.cs_part[(m0 / BM) * p.N + n0 + c] = v;
      }
    }
  }
}

// One block of a product: output tile (or column-sum unit) number `block` of
// the product's 1-D grid.
template <int BM, int BN, int WM, int WN, int BK, int S, bool AK, bool BKC, int EK, int F8 = 0,
          int POOL = 0>
__device__ __forceinline__ void gemm_pipe_block(const GemmParams& p, const int block) {
  constexpr int NW = WM * WN;
  using OA = std::conditional_t<(F8 > 0), OperandF8<BM, NW>, Operand<AK, BM, BK, NW>>;
  using OB = std::conditional_t<(F8 > 0), OperandF8<BN, NW>, Operand<BKC, BN, BK, NW>>;
  constexpr int SB = OA::BYTES + OB::BYTES;
  // ---- output tile
  const int tiles_m = static_cast<int>(p.M / BM);
  const int tiles_n = static_cast<int>(p.N / BN);
  const int ntiles = tiles_m * tiles_n;
  // One block per (K slice z, tile) in a 1-D grid, slice-major; blocks past
  // the last slice's tiles run column-sum pass-1 units.
  const int z = block / ntiles;
  if constexpr (EK == kEpiF32) {
    if (z >= p.splitk) {
      const int e = block - p.splitk * ntiles, ncb = static_cast<int>((p.cs.N + 255) / 256);
      float(*part)[256] = reinterpret_cast<float(*)[256]>(stage_ptr<0, SB, POOL>());
      for (int u = e; u < p.cs_units; u += p.cs_blocks)
        colsum_vec_unit(p.cs, u % ncb, u / ncb, p.cs_nchunks, part);
      return;
    }
  }
  int64_t m0, n0;
  tile_origin<BM, BN>(p, block - z * ntiles, &m0, &n0);

  const int64_t kbeg = static_cast<int64_t>(z) * p.k_chunk;
  const int nk = static_cast<int>((min(p.K, kbeg + p.k_chunk) - kbeg) / BK);
  gemm_pipe_tile<BM, BN, WM, WN, BK, S, AK, BKC, EK, F8, POOL>(p, m0, n0, z, kbeg, nk);
}

}  // namespace
}  // namespace tpmlp
