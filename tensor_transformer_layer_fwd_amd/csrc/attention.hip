// Attention core of one shard, forward: for each sequence and each of the
// shard's heads, C = softmax(Q K^T / sqrt(64)) V under a causal mask, plus the
// per-query log-normaliser. Flash-style: one pass over the keys with a running
// maximum and sum, scores never leave registers.
//
// The scores are computed transposed, S^T = K Q^T, with 32x32x16 bf16 MFMAs:
// a lane then holds one query (lane & 31) and 16 keys per 32-key block, so the
// softmax statistics of a query live in one lane (plus its partner lane + 32).
// The output is accumulated transposed as well, O^T = V^T P^T: the probability
// registers of a 16-key step are directly the B operand once their keys are
// paired with the same keys in the A operand. That pairing is a permuted key
// order (lanes 0-31 carry keys 0-3 and 8-11 of the step, lanes 32-63 keys 4-7
// and 12-15), which two transposed LDS reads of the V tile produce at rows
// base + 4*(lane/32) and base + 8 + 4*(lane/32).
//
// Per block: 128 queries of one (sequence, head), 4 waves of 32 queries. K and
// V tiles of 64 keys go HBM -> LDS with direct copies through 3 stages.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace tpmlp {
namespace {

constexpr int kD = 64;        // head dimension
constexpr int kQB = 128;      // queries per block
constexpr int kKB = 64;       // keys per tile
constexpr int kStages = 3;
constexpr int kTileBytes = kKB * kD * 2;  // one K or V tile
constexpr int kStageBytes = 2 * kTileBytes;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));

// All stages in one LDS array, so a stage is a constant offset: fragment reads
// use the instruction's immediate offset and keep one address register each.
__device__ __forceinline__ uint8_t* attn_lds() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[kStages * kStageBytes];
  return buf;
}

__device__ __forceinline__ uint32_t attn_lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}

// 16-byte chunk swizzles of the 128-byte tile rows (key r): the K tile is read
// along rows (16-byte reads of 32 consecutive rows), the V tile across rows
// (transposed 8-byte reads of four consecutive rows).
__device__ __forceinline__ int kswz(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int vswz(int r) { return 4 * ((r >> 1) & 1); }

template <int N>
__device__ __forceinline__ void attn_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void attn_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nqb = static_cast<int>((p.seq + kQB - 1) / kQB);
  // the longest causal rows first: query blocks in decreasing order
  const int qb = nqb - 1 - static_cast<int>(blockIdx.x % nqb);
  const int bh = static_cast<int>(blockIdx.x / nqb);
  const int h = bh % static_cast<int>(p.heads);
  const int64_t b = bh / p.heads;
  const int64_t seq = p.seq;
  const uint16_t* qkv = static_cast<const uint16_t*>(p.qkv);
  const int64_t row0 = b * seq;  // first token of the sequence
  const int64_t hd = p.heads * kD;

  // ---- Q fragments (B operand of S^T = K Q^T), kept for the whole pass
  const int ql = lane & 31, half = lane >> 5;
  const int q = qb * kQB + wave * 32 + ql;
  const int64_t qrow = row0 + (q < seq ? q : seq - 1);
  bf16x8_t qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8_t*>(qkv + qrow * p.ld_qkv + h * kD + 16 * ks + 8 * half);
  // land them before any tile copy, so the copy waits below count copies only
  attn_wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(qf[ks]));

  // ---- tile copies: 16 windows of 1 KiB per stage (8 of K, 8 of V), four
  // per wave; window w covers rows 8*(w%8) .. +7 of its tile, lane L copies
  // row 8*(w%8) + L/8, physical chunk L%8.
  const uint16_t* src[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int w = wave * 4 + i, t = w / 8, r = 8 * (w % 8) + lane / 8, pc = lane % 8;
    const int c = pc ^ (t == 0 ? kswz(r) : vswz(r));
    src[i] = qkv + (row0 + r) * p.ld_qkv + (1 + t) * hd + h * kD + c * 8;
  }
  auto issue = [&](auto stage_c, int kb) {
    uint8_t* st = attn_lds() + decltype(stage_c)::value * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int w = wave * 4 + i, r = 8 * (w % 8) + lane / 8;
      // keys past the sequence read its last row (they are masked)
      const int64_t over = static_cast<int64_t>(kb) * kKB + r - (seq - 1);
      const uint16_t* g = src[i] + static_cast<int64_t>(kb) * kKB * p.ld_qkv -
                          (over > 0 ? over * p.ld_qkv : 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                       (__attribute__((address_space(3))) void*)(st + w * 1024),
                                       16, 0, 0);
    }
  };

  // key tiles this block needs: all tiles up to its last query's
  const int nkb_seq = static_cast<int>((seq + kKB - 1) / kKB);
  const int qlast = min(static_cast<int>(seq) - 1, qb * kQB + kQB - 1);
  const int nkb = p.causal ? min(nkb_seq, qlast / kKB + 1) : nkb_seq;
  const int wq_last = qb * kQB + wave * 32 + 31;  // this wave's last query

  const float scale = p.scale_log2;  // log2(e) / sqrt(64)
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16_t o[2] = {f32x16_t{}, f32x16_t{}};

  const int wq_first = qb * kQB + wave * 32;     // this wave's first query

  // per-lane LDS byte addresses of the fragment reads within stage 0
  const uint32_t lds0 = attn_lds_addr(attn_lds());
  uint32_t ka[2][4];  // K tile: key row 32m + ql, 16-byte chunk 2ks + half
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int r = 32 * m + ql, c = 2 * ks + half;
      ka[m][ks] = lds0 + r * 128 + ((c ^ kswz(r)) << 4);
    }
  uint32_t va[4][2];  // V tile, transposed reads: key rows kr and kr + 8, columns d .. d+3
  {
    const int g = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int kr = 16 * st + 4 * (g >> 1) + (sl >> 2);
        const int d = 32 * db + 16 * (g & 1) + 4 * (sl & 3);
        va[st][db] = lds0 + kTileBytes + kr * 128 + (((d >> 3) ^ vswz(kr)) << 4) + (d & 7) * 2;
      }
  }

  auto compute = [&](auto stage_c, int kb) {
    constexpr int SOFF = decltype(stage_c)::value * kStageBytes;
    const int k0 = kb * kKB;
    if (p.causal && k0 > wq_last) return;  // every key of the tile is masked for this wave
    // K fragments for S^T
    bf16x8_t kf[2][4];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(kf[m][ks]) : "v"(ka[m][ks]), "i"(SOFF));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) asm volatile("" : "+v"(kf[m][ks]));
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        s[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[m][ks], qf[ks], s[m], 0, 0, 0);
    // the transposed V fragments, read while the softmax arithmetic runs
    // (not before: the K and V fragments would then be live together)
    __builtin_amdgcn_sched_barrier(0);
    bf16x8_t vf[4][2];  // [16-key step][32-wide d block]
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        s16x4_t lo, hi;
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(va[st][db]), "i"(SOFF));
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                     : "=v"(hi) : "v"(va[st][db]), "i"(SOFF + 8 * 128));  // key row + 8
        vf[st][db] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    // scale and mask (register r of half m: key k0 + 32m + 8*(r/4) + 4*half + r%4);
    // tiles wholly below the diagonal and inside the sequence need no mask
    const bool interior = (!p.causal || k0 + kKB - 1 <= wq_first) && k0 + kKB <= seq;
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[m][r] * scale;
        if (!interior) {
          const int key = k0 + 32 * m + 8 * (r / 4) + 4 * half + (r % 4);
          if (key >= seq || (p.causal && key > q)) v = -INFINITY;
        }
        s[m][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;  // a row with no visible key yet
    const float corr = __builtin_amdgcn_exp2f(m_run - m_use);
    float sum = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(s[m][r] - m_use);  // argument <= 0
        s[m][r] = e;
        sum += e;
      }
    sum += __shfl_xor(sum, 32);
    l_run = l_run * corr + sum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < 2; ++db) o[db] *= corr;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int db = 0; db < 2; ++db) asm volatile("" : "+v"(vf[st][db]));
    // O^T += V^T P^T over four 16-key steps (step st: half m = st/2, registers 8*(st%2) ..)
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int m = st >> 1, hh = st & 1;
      f32x8_t pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = s[m][8 * hh + e];
      const bf16x8_t pf = __builtin_convertvector(pv, bf16x8_t);  // round to nearest even
#pragma unroll
      for (int db = 0; db < 2; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st][db], pf, o[db], 0, 0, 0);
    }
  };

  // ---- pass over the key tiles: 3 stages, two tiles in flight
  Unroll<0, 2>::run([&](auto jc) {
    if (decltype(jc)::value < nkb) issue(jc, decltype(jc)::value);
  });
  for (int kb0 = 0; kb0 < nkb; kb0 += kStages) {
    Unroll<0, kStages>::run([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      const int kb = kb0 + J;
      if (kb < nkb) {
        if (kb + 1 < nkb) attn_wait_vmcnt<4>();  // tile kb+1's copies may still fly
        else attn_wait_vmcnt<0>();
        attn_sync();  // tile kb landed for every wave; stage (kb+2)%3 is free
        if (kb + 2 < nkb) issue(std::integral_constant<int, (J + 2) % kStages>{}, kb + 2);
        compute(jc, kb);
      }
    });
  }

  // ---- output: lane holds query q and d = 32*db + 8*(r/4) + 4*half + r%4
  if (q < seq) {
    const float inv = 1.0f / l_run;
    uint16_t* crow = static_cast<uint16_t*>(p.c) + (row0 + q) * p.ld_c + h * kD;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint2 w;
        w.x = pack_bf16x2(o[db][4 * r4] * inv, o[db][4 * r4 + 1] * inv);
        w.y = pack_bf16x2(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
        *reinterpret_cast<uint2*>(crow + 32 * db + 8 * r4 + 4 * half) = w;
      }
    if (p.lse && half == 0)
      p.lse[(b * p.heads + h) * seq + q] = (m_run + __log2f(l_run)) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_attention_fwd(const AttnParams& p, hipStream_t s) {
  const int64_t blocks = p.batch * p.heads * ((p.seq + kQB - 1) / kQB);
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace tpmlp
