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
// Per block: 128 queries of one (sequence, head), 4 waves of 32 queries (and
// up to two key groups). K and V tiles of 64 keys go HBM -> LDS with direct
// copies through 3 stages. The running maximum of a row moves only when the
// row's maximum grows by more than 2^8, so the outputs are rescaled rarely
// and the exponents stay <= 8 (exact in the final division by the sum).
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
// growth of a row's running maximum (log2 units) before the forward rescales
constexpr float kRegrow = 8.0f;

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));

// All stages in one LDS array, so a stage is a constant offset: fragment reads
// use the instruction's immediate offset and keep one address register each.
template <int BYTES = kStages * kStageBytes>
__device__ __forceinline__ uint8_t* attn_lds() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[BYTES];
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

// A block takes QW * 32 queries of one (sequence, head) in QW query groups of
// one wave each, and KG key groups: waves w and w + QW take the same 32
// queries and alternate key tiles (group g the tiles KG*i + g, through an
// NS-stage ring of its own), and merge their running statistics and outputs
// through LDS at the end. Key groups shorten the serial chain of a long causal
// row and put several waves on each SIMD when a shard has few queries, so one
// wave's softmax runs beside another's MFMAs.
template <int QW, int KG, int NS>
__global__ __launch_bounds__(64 * QW * KG) void attn_fwd_kernel(AttnParams p) {
  constexpr int QB = 32 * QW;  // queries per block
  constexpr int WPW = 16 / QW;  // 1 KiB copy windows per wave and stage
  static_assert(QW == 2 || QW == 4, "query groups");
  static_assert(NS >= 2 && NS <= 4, "stages");
  // one ring of (K, V) tile pairs per key group, so that every stage offset a
  // fragment read adds fits the instruction's 16-bit immediate
  constexpr int kRing = NS * kStageBytes;
  constexpr int kLds = KG * kRing;
  static_assert((KG - 1) * QW * 34 * 64 * 4 <= kLds, "LDS for the key-group merge");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qw = wave % QW, grp = wave / QW;  // query group, key group
  const int nqb = static_cast<int>((p.seq + QB - 1) / QB);
  // the longest causal rows first: query blocks in decreasing order
  const int qb = nqb - 1 - static_cast<int>(blockIdx.x % nqb);
  const int bh = static_cast<int>(blockIdx.x / nqb);
  const int h = bh % static_cast<int>(p.heads);
  const int64_t b = bh / p.heads;
  const int64_t seq = p.seq;
  const uint16_t* qkv = static_cast<const uint16_t*>(p.qkv);
  const int64_t row0 = b * seq;  // first token of the sequence
  const int64_t hd = p.group * kD;  // Q to K, K to V
  const int64_t qcol = (h / p.group) * 3 * hd + (h % p.group) * kD;  // this head's Q

  // ---- Q fragments (B operand of S^T = K Q^T), kept for the whole pass
  const int ql = lane & 31, half = lane >> 5;
  const int q = qb * QB + qw * 32 + ql;
  const int64_t qrow = row0 + (q < seq ? q : seq - 1);
  bf16x8_t qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8_t*>(qkv + qrow * p.ld_qkv + qcol + 16 * ks + 8 * half);
  // (issued before the first tile copies and so, loads returning in order,
  // landed whenever those copies have)

  // ---- tile copies: 16 windows of 1 KiB per (K, V) pair (8 of K, 8 of V),
  // KG pairs per stage, WPW windows per wave; window w goes to group w/16's
  // ring, tile (w/8)%2 (K or V), rows 8*(w%8) .. +7; lane L copies row
  // 8*(w%8) + L/8, physical chunk L%8.
  const uint16_t* src[WPW];
#pragma unroll
  for (int i = 0; i < WPW; ++i) {
    const int w = wave * WPW + i, t = (w / 8) % 2, r = 8 * (w % 8) + lane / 8, pc = lane % 8;
    const int c = pc ^ (t == 0 ? kswz(r) : vswz(r));
    src[i] = qkv + (row0 + r) * p.ld_qkv + qcol + (1 + t) * hd + c * 8;
  }
  // stage of key tiles KG*kp .. KG*kp + KG-1; a tile past the last one is
  // still copied (its rows clamp to the sequence's last) so that every wave
  // issues the same number of copies, and is never used
  auto issue = [&](auto stage_c, int kp) {
    uint8_t* st = attn_lds<kLds>() + decltype(stage_c)::value * kStageBytes;
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      const int w = wave * WPW + i, r = 8 * (w % 8) + lane / 8;
      const int64_t kb = static_cast<int64_t>(kp) * KG + w / 16;
      // keys past the sequence read its last row (they are masked)
      const int64_t over = kb * kKB + r - (seq - 1);
      const uint16_t* g = src[i] + kb * kKB * p.ld_qkv - (over > 0 ? over * p.ld_qkv : 0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)g,
          (__attribute__((address_space(3))) void*)(st + (w / 16) * kRing + (w % 16) * 1024), 16,
          0, 0);
    }
  };

  // key tiles this block needs: all tiles up to its last query's
  const int nkb_seq = static_cast<int>((seq + kKB - 1) / kKB);
  const int qlast = min(static_cast<int>(seq) - 1, qb * QB + QB - 1);
  const int nkb = p.causal ? min(nkb_seq, qlast / kKB + 1) : nkb_seq;
  const int wq_last = qb * QB + qw * 32 + 31;  // this wave's last query

  const float scale = p.scale_log2;  // log2(e) / sqrt(64)
  float m_run = -INFINITY, l_run = 0.0f;
  f32x16_t o[2] = {f32x16_t{}, f32x16_t{}};

  const int wq_first = qb * QB + qw * 32;     // this wave's first query

  // per-lane LDS byte addresses of the fragment reads within stage 0 (this
  // key group's tile pair)
  const uint32_t lds0 = attn_lds_addr(attn_lds<kLds>()) + grp * kRing;
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
    if (kb >= nkb || (p.causal && k0 > wq_last)) return;  // no visible key in the tile
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
    // mask (register r of half m: key k0 + 32m + 8*(r/4) + 4*half + r%4, seen
    // when 32m + 8*(r/4) + r%4 <= lim); tiles wholly below the diagonal and
    // inside the sequence need no mask. The maximum is taken on the raw scores
    // (the scale is positive).
    const bool interior = (!p.causal || k0 + kKB - 1 <= wq_first) && k0 + kKB <= seq;
    float mx = -INFINITY;
    if (interior) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[m][r], s[m][r + 1]));
    } else {
      const int lim = min(p.causal ? q : 0x7fffffff, static_cast<int>(seq) - 1) - k0 - 4 * half;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float v = 32 * m + 8 * (r / 4) + (r % 4) <= lim ? s[m][r] : -INFINITY;
          s[m][r] = v;
          mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32)) * scale;
    // Lazy rescaling: the running maximum moves only when a row's maximum
    // grows by more than kRegrow (log2 units), so exponents stay <= kRegrow
    // and most tiles skip rescaling the outputs. The lanes of a query (lane,
    // lane + 32) hold the same mx and m_run.
    const bool grow = mx > m_run + kRegrow;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float corr = grow ? __builtin_amdgcn_exp2f(m_run - mx) : 1.0f;  // 0 from -inf
      m_run = grow ? mx : m_run;
      l_run *= corr;
#pragma unroll
      for (int db = 0; db < 2; ++db) o[db] *= corr;
    }
    const float m_use = m_run == -INFINITY ? 0.0f : m_run;  // a row with no visible key yet
    float sum = 0.0f;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[m][r], scale, -m_use));
        s[m][r] = e;
        sum += e;
      }
    sum += __shfl_xor(sum, 32);
    l_run += sum;
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

  // ---- pass over the key tiles: NS stages of KG tiles, NS-1 in flight
  const int nkp = (nkb + KG - 1) / KG;
  Unroll<0, NS - 1>::run([&](auto jc) {
    if (decltype(jc)::value < nkp) issue(jc, decltype(jc)::value);
  });
  for (int kp0 = 0; kp0 < nkp; kp0 += NS) {
    Unroll<0, NS>::run([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      const int kp = kp0 + J;
      if (kp < nkp) {
        // the copies of the stages after kp (up to NS - 2 of them) may still fly
        const int later = min(NS - 2, nkp - 1 - kp);
        if (NS >= 4 && later >= 2) attn_wait_vmcnt<(NS >= 4 ? 2 : 0) * WPW>();
        else if (NS >= 3 && later >= 1) attn_wait_vmcnt<(NS >= 3 ? 1 : 0) * WPW>();
        else attn_wait_vmcnt<0>();
        attn_sync();  // stage kp landed for every wave; stage (kp+NS-1)%NS is free
        if (kp + NS - 1 < nkp) issue(std::integral_constant<int, (J + NS - 1) % NS>{}, kp + NS - 1);
        compute(jc, kp * KG + grp);
      }
    });
  }
  if constexpr (KG > 1) {
    // merge the key groups in group order: groups 1 .. KG-1 leave (m, l, O^T)
    // in LDS, group 0 folds them into its own; lane data of group g, query
    // group qw at float index (((g - 1) * QW + qw) * 34 + j) * 64 + lane
    attn_sync();  // every wave is done with the stages
    float* base = reinterpret_cast<float*>(attn_lds<kLds>()) + lane;
    if (grp > 0) {
      float* x = base + ((grp - 1) * QW + qw) * 34 * 64;
      x[0] = m_run;
      x[64] = l_run;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[(2 + 16 * db + r) * 64] = o[db][r];
    }
    attn_sync();
    if (grp > 0) return;
#pragma unroll
    for (int g = 1; g < KG; ++g) {
      const float* x = base + ((g - 1) * QW + qw) * 34 * 64;
      const float m1 = x[0], l1 = x[64];
      const float m_new = fmaxf(m_run, m1);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;
      const float c0 = __builtin_amdgcn_exp2f(m_run - m_use), c1 = __builtin_amdgcn_exp2f(m1 - m_use);
      l_run = l_run * c0 + l1 * c1;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * c0 + x[(2 + 16 * db + r) * 64] * c1;
    }
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

// ===========================================================================
// Backward. With P = softmax(S), S = Q K^T / 8 (masked), delta[q] =
// rowsum(dC * C)[q]:  dV = P^T dC,  dP = dC V^T,  dS = P (dP - delta),
// dQ = dS K / 8,  dK = dS^T Q / 8.  P is recomputed from the saved lse.
// Two kernels, each owning its outputs (no atomics, so the result does not
// depend on scheduling): one per 128-key block, walking the query tiles, for
// dK and dV; one per 128-query block, walking the key tiles, for dQ.
// ===========================================================================

// Chunk swizzle for a [64][64] bf16 tile read both along rows (16-byte reads
// of 32 consecutive rows) and across rows (transposed reads of rows k..k+3
// and k+8..k+11): an XOR of the row bits found by exhaustive search over such
// maps, conflict-free for both patterns.
__device__ __forceinline__ int dswz(int r) {
  return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 2);
}

constexpr int kBStages = 3;
// a stage: two [64][64] bf16 tiles, then (dK/dV kernel) the lse and delta of
// the tile's 64 queries, each twice so that every wave issues one copy
constexpr int kBStatBytes = 1024;
constexpr int kBStageBytes = 2 * kTileBytes + kBStatBytes;

template <int BYTES>
__device__ __forceinline__ uint8_t* attn_bwd_lds() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[BYTES];
  return buf;
}

// delta[b, h, q] = sum over d of dC[t, h*64 + d] * C[t, h*64 + d], t = b*seq + q
__global__ __launch_bounds__(256) void attn_delta_kernel(AttnBwdParams p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= p.batch * p.seq * p.heads) return;
  const int64_t t = i / p.heads;
  const int h = static_cast<int>(i % p.heads);
  const uint16_t* dc = static_cast<const uint16_t*>(p.dc) + t * p.ld_dc + h * kD;
  const uint16_t* c = static_cast<const uint16_t*>(p.c) + t * p.ld_c + h * kD;
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < kD; j += 8) {
    float a[8], v[8];
    load8_bf16(dc, j, a);
    load8_bf16(c, j, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(a[e], v[e], acc);
  }
  const int64_t b = t / p.seq, q = t % p.seq;
  p.delta[(b * p.heads + h) * p.seq + q] = acc;
}

// Copies of a [64][64] tile (rows = tokens row0 + r0 + 0..63, clamped to the
// sequence; 64 columns from col) into LDS at dst, swizzled with dswz: 8
// windows of 1 KiB, window w = 8 rows; this wave copies windows w0..w0+1.
struct TileCopy {
  const uint16_t* src[2];
  __device__ __forceinline__ void init(const uint16_t* base, int64_t ld, int64_t row0, int64_t col,
                                       int w0, int lane) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * (w0 + i) + lane / 8, c = (lane % 8) ^ dswz(r);
      src[i] = base + (row0 + r) * ld + col + c * 8;
    }
  }
  // rows r0 + r; rows past seq read row seq-1 (callers mask them)
  __device__ __forceinline__ void issue(uint8_t* dst, int64_t r0, int64_t seq, int64_t ld, int w0,
                                        int lane) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 8 * (w0 + i) + lane / 8;
      const int64_t over = r0 + r - (seq - 1);
      const uint16_t* g = src[i] + r0 * ld - (over > 0 ? over * ld : 0);
      __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                       (__attribute__((address_space(3))) void*)(dst + (w0 + i) * 1024),
                                       16, 0, 0);
    }
  }
};

// Per-lane LDS addresses of a tile's fragment reads, relative to the tile.
// Row reads: row 32m + (lane & 31), chunk 2ks + lane/32. Transposed reads
// (A operand with the permuted 16-token order of the forward): rows
// 16st + 4*(lane/32) + (lane%16)/4 and that + 8, columns 32db + 16*((lane/16)%2)
// + 4*(lane%4).
__device__ __forceinline__ uint32_t row_addr(int m, int ks, int lane) {
  const int r = 32 * m + (lane & 31), c = 2 * ks + (lane >> 5);
  return r * 128 + ((c ^ dswz(r)) << 4);
}
__device__ __forceinline__ uint32_t tr_addr(int st, int db, int second, int lane) {
  const int g = lane >> 4, sl = lane & 15;
  const int r = 16 * st + 4 * (g >> 1) + (sl >> 2) + 8 * second;
  const int d = 32 * db + 16 * (g & 1) + 4 * (sl & 3);
  return r * 128 + (((d >> 3) ^ dswz(r)) << 4) + (d & 7) * 2;
}

template <int N>
__device__ __forceinline__ void lds_tie(bf16x8_t (&f)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(f[i]));
}

// 32x32x16 operand from two transposed reads at LDS byte addresses a0 + OFF,
// a1 + OFF (OFF: a stage's constant offset, in the instruction's immediate).
template <int OFF>
__device__ __forceinline__ bf16x8_t tr_frag(uint32_t a0, uint32_t a1) {
  static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset");
  s16x4_t lo, hi;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(a0), "i"(OFF));
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(a1), "i"(OFF));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int OFF>
__device__ __forceinline__ bf16x8_t row_frag(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "16-bit LDS offset");
  bf16x8_t f;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f) : "v"(a), "i"(OFF));
  return f;
}

// Per-lane fragment addresses of one tile set (relative addresses + base):
// row reads ra[m][ks], transposed reads tr0 / tr1[st][db] (rows r and r + 8).
struct FragAddr {
  uint32_t ra[2][4], tr0[4][2], tr1[4][2];
  __device__ __forceinline__ void init(uint32_t base, int lane) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) ra[m][ks] = base + row_addr(m, ks, lane);
#pragma unroll
    for (int st = 0; st < 4; ++st)
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        tr0[st][db] = base + tr_addr(st, db, 0, lane);
        tr1[st][db] = base + tr_addr(st, db, 1, lane);
      }
  }
};

// bf16 operand from registers 8*hh .. 8*hh+7 of an accumulator
__device__ __forceinline__ bf16x8_t pack8(const f32x16_t& v, int hh) {
  f32x8_t t;
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = v[8 * hh + e];
  return __builtin_convertvector(t, bf16x8_t);
}

// ---- dK, dV: block = 128 keys of one (sequence, head), 4 waves of 32 keys
// per query group; with QG = 2 groups, waves w and w + 4 hold the same keys and
// alternate query tiles, and add their dK, dV through LDS at the end (in a
// fixed order). Per 64-query tile and 32-query half m: S = Q K^T and
// dP = dC V^T (lane = key, registers = queries), P, dS, then dV^T += dC^T P
// and dK^T += Q^T dS.
// dK and dV of key block `block` (blocks key-block-major within a (batch,
// head)); LDS: its own array, or a pool of POOL bytes shared with the dQ blocks
// of the same launch.
template <int QG, int POOL = 0>
__device__ __forceinline__ void attn_bwd_kv_block(const AttnBwdParams& p, const int block) {
  // one 3-stage ring of query tiles (Q, dC, stats) per group: every stage
  // offset fits the 16-bit immediate of the fragment reads
  constexpr int NS = kBStages;
  constexpr int kRing = NS * kBStageBytes;
  constexpr int kLds = QG * kRing;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = wave & 3, grp = wave >> 2;
  const int64_t seq = p.seq;
  const int nkb = static_cast<int>((seq + 127) / 128);
  const int kb = block % nkb;  // the keys most queries see first
  const int bh = block / nkb;
  const int h = bh % static_cast<int>(p.heads);
  const int64_t b = bh / p.heads;
  const int64_t row0 = b * seq, hd = p.group * kD;
  const int64_t qcol = (h / p.group) * 3 * hd + (h % p.group) * kD;
  const int64_t lbase = (b * p.heads + h) * seq;
  const uint16_t* qkv = static_cast<const uint16_t*>(p.qkv);
  const uint16_t* dcp = static_cast<const uint16_t*>(p.dc);
  const int kl = lane & 31, half = lane >> 5;
  const int key = kb * 128 + kw * 32 + kl;
  const int64_t krow = row0 + (key < seq ? key : seq - 1);

  // K and V fragments of this wave's 32 keys (B operands: column = key)
  bf16x8_t kf[4], vf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kf[ks] = *reinterpret_cast<const bf16x8_t*>(qkv + krow * p.ld_qkv + qcol + hd + 16 * ks + 8 * half);
    vf[ks] = *reinterpret_cast<const bf16x8_t*>(qkv + krow * p.ld_qkv + qcol + 2 * hd + 16 * ks + 8 * half);
  }
  attn_wait_vmcnt<0>();
  lds_tie(kf);
  lds_tie(vf);

  // query tiles: causal rows q >= the block's first key; group g takes tiles
  // qt0 + QG*i + g from slot g of stage i
  const int nqt = static_cast<int>((seq + 63) / 64);
  const int qt0 = p.causal ? kb * 2 : 0;
  const int nst = (nqt - qt0 + QG - 1) / QG;
  TileCopy cq, cd;
  cq.init(qkv, p.ld_qkv, row0, qcol, 2 * kw, lane);  // Q tile: windows 2kw, 2kw+1
  cd.init(dcp, p.ld_dc, row0, h * kD, 2 * kw, lane);   // dC tile
  static_assert(POOL == 0 || POOL >= kLds, "LDS pool");
  uint8_t* const lds = attn_bwd_lds<POOL ? POOL : kLds>();
  FragAddr fa;
  fa.init(attn_lds_addr(lds) + grp * kRing, lane);
  // stats copy: waves 0 and 2 of a group copy lse, 1 and 3 delta, of queries
  // qt*64 + lane (a tile past the last one is copied clamped and never used)
  const float* stat_src = (kw & 1 ? p.delta : p.lse) + lbase;
  auto issue = [&](auto stage_c, int si) {
    uint8_t* st = lds + grp * kRing + decltype(stage_c)::value * kBStageBytes;
    const int64_t q0 = static_cast<int64_t>(qt0 + si * QG + grp) * 64;
    cq.issue(st, q0, seq, p.ld_qkv, 2 * kw, lane);
    cd.issue(st + kTileBytes, q0, seq, p.ld_dc, 2 * kw, lane);
    const int64_t qq = q0 + lane;
    __builtin_amdgcn_global_load_lds(
        (const __attribute__((address_space(1))) void*)(stat_src + (qq < seq ? qq : seq - 1)),
        (__attribute__((address_space(3))) void*)(st + 2 * kTileBytes + kw * 256), 4, 0, 0);
  };

  f32x16_t dv[2] = {f32x16_t{}, f32x16_t{}}, dk[2] = {f32x16_t{}, f32x16_t{}};
  const float scale = p.scale_log2;
  const int wk_first = kb * 128 + kw * 32;  // this wave's first key

  auto compute = [&](auto stage_c, int qt) {
    constexpr int SO = decltype(stage_c)::value * kBStageBytes;
    const float* stats = reinterpret_cast<const float*>(lds + grp * kRing + SO + 2 * kTileBytes);
    const int q0 = qt * 64;
    if (qt >= nqt || (p.causal && q0 + 63 < wk_first)) return;  // no query sees these keys
    const bool interior = (!p.causal || q0 >= wk_first + 31) && q0 + 64 <= seq;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      // S and dP for queries q0 + 32m .. +31 (register r: query
      // q0 + 32m + 8*(r/4) + 4*half + r%4)
      bf16x8_t qa[4], da[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        qa[ks] = row_frag<SO>(fa.ra[m][ks]);
        da[ks] = row_frag<SO + kTileBytes>(fa.ra[m][ks]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_tie(qa);
      lds_tie(da);
      f32x16_t sv = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[ks], kf[ks], sv, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[ks], vf[ks], dp, 0, 0, 0);
      }
      // P and dS (masked entries 0): register r = 4j + e holds query
      // q0 + 4*half + off, off = 32m + 8j + e, seen when lo <= off <= hi. The
      // mask is taken on one wave-uniform branch, not per element.
      auto p_ds = [&](auto masked_c) {
        constexpr bool kMasked = decltype(masked_c)::value;
        const int base = q0 + 4 * half;
        const int lo = p.causal ? key - base : -0x7fffffff;
        const int hi = static_cast<int>(seq) - 1 - base;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int qi = 32 * m + 8 * j + 4 * half;
          const float4 l4 = *reinterpret_cast<const float4*>(stats + qi);
          const float4 d4 = *reinterpret_cast<const float4*>(stats + 64 + qi);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * j + e, off = 32 * m + 8 * j + e;
            float pr = __builtin_amdgcn_exp2f(sv[r] * scale - lv[e] * 1.4426950408889634f);
            if constexpr (kMasked) pr = (off >= lo && off <= hi) ? pr : 0.0f;
            sv[r] = pr;
            dp[r] = pr * (dp[r] - dl[e]);
          }
        }
      };
      if (interior) p_ds(std::false_type{});
      else p_ds(std::true_type{});
      // dV^T += dC^T P and dK^T += Q^T dS over the half's two 16-query steps
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int st = 2 * m + hh;
        const bf16x8_t pf = pack8(sv, hh), sf = pack8(dp, hh);
        bf16x8_t ta[2], tq[2];
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          ta[db] = tr_frag<SO + kTileBytes>(fa.tr0[st][db], fa.tr1[st][db]);
          tq[db] = tr_frag<SO>(fa.tr0[st][db], fa.tr1[st][db]);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_tie(ta);
        lds_tie(tq);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[db], pf, dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tq[db], sf, dk[db], 0, 0, 0);
        }
      }
    }
  };

  Unroll<0, NS - 1>::run([&](auto jc) {
    if (decltype(jc)::value < nst) issue(jc, decltype(jc)::value);
  });
  for (int i0 = 0; i0 < nst; i0 += NS) {
    Unroll<0, NS>::run([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      const int si = i0 + J;
      if (si < nst) {
        if constexpr (NS == 3) {
          if (si + 1 < nst) attn_wait_vmcnt<5>();  // stage si+1's five copies may still fly
          else attn_wait_vmcnt<0>();
        } else {
          attn_wait_vmcnt<0>();
        }
        attn_sync();
        if (si + NS - 1 < nst) issue(std::integral_constant<int, (J + NS - 1) % NS>{}, si + NS - 1);
        compute(jc, qt0 + si * QG + grp);
      }
    });
  }
  if constexpr (QG == 2) {
    // group 0 adds group 1's sums (64 floats per lane at (kw*64 + j)*64 + lane)
    attn_sync();
    float* x = reinterpret_cast<float*>(lds) + kw * 64 * 64 + lane;
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          x[(16 * db + r) * 64] = dv[db][r];
          x[(32 + 16 * db + r) * 64] = dk[db][r];
        }
    }
    attn_sync();
    if (grp == 1) return;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        dv[db][r] += x[(16 * db + r) * 64];
        dk[db][r] += x[(32 + 16 * db + r) * 64];
      }
  }

  // dK = dK^T^T / 8, dV = dV^T^T: lane holds key `key`, d = 32db + 8*(r/4) + 4*half + r%4
  if (key < seq) {
    uint16_t* out = static_cast<uint16_t*>(p.dqkv) + (row0 + key) * p.ld_dqkv + qcol;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * half;
        uint2 wk, wv;
        wk.x = pack_bf16x2(dk[db][4 * r4] * 0.125f, dk[db][4 * r4 + 1] * 0.125f);
        wk.y = pack_bf16x2(dk[db][4 * r4 + 2] * 0.125f, dk[db][4 * r4 + 3] * 0.125f);
        wv.x = pack_bf16x2(dv[db][4 * r4], dv[db][4 * r4 + 1]);
        wv.y = pack_bf16x2(dv[db][4 * r4 + 2], dv[db][4 * r4 + 3]);
        *reinterpret_cast<uint2*>(out + hd + d) = wk;
        *reinterpret_cast<uint2*>(out + 2 * hd + d) = wv;
      }
  }
}

// ---- dQ: block = 128 queries, 4 waves of 32 queries per key group; with
// KG = 2 groups, waves w and w + 4 hold the same queries, alternate key tiles
// and add their dQ through LDS at the end. Per 64-key tile and 32-key half m:
// S^T = K Q^T, dP^T = V dC^T (lane = query), P^T, dS^T, dQ^T += K^T dS^T.
// dQ of query block `block`; LDS as attn_bwd_kv_block. Blocks are taken
// longest causal row first within each (batch, head), or with BYLEN across all
// of them (every head's last query block first), which pairs the longest rows
// with the CUs that the dK/dV blocks of the same launch free first.
template <int KG, int POOL = 0, bool BYLEN = false>
__device__ __forceinline__ void attn_bwd_q_block(const AttnBwdParams& p, const int block) {
  constexpr int kPair = 2 * kTileBytes;  // one K and one V tile
  constexpr int NS = kBStages;            // a 3-stage ring of pairs per group
  constexpr int kRing = NS * kPair;
  constexpr int kLds = KG * kRing;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qw = wave & 3, grp = wave >> 2;
  const int64_t seq = p.seq;
  const int nqb = static_cast<int>((seq + kQB - 1) / kQB);
  const int nbh = static_cast<int>(p.batch * p.heads);
  const int qb = nqb - 1 - (BYLEN ? block / nbh : block % nqb);
  const int bh = BYLEN ? block % nbh : block / nqb;
  const int h = bh % static_cast<int>(p.heads);
  const int64_t b = bh / p.heads;
  const int64_t row0 = b * seq, hd = p.group * kD;
  const int64_t qcol = (h / p.group) * 3 * hd + (h % p.group) * kD;
  const int64_t lbase = (b * p.heads + h) * seq;
  const uint16_t* qkv = static_cast<const uint16_t*>(p.qkv);
  const uint16_t* dcp = static_cast<const uint16_t*>(p.dc);
  const int ql = lane & 31, half = lane >> 5;
  const int q = qb * kQB + qw * 32 + ql;
  const int64_t qrow = row0 + (q < seq ? q : seq - 1);
  bf16x8_t qf[4], df[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    qf[ks] = *reinterpret_cast<const bf16x8_t*>(qkv + qrow * p.ld_qkv + qcol + 16 * ks + 8 * half);
    df[ks] = *reinterpret_cast<const bf16x8_t*>(dcp + qrow * p.ld_dc + h * kD + 16 * ks + 8 * half);
  }
  const float lq = p.lse[lbase + (q < seq ? q : seq - 1)] * 1.4426950408889634f;
  const float dl = p.delta[lbase + (q < seq ? q : seq - 1)];
  attn_wait_vmcnt<0>();
  lds_tie(qf);
  lds_tie(df);

  const int nkt_seq = static_cast<int>((seq + 63) / 64);
  const int qlast = min(static_cast<int>(seq) - 1, qb * kQB + kQB - 1);
  const int nkt = p.causal ? min(nkt_seq, qlast / 64 + 1) : nkt_seq;
  const int nst = (nkt + KG - 1) / KG;
  const int wq_first = qb * kQB + qw * 32, wq_last = wq_first + 31;
  TileCopy ck, cv;
  ck.init(qkv, p.ld_qkv, row0, qcol + hd, 2 * qw, lane);
  cv.init(qkv, p.ld_qkv, row0, qcol + 2 * hd, 2 * qw, lane);
  static_assert(POOL == 0 || POOL >= kLds, "LDS pool");
  uint8_t* const lds = attn_bwd_lds<POOL ? POOL : kLds>();
  FragAddr fa;
  fa.init(attn_lds_addr(lds) + grp * kRing, lane);
  // stage si holds key tiles KG*si .. KG*si + KG-1 (one past the last is
  // copied clamped and never used)
  auto issue = [&](auto stage_c, int si) {
    uint8_t* st = lds + grp * kRing + decltype(stage_c)::value * kPair;
    const int64_t k0 = static_cast<int64_t>(si * KG + grp) * 64;
    ck.issue(st, k0, seq, p.ld_qkv, 2 * qw, lane);
    cv.issue(st + kTileBytes, k0, seq, p.ld_qkv, 2 * qw, lane);
  };
  f32x16_t dqa[2] = {f32x16_t{}, f32x16_t{}};
  const float scale = p.scale_log2;

  auto compute = [&](auto stage_c, int kt) {
    constexpr int SO = decltype(stage_c)::value * kPair;
    const int k0 = kt * 64;
    if (kt >= nkt || (p.causal && k0 > wq_last)) return;
    const bool interior = (!p.causal || k0 + 63 <= wq_first) && k0 + 64 <= seq;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x8_t ka[4], va[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        ka[ks] = row_frag<SO>(fa.ra[m][ks]);
        va[ks] = row_frag<SO + kTileBytes>(fa.ra[m][ks]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      lds_tie(ka);
      lds_tie(va);
      f32x16_t sv = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        sv = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], sv, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[ks], df[ks], dp, 0, 0, 0);
      }
      // dS (masked entries 0): register r holds key k0 + 4*half + off,
      // off = 32m + 8*(r/4) + r%4, seen when off <= lim; one wave-uniform
      // branch, not per element
      auto ds = [&](auto masked_c) {
        constexpr bool kMasked = decltype(masked_c)::value;
        const int lim =
            min(p.causal ? q : 0x7fffffff, static_cast<int>(seq) - 1) - k0 - 4 * half - 32 * m;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pr = __builtin_amdgcn_exp2f(sv[r] * scale - lq);
          if constexpr (kMasked) pr = 8 * (r / 4) + (r % 4) <= lim ? pr : 0.0f;
          dp[r] = pr * (dp[r] - dl);
        }
      };
      if (interior) ds(std::false_type{});
      else ds(std::true_type{});
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int st = 2 * m + hh;
        const bf16x8_t sf = pack8(dp, hh);
        bf16x8_t ta[2];
#pragma unroll
        for (int db = 0; db < 2; ++db) ta[db] = tr_frag<SO>(fa.tr0[st][db], fa.tr1[st][db]);
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        lds_tie(ta);
#pragma unroll
        for (int db = 0; db < 2; ++db)
          dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[db], sf, dqa[db], 0, 0, 0);
      }
    }
  };

  Unroll<0, NS - 1>::run([&](auto jc) {
    if (decltype(jc)::value < nst) issue(jc, decltype(jc)::value);
  });
  for (int i0 = 0; i0 < nst; i0 += NS) {
    Unroll<0, NS>::run([&](auto jc) {
      constexpr int J = decltype(jc)::value;
      const int si = i0 + J;
      if (si < nst) {
        if constexpr (NS == 3) {
          if (si + 1 < nst) attn_wait_vmcnt<4>();
          else attn_wait_vmcnt<0>();
        } else {
          attn_wait_vmcnt<0>();
        }
        attn_sync();
        if (si + NS - 1 < nst) issue(std::integral_constant<int, (J + NS - 1) % NS>{}, si + NS - 1);
        compute(jc, si * KG + grp);
      }
    });
  }
  if constexpr (KG == 2) {
    attn_sync();
    float* x = reinterpret_cast<float*>(lds) + qw * 32 * 64 + lane;
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[(16 * db + r) * 64] = dqa[db][r];
    }
    attn_sync();
    if (grp == 1) return;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dqa[db][r] += x[(16 * db + r) * 64];
  }

  if (q < seq) {
    uint16_t* out = static_cast<uint16_t*>(p.dqkv) + (row0 + q) * p.ld_dqkv + qcol;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        uint2 w;
        w.x = pack_bf16x2(dqa[db][4 * r4] * 0.125f, dqa[db][4 * r4 + 1] * 0.125f);
        w.y = pack_bf16x2(dqa[db][4 * r4 + 2] * 0.125f, dqa[db][4 * r4 + 3] * 0.125f);
        *reinterpret_cast<uint2*>(out + 32 * db + 8 * r4 + 4 * half) = w;
      }
  }
}

template <int QG>
__global__ __launch_bounds__(256 * QG) void attn_bwd_kv_kernel(AttnBwdParams p) {
  attn_bwd_kv_block<QG>(p, static_cast<int>(blockIdx.x));
}

template <int KG>
__global__ __launch_bounds__(256 * KG) void attn_bwd_q_kernel(AttnBwdParams p) {
  attn_bwd_q_block<KG>(p, static_cast<int>(blockIdx.x));
}

// Both passes in one launch (each reads only the inputs and delta): the dK/dV
// blocks first, then the dQ blocks, in one LDS pool sized for the larger.
template <int G>
__global__ __launch_bounds__(256 * G) void attn_bwd_kvq_kernel(AttnBwdParams p, int kv_blocks) {
  constexpr int kKv = G * kBStages * kBStageBytes, kQ = G * kBStages * 2 * kTileBytes;
  constexpr int kPool = kKv > kQ ? kKv : kQ;
  const int b = static_cast<int>(blockIdx.x);
  if (b < kv_blocks) attn_bwd_kv_block<G, kPool>(p, b);
  else attn_bwd_q_block<G, kPool, true>(p, b - kv_blocks);
}

}  // namespace

hipError_t launch_attention_bwd(const AttnBwdParams& p, hipStream_t s) {
  const int64_t bh = p.batch * p.heads;
  const int64_t rows = p.batch * p.seq * p.heads;
  hipLaunchKernelGGL(attn_delta_kernel, dim3(static_cast<unsigned>((rows + 255) / 256)), dim3(256),
                     0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // two query (key) groups per block below four blocks per CU: measured on the
  // ~350M layer's four shards in one launch (768 dK/dV blocks), two groups
  // took 117 us against 161 us with one; the attention-projection shards'
  // 512 took 59 against 70 us
  const int64_t kv_blocks = bh * ((p.seq + 127) / 128), q_blocks = bh * ((p.seq + kQB - 1) / kQB);
  const int64_t two_below = 4 * static_cast<int64_t>(device_shape().cus);
  const bool kv2 = kv_blocks < two_below, q2 = q_blocks < two_below;
  if (kv2 == q2 && kv_blocks + q_blocks <= 0x7fffffff) {  // one launch for both passes
    const unsigned grid = static_cast<unsigned>(kv_blocks + q_blocks);
    if (kv2)
      hipLaunchKernelGGL(attn_bwd_kvq_kernel<2>, dim3(grid), dim3(512), 0, s, p,
                         static_cast<int>(kv_blocks));
    else
      hipLaunchKernelGGL(attn_bwd_kvq_kernel<1>, dim3(grid), dim3(256), 0, s, p,
                         static_cast<int>(kv_blocks));
    return hipGetLastError();
  }
  if (kv2)
    hipLaunchKernelGGL(attn_bwd_kv_kernel<2>, dim3(static_cast<unsigned>(kv_blocks)), dim3(512), 0,
                       s, p);
  else
    hipLaunchKernelGGL(attn_bwd_kv_kernel<1>, dim3(static_cast<unsigned>(kv_blocks)), dim3(256), 0,
                       s, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (q2)
    hipLaunchKernelGGL(attn_bwd_q_kernel<2>, dim3(static_cast<unsigned>(q_blocks)), dim3(512), 0, s,
                       p);
  else
    hipLaunchKernelGGL(attn_bwd_q_kernel<1>, dim3(static_cast<unsigned>(q_blocks)), dim3(256), 0, s,
                       p);
  return hipGetLastError();
}

hipError_t launch_attention_fwd(const AttnParams& p, hipStream_t s) {
  const int64_t bh = p.batch * p.heads;
  const int64_t blocks128 = bh * ((p.seq + 127) / 128);
  if (blocks128 > 0x3fffffff) return hipErrorInvalidConfiguration;
  const int cus = device_shape().cus;
  if (blocks128 < 2 * cus)  // two key groups while the grid leaves SIMDs with one wave
    hipLaunchKernelGGL((attn_fwd_kernel<4, 2, 3>), dim3(static_cast<unsigned>(blocks128)),
                       dim3(512), 0, s, p);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<4, 1, 3>), dim3(static_cast<unsigned>(blocks128)),
                       dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace tpmlp
