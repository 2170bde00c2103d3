// The C ABI: host-side validation, then dispatch to the kernels. Every check
// runs before the first HIP call, so a rejected call launches nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "tp_mlp.h"
#include "internal.h"

using namespace tpmlp;

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;

bool dim_ok(int64_t d) { return d >= 1 && d <= kMaxDim; }
bool dtype_ok(int dt) { return dt == TP_F32 || dt == TP_BF16; }
bool act_ok(int a) { return a == TP_ACT_NONE || a == TP_ACT_GELU_TANH; }

int hip_status(hipError_t e) {
  if (e == hipSuccess) return TP_OK;
  g_last_hip_error = static_cast<int>(e);
  return TP_ERR_HIP;
}

// Spare blocks of a weight-gradient GEMM that run column-sum pass-1 units.
constexpr int kColsumBlocks = 128;

// One bf16/fp32 GEMM (+ split-K fix-up). With cs (weight gradients with a
// bias gradient), the column sums ride along with the GEMM and fix-up launches
// when the pipelined kernel runs; otherwise they get launches of their own.
int run_gemm(GemmParams& p, int dt, bool allow_split, size_t ws_bytes, hipStream_t s,
             const ColsumParams* cs = nullptr) {
  if (dt == TP_F32) {
    p.splitk = 1;
    p.k_chunk = p.K;
    hipError_t e = launch_gemm_f32(p, s);
    if (e == hipSuccess && cs) e = launch_colsum(*cs, s);
    return hip_status(e);
  }
  const SplitPlan plan = plan_gemm_bf16(p.M, p.N, p.K, allow_split);
  p.splitk = plan.splitk;
  p.k_chunk = plan.k_chunk;
  if (plan.splitk > 1) {
    const size_t need = static_cast<size_t>(plan.splitk) * p.M * p.N * sizeof(float);
    if (!p.ws || ws_bytes < need) return TP_ERR_WORKSPACE;
  }
  const bool carry = cs && colsum_vec_ok(*cs) && gemm_pipe_epilogue(p, plan) == kEpiF32;
  if (carry) {
    const int64_t nchunks = colsum_chunks(*cs);
    const int64_t units = (cs->N + 255) / 256 * nchunks;
    p.cs = *cs;
    p.cs_nchunks = static_cast<int>(nchunks);
    p.cs_units = static_cast<int>(units);
    p.cs_blocks = static_cast<int>(units < kColsumBlocks ? units : kColsumBlocks);
  }
  hipError_t e = launch_gemm_bf16(p, plan, s);
  if (e == hipSuccess && plan.splitk > 1) e = launch_splitk_fixup(p, s);  // + pass 2
  if (e == hipSuccess && carry && plan.splitk == 1 && p.cs_nchunks > 1)
    e = launch_colsum_pass2(p.cs, p.cs_nchunks, s);
  if (e == hipSuccess && cs && !carry) e = launch_colsum(*cs, s);
  return hip_status(e);
}

// One FP8 GEMM (+ split-K fix-up, + carried column sums). Every check runs
// before the first launch: a shape the FP8 tiles do not cover, or an epilogue
// the FP8 kernel does not have, returns TP_ERR_SHAPE.
int run_gemm_fp8(GemmParams& p, bool allow_split, size_t ws_bytes, hipStream_t s,
                 const ColsumParams* cs = nullptr) {
  const SplitPlan plan = plan_gemm_fp8(p.M, p.N, p.K, allow_split);
  if (plan.tile == 0) return TP_ERR_SHAPE;
  p.splitk = plan.splitk;
  p.k_chunk = plan.k_chunk;
  if (plan.splitk > 1) {
    const size_t need = static_cast<size_t>(plan.splitk) * p.M * p.N * sizeof(float);
    if (!p.ws || ws_bytes < need) return TP_ERR_WORKSPACE;
  }
  if (fp8_pipe_epilogue(p) == kEpiNone) return TP_ERR_SHAPE;
  const bool carry = cs && colsum_vec_ok(*cs) && fp8_pipe_epilogue(p) == kEpiF32;
  if (carry) {
    const int64_t nchunks = colsum_chunks(*cs);
    const int64_t units = (cs->N + 255) / 256 * nchunks;
    p.cs = *cs;
    p.cs_nchunks = static_cast<int>(nchunks);
    p.cs_units = static_cast<int>(units);
    p.cs_blocks = static_cast<int>(units < kColsumBlocks ? units : kColsumBlocks);
  }
  hipError_t e = launch_gemm_fp8(p, plan, s);
  if (e == hipSuccess && plan.splitk > 1) e = launch_splitk_fixup(p, s);
  if (e == hipSuccess && carry && plan.splitk == 1 && p.cs_nchunks > 1)
    e = launch_colsum_pass2(p.cs, p.cs_nchunks, s);
  if (e == hipSuccess && cs && !carry) e = launch_colsum(*cs, s);
  return hip_status(e);
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; }
bool fmt_ok(int f) { return f == TP_FP8_E4M3 || f == TP_FP8_E5M2; }

// FP8 operand codes: 16-byte aligned rows of at least K codes, stride a
// multiple of 16 bytes.
bool fp8_operand_ok(const void* q, int64_t ld, int64_t K) {
  return aligned(q, 16) && ld % 16 == 0 && ld >= K;
}

size_t fp8_wgrad_split_bytes(int64_t T, int64_t k, int64_t n) {
  const SplitPlan plan = plan_gemm_fp8(k, n, T, true);
  if (plan.splitk <= 1) return 0;
  const size_t b = static_cast<size_t>(plan.splitk) * k * n * sizeof(float);
  return (b + 255) / 256 * 256;
}

size_t wgrad_split_bytes(int64_t T, int64_t k, int64_t n, int dt) {
  if (dt != TP_BF16) return 0;
  const SplitPlan plan = plan_gemm_bf16(k, n, T, true);
  if (plan.splitk <= 1) return 0;
  // keep the column-sum partials 256-byte aligned behind the split-K partials
  const size_t b = static_cast<size_t>(plan.splitk) * k * n * sizeof(float);
  return (b + 255) / 256 * 256;
}

// Data gradient dIn[T,k] = dOut[T,n] W[k,n]^T (x act'(U)) as a product.
GemmParams dgrad_params(const void* dOut, const void* W, const void* U, int act, void* dIn,
                        int64_t T, int64_t k, int64_t n, int64_t ld_dout, int64_t ld_w,
                        int64_t ld_u, int64_t ld_din, int out_dt) {
  GemmParams p{};
  p.a = dOut;
  p.b = W;
  p.c = dIn;
  p.u = U;
  p.M = T;
  p.N = k;
  p.K = n;
  p.lda = ld_dout;
  p.ldb = ld_w;
  p.ldc = ld_din;
  p.ldu = ld_u;
  p.epi = act != TP_ACT_NONE ? EPI_DACT : EPI_STORE;
  p.act = act == TP_ACT_GELU_TANH ? ACT_GELU : ACT_NONE;
  p.out_bf16 = out_dt == TP_BF16;
  p.a_kcontig = 1;  // dOut [T, n]
  p.b_kcontig = 1;  // W [k, n] read as W^T: K (= n) contiguous
  return p;
}

// Weight gradient dW[k,n] (+)= In[T,k]^T dOut[T,n] as a product, and the bias
// gradient's column sums of dOut with their partials at cs_ws.
GemmParams wgrad_params(const void* In, const void* dOut, float* dW, int64_t T, int64_t k,
                        int64_t n, int64_t ld_in, int64_t ld_dout, int64_t ld_dw, int accumulate,
                        void* ws) {
  GemmParams p{};
  p.a = In;
  p.b = dOut;
  p.c = dW;
  p.M = k;
  p.N = n;
  p.K = T;
  p.lda = ld_in;
  p.ldb = ld_dout;
  p.ldc = ld_dw;
  p.epi = EPI_STORE;
  p.out_bf16 = 0;
  p.accumulate = accumulate != 0;
  p.ws = static_cast<float*>(ws);
  p.a_kcontig = 0;  // In [T, k] read as In^T: M (= k) contiguous
  p.b_kcontig = 0;  // dOut [T, n]: N contiguous
  return p;
}

ColsumParams bias_grad_params(const void* dOut, float* dbias, int64_t T, int64_t n,
                              int64_t ld_dout, int dt, int accumulate, float* cs_ws) {
  ColsumParams c{};
  c.src = dOut;
  c.T = T;
  c.N = n;
  c.ld = ld_dout;
  c.src_bf16 = dt == TP_BF16;
  c.dbias = dbias;
  c.accumulate = accumulate != 0;
  c.ws = cs_ws;
  return c;
}

// Carried column sums of a weight gradient running on the pipelined kernel.
void carry_colsums(GemmParams* p, const ColsumParams& cs) {
  const int64_t nchunks = colsum_chunks(cs);
  const int64_t units = (cs.N + 255) / 256 * nchunks;
  p->cs = cs;
  p->cs_nchunks = static_cast<int>(nchunks);
  p->cs_units = static_cast<int>(units);
  p->cs_blocks = static_cast<int>(units < kColsumBlocks ? units : kColsumBlocks);
}

size_t two_wgrads_cs_offset(int64_t T, int64_t n0, bool bias0) {
  return bias0 ? (colsum_workspace_bytes(T, n0) + 255) / 256 * 256 : 0;
}

// K slices of the remaining tiles when 128 x 128 tiles leave a remainder over
// the CUs: as many as fit one slice per CU, at most 16, with K a multiple of
// 32 per slice; 0 when no remainder or fewer than 2 slices fit.
int two_wgrads_slices(int64_t tiles, int64_t T, int cus) {
  const int64_t rem = tiles % cus;
  if (rem == 0) return 0;
  for (int64_t sk = std::min<int64_t>(16, cus / rem); sk >= 2; --sk)
    if (T % (32 * sk) == 0) return static_cast<int>(sk);
  return 0;
}

// Whether the stacked launch of these shapes leaves a block slot free on
// every CU for most of its time: at most one whole tile per CU (the split
// tiles' K slices take the other slots only briefly). A row sum riding in
// the launch then runs beside the tiles; otherwise it would run after them.
bool two_wgrads_slot_free(int64_t k0, int64_t n0, int64_t k1, int64_t n1, int64_t T) {
  if (k0 % 128 || n0 % 128 || k1 % 128 || n1 % 128 || T % 32) return false;
  const int cus = device_shape().cus;
  const int64_t tiles = (k0 / 128) * (n0 / 128) + (k1 / 128) * (n1 / 128);
  const int64_t whole = two_wgrads_slices(tiles, T, cus) > 0 ? tiles - tiles % cus : tiles;
  return whole <= cus;
}

// Scratch of the stacked weight gradients: both products' column-sum
// partials, then the K-slice partials of the split tiles (at most one
// 128 x 128 fp32 tile per CU).
size_t two_wgrads_bytes(int64_t T, int64_t n0, int64_t n1) {
  const size_t cs = two_wgrads_cs_offset(T, n0, true) + colsum_workspace_bytes(T, n1);
  return (cs + 255) / 256 * 256 + static_cast<size_t>(device_shape().cus) * 128 * 128 * 4;
}

// Two weight gradients with their bias gradients, overwritten:
// dW0 = In0^T dOut0 (k0 x n0), db0 = column sums of dOut0, and the same for 1.
// Where both products tile by 128 x 128 with their column sums carried, one
// launch runs both products (the tiles past the last whole multiple of the CU
// count as K slices, when that fits) and one launch adds the slices and runs
// both column-sum second passes; otherwise they are two tp_linear_bwd_wgrad
// calls. ws holds both products' column-sum partials
// (two_wgrads_cs_offset, then product 1's), then the slices' partials
// (two_wgrads_bytes in all), or either call's workspace. With rs, the
// launch also runs that row sum (in blocks after its tiles), or the two calls
// are followed by the standalone sum.
int two_wgrads(const void* In0, const void* dOut0, float* dW0, float* db0, int64_t k0, int64_t n0,
               int64_t ld_in0, int64_t ld_dout0, int64_t ld_dw0, const void* In1,
               const void* dOut1, float* dW1, float* db1, int64_t k1, int64_t n1, int64_t ld_in1,
               int64_t ld_dout1, int64_t ld_dw1, int64_t T, int dt, void* ws, size_t ws_bytes,
               hipStream_t stream, const RowSumParams* rs = nullptr) {
  if (dt == TP_BF16) {
    // the stacked launch takes both products on 128 x 128 tiles whatever
    // each would plan alone: together they fill the CUs (the tiles past the
    // last whole multiple of the CU count as K slices)
    const SplitPlan pl0{kPipe128x128, 1, T}, pl1{kPipe128x128, 1, T};
    const size_t off1 = two_wgrads_cs_offset(T, n0, db0 != nullptr);
    const size_t need = off1 + (db1 ? colsum_workspace_bytes(T, n1) : 0);
    if (k0 % 128 == 0 && n0 % 128 == 0 && k1 % 128 == 0 && n1 % 128 == 0 && T % 32 == 0 &&
        (need == 0 || (ws && ws_bytes >= need))) {
      char* w = static_cast<char*>(ws);
      GemmParams p0 = wgrad_params(In0, dOut0, dW0, T, k0, n0, ld_in0, ld_dout0, ld_dw0, 0, ws);
      GemmParams p1 = wgrad_params(In1, dOut1, dW1, T, k1, n1, ld_in1, ld_dout1, ld_dw1, 0, ws);
      p0.splitk = p1.splitk = 1;
      p0.k_chunk = p1.k_chunk = T;
      const ColsumParams c0 = bias_grad_params(dOut0, db0, T, n0, ld_dout0, dt, 0,
                                               reinterpret_cast<float*>(w));
      const ColsumParams c1 = bias_grad_params(dOut1, db1, T, n1, ld_dout1, dt, 0,
                                               reinterpret_cast<float*>(w + off1));
      if (gemm_pipe_epilogue(p0, pl0) == kEpiF32 && gemm_pipe_epilogue(p1, pl1) == kEpiF32 &&
          (!db0 || colsum_vec_ok(c0)) && (!db1 || colsum_vec_ok(c1))) {
        if (db0) carry_colsums(&p0, c0);
        if (db1) carry_colsums(&p1, c1);
        const int64_t tiles = (k0 / 128) * (n0 / 128) + (k1 / 128) * (n1 / 128);
        WgradSplit sp{nullptr, static_cast<int>(tiles), 0};
        const int sk = two_wgrads_slices(tiles, T, device_shape().cus);
        const size_t off_part = (need + 255) / 256 * 256;
        const int64_t rest = sk > 0 ? tiles % device_shape().cus : 0;
        if (sk > 0 && ws && ws_bytes >= off_part + static_cast<size_t>(rest * sk) * 128 * 128 * 4) {
          sp.part = reinterpret_cast<float*>(w + off_part);
          sp.whole = static_cast<int>(tiles - rest);
          sp.sk = sk;
        }
        hipError_t e = launch_gemm_wgrad2(p0, p1, sp, rs, stream);
        if (e == hipSuccess)
          e = launch_wgrad2_finish(p0, p1, sp, db0 ? p0.cs_nchunks : 0, db1 ? p1.cs_nchunks : 0,
                                   stream);
        return hip_status(e);
      }
    }
  }
  int st = tp_linear_bwd_wgrad(In0, dOut0, dW0, db0, T, k0, n0, ld_in0, ld_dout0, ld_dw0, 0,
                               static_cast<tp_dtype>(dt), ws, ws_bytes, stream);
  if (st != TP_OK) return st;
  st = tp_linear_bwd_wgrad(In1, dOut1, dW1, db1, T, k1, n1, ld_in1, ld_dout1, ld_dw1, 0,
                           static_cast<tp_dtype>(dt), ws, ws_bytes, stream);
  if (st != TP_OK || !rs) return st;
  ReduceParams r{};
  for (int i = 0; i < rs->p; ++i) r.parts[i] = rs->parts + i * rs->rows * rs->N;
  r.p = rs->p;
  r.out = rs->out;
  r.T = rs->rows;
  r.N = rs->N;
  r.ldp = rs->N;
  r.ldo = rs->ld_out;
  r.out_bf16 = true;
  return hip_status(launch_reduce(r, stream));
}

// Pair kind and K slices of the paired backward launch of a bf16 linear layer
// (kPairNone: the layer's products cannot pair). Operand alignment is checked
// at the call.
SplitPlan pair_plan(int64_t T, int64_t k, int64_t n) { return plan_pair(T, k, n); }

// The weight gradient's own tile in a paired launch.
SplitPlan pair_wgrad_plan(const SplitPlan& pl) {
  return SplitPlan{pl.tile == kPairSame256x192 ? kPipe256x192 : kPipe128x128, pl.splitk,
                   pl.k_chunk};
}

size_t pair_split_bytes(int64_t T, int64_t k, int64_t n) {
  const SplitPlan pl = pair_plan(T, k, n);
  if (pl.tile == kPairNone || pl.splitk <= 1) return 0;
  const size_t b = static_cast<size_t>(pl.splitk) * k * n * sizeof(float);
  return (b + 255) / 256 * 256;
}

// Workspace bytes of one layer's paired launch: split partials, then the
// column-sum partials (256-byte multiples).
size_t pair_bytes(int64_t T, int64_t k, int64_t n, bool dbias) {
  const size_t cs = dbias ? (colsum_workspace_bytes(T, n) + 255) / 256 * 256 : 0;
  return pair_split_bytes(T, k, n) + cs;
}

// Every argument check of one layer's data and weight gradients.
int check_linear_bwd(const void* dOut, const void* W, const void* U, int act, const void* In,
                     const void* dIn, const float* dW, int64_t T, int64_t k, int64_t n,
                     int64_t ld_dout, int64_t ld_w, int64_t ld_u, int64_t ld_in, int64_t ld_din,
                     int64_t ld_dw, int dt, int out_dt) {
  if (!dOut || !W || !dIn || !In || !dW) return TP_ERR_NULL;
  if (!dtype_ok(dt) || !dtype_ok(out_dt)) return TP_ERR_DTYPE;
  if (dt == TP_F32 && out_dt != TP_F32) return TP_ERR_DTYPE;
  if (!act_ok(act)) return TP_ERR_ACT;
  if (act != TP_ACT_NONE && !U) return TP_ERR_NULL;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n)) return TP_ERR_SHAPE;
  if (ld_dout < n || ld_w < n || ld_din < k || ld_in < k || ld_dw < n) return TP_ERR_SHAPE;
  if (act != TP_ACT_NONE && ld_u < k) return TP_ERR_SHAPE;
  return TP_OK;
}

// One bf16 layer's two gradients set up for a paired launch, with the weight
// gradient's split partials at ws and its column-sum partials behind them.
// ok is false where they cannot pair (shapes, alignment, workspace).
struct PairSetup {
  GemmParams pd, pw;
  SplitPlan plan{0, 1, 0};
  int ekd = kEpiNone;
  bool ok = false, carry = false;
};

PairSetup setup_pair(const void* dOut, const void* W, const void* U, int act, const void* In,
                     void* dIn, float* dW, float* dbias, int64_t T, int64_t k, int64_t n,
                     int64_t ld_dout, int64_t ld_w, int64_t ld_u, int64_t ld_in, int64_t ld_din,
                     int64_t ld_dw, int accumulate, int out_dt, char* ws, size_t ws_bytes) {
  PairSetup q;
  q.plan = pair_plan(T, k, n);
  if (q.plan.tile == kPairNone) return q;
  const size_t split_bytes = pair_split_bytes(T, k, n);
  q.pd = dgrad_params(dOut, W, U, act, dIn, T, k, n, ld_dout, ld_w, ld_u, ld_din, out_dt);
  q.pw = wgrad_params(In, dOut, dW, T, k, n, ld_in, ld_dout, ld_dw, accumulate, ws);
  ColsumParams c = bias_grad_params(dOut, dbias, T, n, ld_dout, TP_BF16, accumulate,
                                    dbias ? reinterpret_cast<float*>(ws + split_bytes) : nullptr);
  q.pd.splitk = 1;
  q.pd.k_chunk = n;
  q.pw.splitk = q.plan.splitk;
  q.pw.k_chunk = q.plan.k_chunk;
  q.ekd = gemm_pipe_epilogue(q.pd, plan_gemm_bf16(T, k, n, false));
  const size_t need = pair_bytes(T, k, n, dbias != nullptr);
  q.ok = q.ekd != kEpiNone && gemm_pipe_epilogue(q.pw, pair_wgrad_plan(q.plan)) == kEpiF32 &&
         (!dbias || colsum_vec_ok(c)) && (need == 0 || (ws && ws_bytes >= need));
  if (q.ok && dbias) {
    const int64_t nchunks = colsum_chunks(c);
    const int64_t units = (n + 255) / 256 * nchunks;
    q.pw.cs = c;
    q.pw.cs_nchunks = static_cast<int>(nchunks);
    q.pw.cs_units = static_cast<int>(units);
    // on the CUs the tiles leave free in the first round, where there are at
    // least 16, so the column sums do not push tiles into a second round
    int64_t blocks = units < kColsumBlocks ? units : kColsumBlocks;
    const int free_cus = pair_free_cus(q.plan, T, k, n);
    if (free_cus >= 16 && free_cus < blocks) blocks = free_cus;
    q.pw.cs_blocks = static_cast<int>(blocks);
    q.carry = true;
  }
  return q;
}

// What a paired weight gradient still needs after its launch: the split-K
// fix-up, and pass 2 of its carried column sums.
// Checks and parameters of one tensor quantised into both layouts.
int fp8_both_params(const void* X, int64_t rows, int64_t cols, int64_t ld_x, int dt, int fmt,
                    void* Q, int64_t ld_q, void* Qt, int64_t ld_qt, float* scale_inv,
                    void* workspace, size_t workspace_bytes, Fp8QuantParams* out) {
  if (!X || !Q || !Qt || !scale_inv) return TP_ERR_NULL;
  if (!dtype_ok(dt) || !fmt_ok(fmt)) return TP_ERR_DTYPE;
  if (!dim_ok(rows) || !dim_ok(cols) || rows * cols > (int64_t(1) << 40)) return TP_ERR_SHAPE;
  if (ld_x < cols || ld_q < cols || ld_qt < rows) return TP_ERR_SHAPE;
  if (!aligned(scale_inv, 4) || !aligned(X, dt == TP_BF16 ? 2 : 4)) return TP_ERR_SHAPE;
  if (!workspace || workspace_bytes < kFp8AmaxBlocks * sizeof(float) || !aligned(workspace, 4))
    return TP_ERR_WORKSPACE;
  Fp8QuantParams q{};
  q.x = X;
  q.rows = rows;
  q.cols = cols;
  q.ld_x = ld_x;
  q.x_bf16 = dt == TP_BF16;
  q.fmt = fmt;
  q.transpose = 1;
  q.q = static_cast<uint8_t*>(Qt);
  q.ld_q = ld_qt;
  q.q_rows = static_cast<uint8_t*>(Q);
  q.ld_q_rows = ld_q;
  q.scale_inv = scale_inv;
  q.partial = static_cast<float*>(workspace);
  q.vec_in = aligned(X, 16) && ld_x % (dt == TP_BF16 ? 8 : 4) == 0;
  q.vec_out = aligned(Qt, 16) && ld_qt % 16 == 0;
  q.vec_rows = aligned(Q, 16) && ld_q % 16 == 0;
  *out = q;
  return TP_OK;
}

// Output tile and waves of an FP8 tile (as launched by the FP8 GEMM), or
// false for a tile it does not use.
bool fp8_tile_shape(int tile, int* bm, int* bn, int* waves) {
  switch (tile) {
    case kPipe128x256: *bm = 128, *bn = 256, *waves = 8; return true;
    case kPipe128x128: *bm = 128, *bn = 128, *waves = 4; return true;
    case kPipe256x192: *bm = 256, *bn = 192, *waves = 8; return true;
    case kPipe128x192: *bm = 128, *bn = 192, *waves = 4; return true;
    default: return false;
  }
}

// Amax slots the FP8 epilogue of an unsplit M x N x K product writes: one
// per wave of every output tile of the planned tile; 0 when no FP8 tile fits.
int64_t fp8_amax_slot_count(int64_t M, int64_t N, int64_t K) {
  const SplitPlan pl = plan_gemm_fp8(M, N, K, false);
  int bm = 0, bn = 0, w = 0;
  if (!fp8_tile_shape(pl.tile, &bm, &bn, &w) || M % bm || N % bn) return 0;
  return (M / bm) * (N / bn) * w;
}

bool pair_needs_finish(const PairSetup& q) {
  return q.plan.splitk > 1 || (q.carry && q.pw.cs_nchunks > 1);
}

hipError_t finish_pair(const PairSetup& q, hipStream_t s) {
  if (q.plan.splitk > 1) return launch_splitk_fixup(q.pw, s);  // + pass 2
  if (q.carry && q.pw.cs_nchunks > 1) return launch_colsum_pass2(q.pw.cs, q.pw.cs_nchunks, s);
  return hipSuccess;
}

// That work as spare blocks of the next paired launch (vector fix-up only).
bool rider_for(const PairSetup& q, PairRider* r) {
  if (!pair_needs_finish(q)) return true;
  if (q.plan.splitk > 1 && !splitk_fixup_vec_ok(q.pw)) return false;
  r->p = &q.pw;
  const int64_t fix_blocks = (q.pw.M * q.pw.N / 4 + 255) / 256;  // one float4 per thread
  r->nfix = q.plan.splitk > 1 ? static_cast<int>(fix_blocks < 256 ? fix_blocks : 256) : 0;
  r->ncs = (q.carry && q.pw.cs_nchunks > 1) ? static_cast<int>((q.pw.cs.N + 63) / 64) : 0;
  return true;
}

}  // namespace

// Scratch of tp_linear_bwd_wgrad_noalloc: one array per GPU, created with the
// code object. In host code `scratch` only names the symbol; kernels get the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[TP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 256;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array, looked up once per
// device (with that device current) and kept.
int current_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return hip_status(hipErrorInvalidDevice);
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_status(e);
      if (!ptr) return hip_status(hipErrorInvalidSymbol);
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return TP_OK;
}

}  // namespace

extern "C" {

int tp_column_linear_fwd(const void* X, const void* A_i, const void* bias_i, void* Y_i,
                         void* U_i, int64_t T, int64_t h, int64_t n, int64_t ld_x,
                         int64_t ld_a, int64_t ld_y, tp_dtype dt, tp_act act, hipStream_t stream) {
  if (!X || !A_i || !Y_i) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!act_ok(act)) return TP_ERR_ACT;
  if (act != TP_ACT_NONE && !U_i) return TP_ERR_NULL;
  if (!dim_ok(T) || !dim_ok(h) || !dim_ok(n)) return TP_ERR_SHAPE;
  if (ld_x < h || ld_a < n || ld_y < n) return TP_ERR_SHAPE;
  GemmParams p{};
  p.a = X;
  p.b = A_i;
  p.c = Y_i;
  p.c2 = U_i;
  p.bias = bias_i;
  p.M = T;
  p.N = n;
  p.K = h;
  p.lda = ld_x;
  p.ldb = ld_a;
  p.ldc = ld_y;
  p.ldc2 = ld_y;
  p.epi = EPI_BIAS_ACT;
  p.act = act == TP_ACT_GELU_TANH ? ACT_GELU : ACT_NONE;
  p.out_bf16 = dt == TP_BF16;
  p.a_kcontig = 1;  // X [T, h]
  p.b_kcontig = 0;  // A_i [h, n]
  return run_gemm(p, dt, false, 0, stream);
}

int tp_row_linear_fwd_partial(const void* Y_i, const void* B_i, float* Zp_i, int64_t T,
                              int64_t k, int64_t h, int64_t ld_y, int64_t ld_b,
                              int64_t ld_z, tp_dtype dt, hipStream_t stream) {
  if (!Y_i || !B_i || !Zp_i) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(h)) return TP_ERR_SHAPE;
  if (ld_y < k || ld_b < h || ld_z < h) return TP_ERR_SHAPE;
  GemmParams p{};
  p.a = Y_i;
  p.b = B_i;
  p.c = Zp_i;
  p.M = T;
  p.N = h;
  p.K = k;
  p.lda = ld_y;
  p.ldb = ld_b;
  p.ldc = ld_z;
  p.epi = EPI_STORE;
  p.out_bf16 = 0;
  p.a_kcontig = 1;  // Y_i [T, k]
  p.b_kcontig = 0;  // B_i [k, h]
  return run_gemm(p, dt, false, 0, stream);
}

int tp_linear_bwd_dgrad(const void* dOut, const void* W, const void* U, tp_act act, void* dIn,
                        int64_t T, int64_t k, int64_t n, int64_t ld_dout, int64_t ld_w,
                        int64_t ld_u, int64_t ld_din, tp_dtype dt, tp_dtype out_dt,
                        hipStream_t stream) {
  if (!dOut || !W || !dIn) return TP_ERR_NULL;
  if (!dtype_ok(dt) || !dtype_ok(out_dt)) return TP_ERR_DTYPE;
  if (dt == TP_F32 && out_dt != TP_F32) return TP_ERR_DTYPE;
  if (!act_ok(act)) return TP_ERR_ACT;
  if (act != TP_ACT_NONE && !U) return TP_ERR_NULL;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n)) return TP_ERR_SHAPE;
  if (ld_dout < n || ld_w < n || ld_din < k) return TP_ERR_SHAPE;
  if (act != TP_ACT_NONE && ld_u < k) return TP_ERR_SHAPE;
  GemmParams p = dgrad_params(dOut, W, U, act, dIn, T, k, n, ld_dout, ld_w, ld_u, ld_din, out_dt);
  return run_gemm(p, dt, false, 0, stream);
}

int tp_linear_bwd_dgrad_recompute(const void* dOut, const void* W, const void* U, tp_act act,
                                  void* dIn, void* Y, int64_t T, int64_t k, int64_t n,
                                  int64_t ld_dout, int64_t ld_w, int64_t ld_u, int64_t ld_din,
                                  int64_t ld_y, tp_dtype dt, hipStream_t stream) {
  if (!dOut || !W || !U || !dIn || !Y) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (act != TP_ACT_GELU_TANH) return TP_ERR_ACT;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n)) return TP_ERR_SHAPE;
  if (ld_dout < n || ld_w < n || ld_din < k || ld_u < k || ld_y < k) return TP_ERR_SHAPE;
  GemmParams p{};
  p.a = dOut;
  p.b = W;
  p.c = dIn;
  p.c2 = Y;
  p.u = U;
  p.M = T;
  p.N = k;
  p.K = n;
  p.lda = ld_dout;
  p.ldb = ld_w;
  p.ldc = ld_din;
  p.ldc2 = ld_y;
  p.ldu = ld_u;
  p.epi = EPI_DACT;
  p.act = ACT_GELU;
  p.out_bf16 = dt == TP_BF16;
  p.a_kcontig = 1;  // dOut [T, n]
  p.b_kcontig = 1;  // W [k, n] read as W^T: K (= n) contiguous
  return run_gemm(p, dt, false, 0, stream);
}

int tp_linear_bwd_wgrad_workspace_size(int64_t T, int64_t k, int64_t n, tp_dtype dt,
                                       size_t* bytes) {
  if (!bytes) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n)) return TP_ERR_SHAPE;
  *bytes = wgrad_split_bytes(T, k, n, dt) + colsum_workspace_bytes(T, n);
  return TP_OK;
}

int tp_linear_bwd_wgrad(const void* In, const void* dOut, float* dW, float* dbias, int64_t T,
                        int64_t k, int64_t n, int64_t ld_in, int64_t ld_dout, int64_t ld_dw,
                        int accumulate, tp_dtype dt, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  if (!In || !dOut || !dW) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n)) return TP_ERR_SHAPE;
  if (ld_in < k || ld_dout < n || ld_dw < n) return TP_ERR_SHAPE;
  const size_t split_bytes = wgrad_split_bytes(T, k, n, dt);
  const size_t cs_bytes = dbias ? colsum_workspace_bytes(T, n) : 0;
  if (split_bytes + cs_bytes > 0 && (!workspace || workspace_bytes < split_bytes + cs_bytes))
    return TP_ERR_WORKSPACE;
  GemmParams p = wgrad_params(In, dOut, dW, T, k, n, ld_in, ld_dout, ld_dw, accumulate, workspace);
  ColsumParams c = bias_grad_params(
      dOut, dbias, T, n, ld_dout, dt, accumulate,
      dbias ? reinterpret_cast<float*>(static_cast<char*>(workspace) + split_bytes) : nullptr);
  return run_gemm(p, dt, true, split_bytes, stream, dbias ? &c : nullptr);
}

int tp_linear_bwd_wgrad_noalloc(const void* In, const void* dOut, float* dW, float* dbias,
                                int64_t T, int64_t k, int64_t n, int64_t ld_in, int64_t ld_dout,
                                int64_t ld_dw, int accumulate, tp_dtype dt, hipStream_t stream) {
  if (!In || !dOut || !dW) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n)) return TP_ERR_SHAPE;
  if (ld_in < k || ld_dout < n || ld_dw < n) return TP_ERR_SHAPE;
  size_t need = 0;
  int st = tp_linear_bwd_wgrad_workspace_size(T, k, n, dt, &need);
  if (st != TP_OK) return st;
  if (need > TP_NOALLOC_SCRATCH_BYTES) return TP_ERR_SCRATCH;
  void* ws = nullptr;
  st = current_scratch(&ws);
  if (st != TP_OK) return st;
  return tp_linear_bwd_wgrad(In, dOut, dW, dbias, T, k, n, ld_in, ld_dout, ld_dw, accumulate, dt,
                             ws, TP_NOALLOC_SCRATCH_BYTES, stream);
}

int tp_linear_bwd_workspace_size(int64_t T, int64_t k, int64_t n, tp_dtype dt, size_t* bytes) {
  if (!bytes) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n)) return TP_ERR_SHAPE;
  const size_t alone = wgrad_split_bytes(T, k, n, dt) + colsum_workspace_bytes(T, n);
  const size_t pair = dt == TP_BF16 ? pair_bytes(T, k, n, true) : 0;
  *bytes = pair > alone ? pair : alone;
  return TP_OK;
}

int tp_linear_bwd_plan(int64_t T, int64_t k, int64_t n, int* pairing, int* splitk) {
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n)) return TP_ERR_SHAPE;
  const SplitPlan pl = pair_plan(T, k, n);
  if (pairing) *pairing = pl.tile;
  if (splitk) *splitk = pl.tile == kPairNone ? 1 : pl.splitk;
  return TP_OK;
}

int tp_mlp_bwd_workspace_size(int64_t T, int64_t h, int64_t F, tp_dtype dt, size_t* bytes) {
  if (!bytes) return TP_ERR_NULL;
  size_t b2 = 0, b1 = 0;
  int st = tp_linear_bwd_workspace_size(T, F, h, dt, &b2);
  if (st == TP_OK) st = tp_linear_bwd_workspace_size(T, h, F, dt, &b1);
  if (st != TP_OK) return st;
  const size_t alone = b2 > b1 ? b2 : b1;
  // fc2's pair, fc1's pair, then the column partials of dU_i (128-row tiles at most)
  const size_t both = dt == TP_BF16 ? pair_bytes(T, F, h, true) + pair_bytes(T, h, F, false) +
                                          static_cast<size_t>((T + 127) / 128) * F * sizeof(float)
                                    : 0;
  *bytes = both > alone ? both : alone;
  return TP_OK;
}

int tp_mlp_bwd(const void* dZ, const void* X, const void* A_i, const void* B_i, const void* U_i,
               const void* Y_i, void* dU_i, float* dB_i, float* db, float* dXp_i, float* dA_i,
               float* da_i, int64_t T, int64_t h, int64_t F, int64_t ld_dz, int64_t ld_x,
               int64_t ld_a, int64_t ld_b, int64_t ld_u, int64_t ld_y, int64_t ld_du,
               int64_t ld_dxp, int64_t ld_db, int64_t ld_da, int accumulate, tp_dtype dt,
               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  // fc2 (row-parallel, GeLU before it): dOut dZ [T,h], W = B_i [F,h], In = Y_i
  // fc1 (column-parallel): dOut dU_i [T,F], W = A_i [h,F], In = X, fp32 dX partial
  int st = check_linear_bwd(dZ, B_i, U_i, TP_ACT_GELU_TANH, Y_i, dU_i, dB_i, T, F, h, ld_dz,
                            ld_b, ld_u, ld_y, ld_du, ld_db, dt, dt);
  if (st == TP_OK)
    st = check_linear_bwd(dU_i, A_i, nullptr, TP_ACT_NONE, X, dXp_i, dA_i, T, h, F, ld_du, ld_a,
                          h, ld_x, ld_dxp, ld_da, dt, TP_F32);
  if (st != TP_OK) return st;
  const size_t alone2 = wgrad_split_bytes(T, F, h, dt) + (db ? colsum_workspace_bytes(T, h) : 0);
  const size_t alone1 = wgrad_split_bytes(T, h, F, dt) + (da_i ? colsum_workspace_bytes(T, F) : 0);
  const size_t alone = alone2 > alone1 ? alone2 : alone1;
  if (alone > 0 && (!workspace || workspace_bytes < alone)) return TP_ERR_WORKSPACE;

  if (dt == TP_BF16) {
    // fc2's pair first; its fix-up rides in fc1's pair, so the two layers'
    // partials sit one after the other in the workspace
    char* ws = static_cast<char*>(workspace);
    const size_t b2 = pair_bytes(T, F, h, db != nullptr);
    PairSetup q2 = setup_pair(dZ, B_i, U_i, TP_ACT_GELU_TANH, Y_i, dU_i, dB_i, db, T, F, h, ld_dz,
                              ld_b, ld_u, ld_y, ld_du, ld_db, accumulate, dt, ws, workspace_bytes);
    // fc1's bias gradient da_i = column sums of dU_i: fc2's data-gradient
    // epilogue adds each block tile's rows as it stores dU_i, and the partials
    // (behind both layers' own) are added in fc1's launch
    const size_t b1 = pair_bytes(T, h, F, false);
    const PairSetup q1 =
        setup_pair(dU_i, A_i, nullptr, TP_ACT_NONE, X, dXp_i, dA_i, nullptr, T, h, F, ld_du, ld_a,
                   h, ld_x, ld_dxp, ld_da, accumulate, TP_F32, ws ? ws + b2 : nullptr,
                   workspace_bytes > b2 ? workspace_bytes - b2 : 0);
    PairRider rider;
    bool part_ok = true;
    if (da_i && q2.ok) {
      const int64_t bm = q2.plan.tile == kPairSame256x192 ? 256 : 128;  // data-gradient tile rows
      const size_t part_bytes = static_cast<size_t>(T / bm) * F * sizeof(float);
      part_ok = q2.ekd == kEpiDGelu && T % bm == 0 && ws && workspace_bytes >= b2 + b1 + part_bytes;
      if (part_ok) {
        float* part = reinterpret_cast<float*>(ws + b2 + b1);
        q2.pd.cs_part = part;
        rider.cs2 = bias_grad_params(dU_i, da_i, T, F, ld_du, dt, accumulate, part);
        rider.cs2_nchunks = static_cast<int>(T / bm);
        rider.ncs2 = static_cast<int>((F + 63) / 64);
      }
    }
    if (q2.ok && q1.ok && part_ok && rider_for(q2, &rider)) {
      hipError_t e = launch_gemm_bwd_pair(q2.pw, q2.pd, q2.plan.tile, q2.ekd, PairRider{}, stream);
      if (e == hipSuccess)
        e = launch_gemm_bwd_pair(q1.pw, q1.pd, q1.plan.tile, q1.ekd, rider, stream);
      if (e == hipSuccess) e = finish_pair(q1, stream);
      return hip_status(e);
    }
  }
  // the two layers one after the other
  st = tp_linear_bwd(dZ, B_i, U_i, TP_ACT_GELU_TANH, Y_i, dU_i, dB_i, db, T, F, h, ld_dz, ld_b,
                     ld_u, ld_y, ld_du, ld_db, accumulate, dt, dt, workspace, workspace_bytes,
                     stream);
  if (st != TP_OK) return st;
  return tp_linear_bwd(dU_i, A_i, nullptr, TP_ACT_NONE, X, dXp_i, dA_i, da_i, T, h, F, ld_du, ld_a,
                       h, ld_x, ld_dxp, ld_da, accumulate, dt, TP_F32, workspace, workspace_bytes,
                       stream);
}

int tp_linear_bwd(const void* dOut, const void* W, const void* U, tp_act act, const void* In,
                  void* dIn, float* dW, float* dbias, int64_t T, int64_t k, int64_t n,
                  int64_t ld_dout, int64_t ld_w, int64_t ld_u, int64_t ld_in, int64_t ld_din,
                  int64_t ld_dw, int accumulate, tp_dtype dt, tp_dtype out_dt, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  // every check of both products first
  const int st = check_linear_bwd(dOut, W, U, act, In, dIn, dW, T, k, n, ld_dout, ld_w, ld_u,
                                  ld_in, ld_din, ld_dw, dt, out_dt);
  if (st != TP_OK) return st;
  const size_t need_split = wgrad_split_bytes(T, k, n, dt);
  const size_t cs_bytes = dbias ? colsum_workspace_bytes(T, n) : 0;
  if (need_split + cs_bytes > 0 && (!workspace || workspace_bytes < need_split + cs_bytes))
    return TP_ERR_WORKSPACE;

  if (dt == TP_BF16) {
    const PairSetup q = setup_pair(dOut, W, U, act, In, dIn, dW, dbias, T, k, n, ld_dout, ld_w,
                                   ld_u, ld_in, ld_din, ld_dw, accumulate, out_dt,
                                   static_cast<char*>(workspace), workspace_bytes);
    if (q.ok) {
      hipError_t e = launch_gemm_bwd_pair(q.pw, q.pd, q.plan.tile, q.ekd, PairRider{}, stream);
      if (e == hipSuccess) e = finish_pair(q, stream);
      return hip_status(e);
    }
  }
  // the two products one after the other
  const int r = tp_linear_bwd_dgrad(dOut, W, U, act, dIn, T, k, n, ld_dout, ld_w, ld_u, ld_din,
                                    dt, out_dt, stream);
  if (r != TP_OK) return r;
  return tp_linear_bwd_wgrad(In, dOut, dW, dbias, T, k, n, ld_in, ld_dout, ld_dw, accumulate, dt,
                             workspace, workspace_bytes, stream);
}

int tp_mlp_step_workspace_size(int64_t T, int64_t h, int64_t F, int p, tp_dtype dt,
                               size_t* bytes) {
  if (!bytes) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(h) || !dim_ok(F) || p < 1 || p > kMaxPartials) return TP_ERR_SHAPE;
  const int64_t pF = static_cast<int64_t>(p) * F;
  if (!dim_ok(pF)) return TP_ERR_SHAPE;
  size_t fb = 0, w2 = 0, w1 = 0;
  int st = tp_mlp_bwd_workspace_size(T, h, F, dt, &fb);
  if (st == TP_OK) st = tp_linear_bwd_wgrad_workspace_size(T, pF, h, dt, &w2);
  if (st == TP_OK) st = tp_linear_bwd_wgrad_workspace_size(T, h, pF, dt, &w1);
  if (st != TP_OK) return st;
  // the row launch's counters, then the stacked weight gradients' scratch;
  // the per-product path uses the workspace from its start
  const size_t rows = dt == TP_BF16 ? mlp_step_workspace_bytes(T, h, F, p) : 0;
  // either weight gradient's own call, or the stacked products' scratch
  const size_t both = two_wgrads_bytes(T, h, pF);
  size_t wg = w1 > w2 ? w1 : w2;
  wg = wg > both ? wg : both;
  // (the per-product path's scratch also starts past the row counters, so
  // that calls of either path can share one workspace)
  const size_t each = fb > wg ? fb : wg;
  *bytes = rows + each;
  return TP_OK;
}

int tp_mlp_step_plan(int64_t T, int64_t h, int64_t F, int p, tp_dtype dt, int* fused) {
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(h) || !dim_ok(F) || p < 1 || p > kMaxPartials) return TP_ERR_SHAPE;
  if (fused) *fused = dt == TP_BF16 && mlp_step_supported(T, h, F, p);
  return TP_OK;
}

int tp_set_wait_limit(int64_t polls) {
  set_step_wait_limit(polls);
  return TP_OK;
}

// Phases of mlp_step_impl: the forward and the Z sum, the data gradients and
// the dX sum, the weight and bias gradients.
constexpr int kPhFwd = 1, kPhWgrad = 2, kPhBwd = 4;

static int mlp_step_impl(const void* X, const void* A, const void* a, const void* B, const void* b,
                const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                float* db, float* dA, float* da, float* dXp, void* dX, int64_t T, int64_t h,
                int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b, int64_t ld_dz,
                int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db, int64_t ld_da,
                tp_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream,
                int phases, int recompute) {
  if (!X || !A || !B || !dZ || !U || !Y || !Zp || !Z || !dU || !dB || !dA || !dXp || !dX)
    return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(h) || !dim_ok(F) || p < 1 || p > kMaxPartials) return TP_ERR_SHAPE;
  const int64_t pF = static_cast<int64_t>(p) * F;
  if (!dim_ok(pF) || T * h > kMaxDim * 4 || ld_x < h || ld_a < pF || ld_b < h || ld_dz < h ||
      ld_u < pF || ld_z < h || ld_dx < h || ld_db < h || ld_da < pF)
    return TP_ERR_SHAPE;
  size_t need = 0;
  int st = tp_mlp_step_workspace_size(T, h, F, p, dt, &need);
  if (st != TP_OK) return st;
  if (need > 0 && (!workspace || workspace_bytes < need)) return TP_ERR_WORKSPACE;
  const size_t es = dt == TP_BF16 ? 2 : 4;
  auto row_ok = [](const void* q, int64_t ld, size_t e) {
    return aligned(q, 16) && (ld * static_cast<int64_t>(e)) % 16 == 0;
  };
  const bool fused = dt == TP_BF16 && mlp_step_supported(T, h, F, p) &&
                     row_ok(X, ld_x, es) && row_ok(A, ld_a, es) && row_ok(B, ld_b, es) &&
                     row_ok(dZ, ld_dz, es) && row_ok(U, ld_u, es) && row_ok(Y, ld_u, es) &&
                     row_ok(dU, ld_u, es) && row_ok(Z, ld_z, es) && row_ok(dX, ld_dx, es) &&
                     row_ok(Zp, h, 4) && row_ok(dXp, h, 4) && row_ok(dB, ld_db, 4) &&
                     row_ok(dA, ld_da, 4) && (!a || aligned(a, 16)) && (!b || aligned(b, 16)) &&
                     aligned(workspace, 256);
  const int64_t ld_y = ld_u;
  // Weight and bias gradients of every shard as two products over the stacked
  // shards: dB = Y^T dZ ([p*F, h]) with db = column sums of dZ, and
  // dA = X^T dU ([h, p*F]) with da = column sums of dU.
  // With the row launch's data gradients in the same call, the stacked launch
  // also sums the dX partials (the row launch leaves that sum out) where it
  // leaves block slots free beside its tiles.
  const bool dx_in_wgrads = fused && (phases & kPhBwd) && (phases & kPhWgrad) &&
                            two_wgrads_slot_free(pF, h, h, pF, T);
  const RowSumParams dxsum{dXp, p, dX, T, h, ld_dx};
  auto wgrads = [&](void* ws, size_t ws_bytes) {
    return two_wgrads(Y, dZ, dB, db, pF, h, ld_y, ld_dz, ld_db, X, dU, dA, da, h, pF, ld_x, ld_u,
                      ld_da, T, dt, ws, ws_bytes, stream, dx_in_wgrads ? &dxsum : nullptr);
  };
  if (fused) {
    if (phases & (kPhFwd | kPhBwd)) {
      StepParams s{};
      s.x = X;
      s.a = A;
      s.bias_a = a;
      s.b = B;
      s.bias_b = b;
      s.dz = dZ;
      s.u = U;
      s.y = Y;
      s.du = dU;
      s.zp = Zp;
      s.dxp = dXp;
      s.z = Z;
      s.dx = dX;
      s.T = T;
      s.h = h;
      s.F = F;
      s.p = p;
      s.ld_x = ld_x;
      s.ld_a = ld_a;
      s.ld_b = ld_b;
      s.ld_dz = ld_dz;
      s.ld_u = ld_u;
      s.ld_z = ld_z;
      s.ld_dx = ld_dx;
      s.phases = ((phases & kPhFwd) ? 1 : 0) | ((phases & kPhBwd) ? 2 : 0);
      s.recompute = recompute != 0;
      s.no_dx_sum = dx_in_wgrads;
      st = hip_status(launch_mlp_rows(s, workspace, stream));
      if (st != TP_OK) return st;
    }
    if (phases & kPhWgrad) {
      const size_t rows = mlp_step_workspace_bytes(T, h, F, p);
      return wgrads(static_cast<char*>(workspace) + rows, workspace_bytes - rows);
    }
    return TP_OK;
  }
  // the per-product path's scratch: past the row counters (where the shapes
  // have them), which must stay zero for the fused calls
  const size_t rows_off = dt == TP_BF16 ? mlp_step_workspace_bytes(T, h, F, p) : 0;
  void* scratch = static_cast<char*>(workspace) + rows_off;
  const size_t scratch_bytes = workspace_bytes - rows_off;
  // the same step as one call per product. The whole step: every shard's
  // forward, the sum, every shard's backward (tp_mlp_bwd, both layers' two
  // gradients), the sum of the dX partials. Otherwise the forward and the sum;
  // the data gradients (with Y_i rebuilt from U_i when recomputing) and their
  // sum; the weight and bias gradients: whichever phases are asked for.
  const float* zparts[kMaxPartials];
  const float* dparts[kMaxPartials];
  auto Ai = [&](int i) { return static_cast<const char*>(A) + i * F * es; };
  auto Bi = [&](int i) { return static_cast<const char*>(B) + i * F * ld_b * es; };
  auto Ui = [&](int i) { return static_cast<char*>(U) + i * F * es; };
  auto Yi = [&](int i) { return static_cast<char*>(Y) + i * F * es; };
  auto dUi = [&](int i) { return static_cast<char*>(dU) + i * F * es; };
  for (int i = 0; i < p; ++i) {
    zparts[i] = Zp + i * T * h;
    dparts[i] = dXp + i * T * h;
  }
  if (phases & kPhFwd) {
    for (int i = 0; i < p; ++i) {
      const void* ai = a ? static_cast<const char*>(a) + i * F * es : nullptr;
      st = tp_column_linear_fwd(X, Ai(i), ai, Yi(i), Ui(i), T, h, F, ld_x, ld_a, ld_u, dt,
                                TP_ACT_GELU_TANH, stream);
      if (st != TP_OK) return st;
      st = tp_row_linear_fwd_partial(Yi(i), Bi(i), Zp + i * T * h, T, F, h, ld_u, ld_b, h, dt,
                                     stream);
      if (st != TP_OK) return st;
    }
    st = tp_reduce_partials(zparts, p, b, Z, T, h, h, ld_z, dt, stream);
    if (st != TP_OK) return st;
  }
  if ((phases & (kPhBwd | kPhWgrad)) == (kPhBwd | kPhWgrad) && !recompute) {
    for (int i = 0; i < p; ++i) {
      st = tp_mlp_bwd(dZ, X, Ai(i), Bi(i), Ui(i), Yi(i), dUi(i), dB + i * F * ld_db,
                      i == 0 ? db : nullptr, dXp + i * T * h, dA + i * F, da ? da + i * F : nullptr,
                      T, h, F, ld_dz, ld_x, ld_a, ld_b, ld_u, ld_u, ld_u, h, ld_db, ld_da, 0, dt,
                      scratch, scratch_bytes, stream);
      if (st != TP_OK) return st;
    }
    return tp_reduce_partials(dparts, p, nullptr, dX, T, h, h, ld_dx, dt, stream);
  }
  if (phases & kPhBwd) {
    for (int i = 0; i < p; ++i) {
      st = recompute ? tp_linear_bwd_dgrad_recompute(dZ, Bi(i), Ui(i), TP_ACT_GELU_TANH, dUi(i),
                                                     Yi(i), T, F, h, ld_dz, ld_b, ld_u, ld_u,
                                                     ld_u, dt, stream)
                     : tp_linear_bwd_dgrad(dZ, Bi(i), Ui(i), TP_ACT_GELU_TANH, dUi(i), T, F, h,
                                           ld_dz, ld_b, ld_u, ld_u, dt, dt, stream);
      if (st != TP_OK) return st;
      st = tp_linear_bwd_dgrad(dUi(i), Ai(i), nullptr, TP_ACT_NONE, dXp + i * T * h, T, h, F,
                               ld_u, ld_a, h, h, dt, TP_F32, stream);
      if (st != TP_OK) return st;
    }
    st = tp_reduce_partials(dparts, p, nullptr, dX, T, h, h, ld_dx, dt, stream);
    if (st != TP_OK) return st;
  }
  if (phases & kPhWgrad) return wgrads(scratch, scratch_bytes);
  return TP_OK;
}

int tp_mlp_step(const void* X, const void* A, const void* a, const void* B, const void* b,
                const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                float* db, float* dA, float* da, float* dXp, void* dX, int64_t T, int64_t h,
                int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b, int64_t ld_dz,
                int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db, int64_t ld_da,
                tp_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mlp_step_impl(X, A, a, B, b, dZ, U, Y, Zp, Z, dU, dB, db, dA, da, dXp, dX, T, h, F, p, ld_x, ld_a, ld_b, ld_dz, ld_u, ld_z, ld_dx, ld_db, ld_da, dt, workspace, workspace_bytes, stream, kPhFwd | kPhBwd | kPhWgrad, 0);
}

int tp_mlp_step_rows(const void* X, const void* A, const void* a, const void* B, const void* b,
                const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                float* db, float* dA, float* da, float* dXp, void* dX, int64_t T, int64_t h,
                int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b, int64_t ld_dz,
                int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db, int64_t ld_da,
                tp_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mlp_step_impl(X, A, a, B, b, dZ, U, Y, Zp, Z, dU, dB, db, dA, da, dXp, dX, T, h, F, p, ld_x, ld_a, ld_b, ld_dz, ld_u, ld_z, ld_dx, ld_db, ld_da, dt, workspace, workspace_bytes, stream, kPhFwd | kPhBwd, 0);
}

int tp_mlp_step_wgrad(const void* X, const void* A, const void* a, const void* B, const void* b,
                const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                float* db, float* dA, float* da, float* dXp, void* dX, int64_t T, int64_t h,
                int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b, int64_t ld_dz,
                int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db, int64_t ld_da,
                tp_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mlp_step_impl(X, A, a, B, b, dZ, U, Y, Zp, Z, dU, dB, db, dA, da, dXp, dX, T, h, F, p, ld_x, ld_a, ld_b, ld_dz, ld_u, ld_z, ld_dx, ld_db, ld_da, dt, workspace, workspace_bytes, stream, kPhWgrad, 0);
}

int tp_mlp_step_fwd(const void* X, const void* A, const void* a, const void* B, const void* b,
                    const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                    float* db, float* dA, float* da, float* dXp, void* dX, int64_t T, int64_t h,
                    int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b, int64_t ld_dz,
                    int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db, int64_t ld_da,
                    tp_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return mlp_step_impl(X, A, a, B, b, dZ, U, Y, Zp, Z, dU, dB, db, dA, da, dXp, dX, T, h, F, p,
                       ld_x, ld_a, ld_b, ld_dz, ld_u, ld_z, ld_dx, ld_db, ld_da, dt, workspace,
                       workspace_bytes, stream, kPhFwd, 0);
}

int tp_mlp_step_bwd(const void* X, const void* A, const void* a, const void* B, const void* b,
                    const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                    float* db, float* dA, float* da, float* dXp, void* dX, int64_t T, int64_t h,
                    int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b, int64_t ld_dz,
                    int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db, int64_t ld_da,
                    int recompute, tp_dtype dt, void* workspace, size_t workspace_bytes,
                    hipStream_t stream) {
  return mlp_step_impl(X, A, a, B, b, dZ, U, Y, Zp, Z, dU, dB, db, dA, da, dXp, dX, T, h, F, p,
                       ld_x, ld_a, ld_b, ld_dz, ld_u, ld_z, ld_dx, ld_db, ld_da, dt, workspace,
                       workspace_bytes, stream, kPhBwd | kPhWgrad, recompute != 0);
}

// ---------------------------------------------------------------------------
// The attention projections of all shards (tp_attn_proj_step)
// ---------------------------------------------------------------------------
int tp_attn_proj_step_workspace_size(int64_t T, int64_t h, int64_t Q, int64_t O, int p,
                                     tp_dtype dt, size_t* bytes) {
  if (!bytes) return TP_ERR_NULL;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(h) || !dim_ok(Q) || !dim_ok(O) || p < 1 || p > kMaxPartials)
    return TP_ERR_SHAPE;
  const int64_t pQ = static_cast<int64_t>(p) * Q, pO = static_cast<int64_t>(p) * O;
  if (!dim_ok(pQ) || !dim_ok(pO)) return TP_ERR_SHAPE;
  size_t w1 = 0, w2 = 0;
  int st = tp_linear_bwd_wgrad_workspace_size(T, pO, h, dt, &w1);
  if (st == TP_OK) st = tp_linear_bwd_wgrad_workspace_size(T, h, pQ, dt, &w2);
  if (st != TP_OK) return st;
  // the row launch's counters, then the stacked weight gradients' scratch
  const size_t rows = dt == TP_BF16 ? proj_step_workspace_bytes(T, h, Q, O, p) : 0;
  size_t wg = w1 > w2 ? w1 : w2;
  const size_t both = two_wgrads_bytes(T, h, pQ);
  wg = wg > both ? wg : both;
  *bytes = rows + wg;
  return TP_OK;
}

int tp_attn_proj_step_plan(int64_t T, int64_t h, int64_t Q, int64_t O, int p, tp_dtype dt,
                           int* fused) {
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(h) || !dim_ok(Q) || !dim_ok(O) || p < 1 || p > kMaxPartials)
    return TP_ERR_SHAPE;
  if (fused) *fused = dt == TP_BF16 && proj_step_supported(T, h, Q, O, p);
  return TP_OK;
}

int tp_attn_proj_step(const void* X, const void* W, const void* Ow, const void* C,
                      const void* dZa, const void* dQKV, void* QKV, float* Zpa, void* Za,
                      void* dC, float* dOw, float* dW, float* dXqp, void* dXq, int64_t T,
                      int64_t h, int64_t Q, int64_t O, int p, int64_t ld_x, int64_t ld_w,
                      int64_t ld_ow, int64_t ld_c, int64_t ld_dz, int64_t ld_dqkv, int64_t ld_qkv,
                      int64_t ld_dc, int64_t ld_za, int64_t ld_dxq, int64_t ld_dow, int64_t ld_dw,
                      int stages, tp_dtype dt, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (stages < 1 || stages > 31) return TP_ERR_SHAPE;
  if (!dtype_ok(dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(h) || !dim_ok(Q) || !dim_ok(O) || p < 1 || p > kMaxPartials)
    return TP_ERR_SHAPE;
  const int64_t pQ = static_cast<int64_t>(p) * Q, pO = static_cast<int64_t>(p) * O;
  if (!dim_ok(pQ) || !dim_ok(pO) || ld_x < h || ld_w < pQ || ld_ow < h || ld_c < pO ||
      ld_dz < h || ld_dqkv < pQ || ld_qkv < pQ || ld_dc < pO || ld_za < h || ld_dxq < h ||
      ld_dow < h || ld_dw < pQ)
    return TP_ERR_SHAPE;
  // the operands each stage reads and writes
  const bool sq = stages & 1, so = stages & 2, sc = stages & 4, sx = stages & 8, sw = stages & 16;
  if ((sq && (!X || !W || !QKV)) || (so && (!C || !Ow || !Zpa || !Za)) ||
      (sc && (!dZa || !Ow || !dC)) || (sx && (!dQKV || !W || !dXqp || !dXq)) ||
      (sw && (!C || !dZa || !dOw || !X || !dQKV || !dW)))
    return TP_ERR_NULL;
  size_t need = 0;
  int st = tp_attn_proj_step_workspace_size(T, h, Q, O, p, dt, &need);
  if (st != TP_OK) return st;
  if (!workspace || workspace_bytes < need) return TP_ERR_WORKSPACE;
  const size_t es = dt == TP_BF16 ? 2 : 4;
  auto row_ok = [](const void* q, int64_t ld, size_t e) {
    return !q || (aligned(q, 16) && (ld * static_cast<int64_t>(e)) % 16 == 0);
  };
  const bool fused = dt == TP_BF16 && proj_step_supported(T, h, Q, O, p) &&
                     row_ok(X, ld_x, es) && row_ok(W, ld_w, es) && row_ok(Ow, ld_ow, es) &&
                     row_ok(C, ld_c, es) && row_ok(dZa, ld_dz, es) &&
                     row_ok(dQKV, ld_dqkv, es) && row_ok(QKV, ld_qkv, es) &&
                     row_ok(dC, ld_dc, es) && row_ok(Za, ld_za, es) && row_ok(dXq, ld_dxq, es) &&
                     row_ok(Zpa, h, 4) && row_ok(dXqp, h, 4) && aligned(workspace, 256);
  const size_t rows = dt == TP_BF16 ? proj_step_workspace_bytes(T, h, Q, O, p) : 0;
  // the dXq sum rides in the stacked weight-gradient launch, as in the MLP step
  const bool dx_in_wgrads = fused && sx && sw && two_wgrads_slot_free(pO, h, h, pQ, T);
  const RowSumParams dxsum{dXqp, p, dXq, T, h, ld_dxq};
  if (fused && (stages & 15)) {
    ProjParams s{};
    s.x = X;
    s.w = W;
    s.ow = Ow;
    s.c = C;
    s.dz = dZa;
    s.dqkv = dQKV;
    s.qkv = QKV;
    s.dc = dC;
    s.zp = Zpa;
    s.dxp = dXqp;
    s.z = Za;
    s.dx = dXq;
    s.T = T;
    s.h = h;
    s.Q = Q;
    s.O = O;
    s.p = p;
    s.ld_x = ld_x;
    s.ld_w = ld_w;
    s.ld_ow = ld_ow;
    s.ld_c = ld_c;
    s.ld_dz = ld_dz;
    s.ld_dqkv = ld_dqkv;
    s.ld_qkv = ld_qkv;
    s.ld_dc = ld_dc;
    s.ld_z = ld_za;
    s.ld_dx = ld_dxq;
    s.phases = stages & 15;
    s.no_dx_sum = dx_in_wgrads;
    st = hip_status(launch_proj_rows(s, workspace, stream));
    if (st != TP_OK) return st;
  } else if (stages & 15) {
    // one call per product, shard by shard, then the sums
    const float* zparts[kMaxPartials];
    const float* dparts[kMaxPartials];
    for (int i = 0; i < p; ++i) {
      zparts[i] = Zpa + i * T * h;
      dparts[i] = dXqp + i * T * h;
    }
    auto col = [&](const void* q, int64_t off) { return static_cast<const char*>(q) + off * es; };
    for (int i = 0; i < p; ++i) {
      const void* Wi = col(W, i * Q);
      const void* Oi = col(Ow, i * O * ld_ow);
      if (sq) {
        st = tp_column_linear_fwd(X, Wi, nullptr, static_cast<char*>(QKV) + i * Q * es, nullptr,
                                  T, h, Q, ld_x, ld_w, ld_qkv, dt, TP_ACT_NONE, stream);
        if (st != TP_OK) return st;
      }
      if (so) {
        st = tp_row_linear_fwd_partial(col(C, i * O), Oi, Zpa + i * T * h, T, O, h, ld_c, ld_ow,
                                       h, dt, stream);
        if (st != TP_OK) return st;
      }
      if (sc) {
        st = tp_linear_bwd_dgrad(dZa, Oi, nullptr, TP_ACT_NONE,
                                 static_cast<char*>(dC) + i * O * es, T, O, h, ld_dz, ld_ow, ld_dc,
                                 ld_dc, dt, dt, stream);
        if (st != TP_OK) return st;
      }
      if (sx) {
        st = tp_linear_bwd_dgrad(col(dQKV, i * Q), Wi, nullptr, TP_ACT_NONE, dXqp + i * T * h, T,
                                 h, Q, ld_dqkv, ld_w, h, h, dt, TP_F32, stream);
        if (st != TP_OK) return st;
      }
    }
    if (so) {
      st = tp_reduce_partials(zparts, p, nullptr, Za, T, h, h, ld_za, dt, stream);
      if (st != TP_OK) return st;
    }
    if (sx) {
      st = tp_reduce_partials(dparts, p, nullptr, dXq, T, h, h, ld_dxq, dt, stream);
      if (st != TP_OK) return st;
    }
  }
  if (sw) {
    // dO = C^T dZa ([p*O, h]) and dW = X^T dQKV ([h, p*Q]) over the stacked shards
    // past the row counters in either path (they must stay zero)
    char* w = static_cast<char*>(workspace) + rows;
    return two_wgrads(C, dZa, dOw, nullptr, pO, h, ld_c, ld_dz, ld_dow, X, dQKV, dW, nullptr, h,
                      pQ, ld_x, ld_dqkv, ld_dw, T, dt, w, workspace_bytes - rows,
                      stream, dx_in_wgrads ? &dxsum : nullptr);
  }
  return TP_OK;
}

int tp_reduce_partials(const float* const* partials, int p, const void* bias, void* out,
                       int64_t T, int64_t h, int64_t ld_p, int64_t ld_out, tp_dtype out_dt,
                       hipStream_t stream) {
  if (!partials || !out) return TP_ERR_NULL;
  if (p < 1 || p > kMaxPartials) return TP_ERR_SHAPE;
  for (int i = 0; i < p; ++i)
    if (!partials[i]) return TP_ERR_NULL;
  if (!dtype_ok(out_dt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(h)) return TP_ERR_SHAPE;
  if (ld_p < h || ld_out < h) return TP_ERR_SHAPE;
  ReduceParams r{};
  for (int i = 0; i < p; ++i) r.parts[i] = partials[i];
  r.p = p;
  r.bias = bias;
  r.out = out;
  r.T = T;
  r.N = h;
  r.ldp = ld_p;
  r.ldo = ld_out;
  r.out_bf16 = out_dt == TP_BF16;
  return hip_status(launch_reduce(r, stream));
}

int tp_bias_act(const void* U, const void* bias, void* Y, int64_t T, int64_t n, int64_t ld_u,
                int64_t ld_y, tp_dtype in_dt, tp_dtype out_dt, tp_act act, hipStream_t stream) {
  if (!U || !Y) return TP_ERR_NULL;
  if (!dtype_ok(in_dt) || !dtype_ok(out_dt)) return TP_ERR_DTYPE;
  if (!act_ok(act)) return TP_ERR_ACT;
  if (!dim_ok(T) || !dim_ok(n)) return TP_ERR_SHAPE;
  if (ld_u < n || ld_y < n) return TP_ERR_SHAPE;
  BiasActParams b{};
  b.u = U;
  b.bias = bias;
  b.y = Y;
  b.T = T;
  b.N = n;
  b.ldu = ld_u;
  b.ldy = ld_y;
  b.in_bf16 = in_dt == TP_BF16;
  b.u_f32 = in_dt == TP_F32;
  b.out_bf16 = out_dt == TP_BF16;
  b.act = act == TP_ACT_GELU_TANH ? ACT_GELU : ACT_NONE;
  return hip_status(launch_bias_act(b, stream));
}

// Attention core of `shards` shards of `heads` heads each in one launch: shard
// s's [Q | K | V] block is columns s*3*heads*64 .. of QKV (as tp_attn_proj_step
// stacks it), its heads are C's columns s*heads*64 .., and lse and delta are
// [batch, shards*heads, seq].
static int attention_fwd_impl(const void* QKV, void* C, float* lse, int64_t batch, int64_t seq,
                              int64_t heads, int64_t shards, int64_t head_dim, int64_t ld_qkv,
                              int64_t ld_c, int causal, tp_dtype dt, hipStream_t stream) {
  if (!QKV || !C) return TP_ERR_NULL;
  if (dt != TP_BF16) return TP_ERR_DTYPE;
  if (!dim_ok(batch) || !dim_ok(seq) || !dim_ok(heads) || shards < 1 || shards > kMaxPartials ||
      head_dim != 64)
    return TP_ERR_SHAPE;
  const int64_t all = heads * shards;
  if (ld_qkv < 3 * all * head_dim || ld_c < all * head_dim) return TP_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(QKV) & 15) || (ld_qkv & 7) ||
      (reinterpret_cast<uintptr_t>(C) & 7) || (ld_c & 3))
    return TP_ERR_SHAPE;
  if (batch * seq > kMaxDim) return TP_ERR_SHAPE;
  AttnParams a{};
  a.qkv = QKV;
  a.c = C;
  a.lse = lse;
  a.batch = batch;
  a.seq = seq;
  a.heads = all;
  a.group = heads;
  a.ld_qkv = ld_qkv;
  a.ld_c = ld_c;
  a.causal = causal != 0;
  a.scale_log2 = static_cast<float>(1.4426950408889634 / 8.0);  // log2(e) / sqrt(64)
  return hip_status(launch_attention_fwd(a, stream));
}

static int attention_bwd_impl(const void* QKV, const void* C, const void* dC, const float* lse,
                              float* delta, void* dQKV, int64_t batch, int64_t seq, int64_t heads,
                              int64_t shards, int64_t head_dim, int64_t ld_qkv, int64_t ld_c,
                              int64_t ld_dc, int64_t ld_dqkv, int causal, tp_dtype dt,
                              hipStream_t stream) {
  if (!QKV || !C || !dC || !lse || !delta || !dQKV) return TP_ERR_NULL;
  if (dt != TP_BF16) return TP_ERR_DTYPE;
  if (!dim_ok(batch) || !dim_ok(seq) || !dim_ok(heads) || shards < 1 || shards > kMaxPartials ||
      head_dim != 64)
    return TP_ERR_SHAPE;
  const int64_t all = heads * shards, hd = all * head_dim;
  if (ld_qkv < 3 * hd || ld_c < hd || ld_dc < hd || ld_dqkv < 3 * hd) return TP_ERR_SHAPE;
  auto al = [](const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) == 0; };
  if (!al(QKV, 16) || (ld_qkv & 7) || !al(C, 16) || (ld_c & 7) || !al(dC, 16) || (ld_dc & 7) ||
      !al(dQKV, 8) || (ld_dqkv & 3) || !al(lse, 4) || !al(delta, 4))
    return TP_ERR_SHAPE;
  if (batch * seq > kMaxDim) return TP_ERR_SHAPE;
  AttnBwdParams a{};
  a.qkv = QKV;
  a.c = C;
  a.dc = dC;
  a.lse = lse;
  a.delta = delta;
  a.dqkv = dQKV;
  a.batch = batch;
  a.seq = seq;
  a.heads = all;
  a.group = heads;
  a.ld_qkv = ld_qkv;
  a.ld_c = ld_c;
  a.ld_dc = ld_dc;
  a.ld_dqkv = ld_dqkv;
  a.causal = causal != 0;
  a.scale_log2 = static_cast<float>(1.4426950408889634 / 8.0);  // log2(e) / sqrt(64)
  return hip_status(launch_attention_bwd(a, stream));
}

int tp_attention_fwd(const void* QKV, void* C, float* lse, int64_t batch, int64_t seq,
                     int64_t heads, int64_t head_dim, int64_t ld_qkv, int64_t ld_c, int causal,
                     tp_dtype dt, hipStream_t stream) {
  return attention_fwd_impl(QKV, C, lse, batch, seq, heads, 1, head_dim, ld_qkv, ld_c, causal, dt,
                            stream);
}

int tp_attention_bwd(const void* QKV, const void* C, const void* dC, const float* lse,
                     float* delta, void* dQKV, int64_t batch, int64_t seq, int64_t heads,
                     int64_t head_dim, int64_t ld_qkv, int64_t ld_c, int64_t ld_dc,
                     int64_t ld_dqkv, int causal, tp_dtype dt, hipStream_t stream) {
  return attention_bwd_impl(QKV, C, dC, lse, delta, dQKV, batch, seq, heads, 1, head_dim, ld_qkv,
                            ld_c, ld_dc, ld_dqkv, causal, dt, stream);
}

int tp_attention_fwd_shards(const void* QKV, void* C, float* lse, int64_t batch, int64_t seq,
                            int64_t heads, int64_t shards, int64_t head_dim, int64_t ld_qkv,
                            int64_t ld_c, int causal, tp_dtype dt, hipStream_t stream) {
  return attention_fwd_impl(QKV, C, lse, batch, seq, heads, shards, head_dim, ld_qkv, ld_c,
                            causal, dt, stream);
}

int tp_attention_bwd_shards(const void* QKV, const void* C, const void* dC, const float* lse,
                            float* delta, void* dQKV, int64_t batch, int64_t seq, int64_t heads,
                            int64_t shards, int64_t head_dim, int64_t ld_qkv, int64_t ld_c,
                            int64_t ld_dc, int64_t ld_dqkv, int causal, tp_dtype dt,
                            hipStream_t stream) {
  return attention_bwd_impl(QKV, C, dC, lse, delta, dQKV, batch, seq, heads, shards, head_dim,
                            ld_qkv, ld_c, ld_dc, ld_dqkv, causal, dt, stream);
}

int tp_fp8_quantize_workspace_size(int64_t rows, int64_t cols, size_t* bytes) {
  if (!bytes) return TP_ERR_NULL;
  if (!dim_ok(rows) || !dim_ok(cols)) return TP_ERR_SHAPE;
  *bytes = kFp8AmaxBlocks * sizeof(float);
  return TP_OK;
}

int tp_fp8_quantize(const void* X, int64_t rows, int64_t cols, int64_t ld_x, tp_dtype dt, tp_fp8_format fmt,
                    int transpose, void* Q, int64_t ld_q, float* scale_inv, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  if (!X || !Q || !scale_inv) return TP_ERR_NULL;
  if (!dtype_ok(dt) || !fmt_ok(fmt)) return TP_ERR_DTYPE;
  if (!dim_ok(rows) || !dim_ok(cols) || rows * cols > (int64_t(1) << 40)) return TP_ERR_SHAPE;
  if (ld_x < cols || ld_q < (transpose ? rows : cols)) return TP_ERR_SHAPE;
  if (!aligned(scale_inv, 4) || !aligned(X, dt == TP_BF16 ? 2 : 4)) return TP_ERR_SHAPE;
  if (!workspace || workspace_bytes < kFp8AmaxBlocks * sizeof(float) || !aligned(workspace, 4))
    return TP_ERR_WORKSPACE;
  Fp8QuantParams q{};
  q.x = X;
  q.rows = rows;
  q.cols = cols;
  q.ld_x = ld_x;
  q.x_bf16 = dt == TP_BF16;
  q.fmt = fmt;
  q.transpose = transpose != 0;
  q.q = static_cast<uint8_t*>(Q);
  q.ld_q = ld_q;
  q.scale_inv = scale_inv;
  q.partial = static_cast<float*>(workspace);
  q.vec_in = aligned(X, 16) && ld_x % (dt == TP_BF16 ? 8 : 4) == 0;
  q.vec_out = q.transpose ? (aligned(Q, 16) && ld_q % 16 == 0) : (aligned(Q, 8) && ld_q % 8 == 0);
  return hip_status(launch_fp8_quantize(q, stream));
}

int tp_fp8_quantize_both(const void* X, int64_t rows, int64_t cols, int64_t ld_x, tp_dtype dt,
                         tp_fp8_format fmt, void* Q, int64_t ld_q, void* Qt, int64_t ld_qt,
                         float* scale_inv, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  Fp8QuantParams q{};
  const int st = fp8_both_params(X, rows, cols, ld_x, dt, fmt, Q, ld_q, Qt, ld_qt, scale_inv,
                                 workspace, workspace_bytes, &q);
  if (st != TP_OK) return st;
  return hip_status(launch_fp8_quantize(q, stream));
}

int tp_fp8_quantize_multi_workspace_size(int n, size_t* bytes) {
  if (!bytes) return TP_ERR_NULL;
  if (n < 1 || n > kFp8MaxMulti) return TP_ERR_SHAPE;
  *bytes = static_cast<size_t>(n) * kFp8AmaxBlocks * sizeof(float);
  return TP_OK;
}

int tp_fp8_quantize_both_multi(int n, const void* const* X, const int64_t* rows,
                               const int64_t* cols, const int64_t* ld_x, const int* dt,
                               const int* fmt, void* const* Q, const int64_t* ld_q,
                               void* const* Qt, const int64_t* ld_qt, float* const* scale_inv,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!X || !rows || !cols || !ld_x || !dt || !fmt || !Q || !ld_q || !Qt || !ld_qt ||
      !scale_inv)
    return TP_ERR_NULL;
  if (n < 1 || n > kFp8MaxMulti) return TP_ERR_SHAPE;
  if (!workspace || workspace_bytes < static_cast<size_t>(n) * kFp8AmaxBlocks * sizeof(float))
    return TP_ERR_WORKSPACE;
  Fp8QuantParams ps[kFp8MaxMulti];
  for (int i = 0; i < n; ++i) {
    // tensor i's per-block maxima in its own slice of the workspace
    void* wi = static_cast<char*>(workspace) + static_cast<size_t>(i) * kFp8AmaxBlocks * sizeof(float);
    const int st = fp8_both_params(X[i], rows[i], cols[i], ld_x[i], dt[i], fmt[i], Q[i], ld_q[i],
                                   Qt[i], ld_qt[i], scale_inv[i], wi,
                                   kFp8AmaxBlocks * sizeof(float), &ps[i]);
    if (st != TP_OK) return st;
  }
  return hip_status(launch_fp8_quantize_multi(ps, n, stream));
}

static int fp8_column_fwd(const void* Xq, const void* Atq, const float* x_scale_inv,
                          const float* a_scale_inv, const void* bias_i, void* Y_i, void* U_i,
                          int64_t T, int64_t h, int64_t n, int64_t ld_x, int64_t ld_at,
                          int64_t ld_y, tp_act act, float* amax, hipStream_t stream) {
  if (!Xq || !Atq || !x_scale_inv || !a_scale_inv || !Y_i) return TP_ERR_NULL;
  if (!act_ok(act)) return TP_ERR_ACT;
  if (act != TP_ACT_NONE && !U_i) return TP_ERR_NULL;
  if (act == TP_ACT_NONE && (bias_i || U_i)) return TP_ERR_ACT;
  if (!dim_ok(T) || !dim_ok(h) || !dim_ok(n) || ld_y < n) return TP_ERR_SHAPE;
  if (!fp8_operand_ok(Xq, ld_x, h) || !fp8_operand_ok(Atq, ld_at, h)) return TP_ERR_SHAPE;
  GemmParams p{};
  p.a = Xq;
  p.b = Atq;
  p.c = Y_i;
  p.c2 = U_i;
  p.bias = bias_i;
  p.M = T;
  p.N = n;
  p.K = h;
  p.lda = ld_x;
  p.ldb = ld_at;
  p.ldc = ld_y;
  p.ldc2 = ld_y;
  p.epi = EPI_BIAS_ACT;
  p.act = act == TP_ACT_GELU_TANH ? ACT_GELU : ACT_NONE;
  p.out_bf16 = 1;
  p.a_kcontig = p.b_kcontig = 1;
  p.f8 = 1;  // E4M3 x E4M3
  p.sa_inv = x_scale_inv;
  p.sb_inv = a_scale_inv;
  p.amax = amax;
  return run_gemm_fp8(p, false, 0, stream);
}

int tp_fp8_column_linear_fwd(const void* Xq, const void* Atq, const float* x_scale_inv,
                             const float* a_scale_inv, const void* bias_i, void* Y_i, void* U_i,
                             int64_t T, int64_t h, int64_t n, int64_t ld_x, int64_t ld_at,
                             int64_t ld_y, tp_act act, hipStream_t stream) {
  return fp8_column_fwd(Xq, Atq, x_scale_inv, a_scale_inv, bias_i, Y_i, U_i, T, h, n, ld_x, ld_at,
                        ld_y, act, nullptr, stream);
}

int tp_fp8_column_linear_fwd_amax(const void* Xq, const void* Atq, const float* x_scale_inv,
                                  const float* a_scale_inv, const void* bias_i, void* Y_i,
                                  void* U_i, int64_t T, int64_t h, int64_t n, int64_t ld_x,
                                  int64_t ld_at, int64_t ld_y, float* y_amax,
                                  hipStream_t stream) {
  if (!y_amax) return TP_ERR_NULL;
  if (fp8_amax_slot_count(T, n, h) == 0) return TP_ERR_SHAPE;
  return fp8_column_fwd(Xq, Atq, x_scale_inv, a_scale_inv, bias_i, Y_i, U_i, T, h, n, ld_x, ld_at,
                        ld_y, TP_ACT_GELU_TANH, y_amax, stream);
}

int tp_fp8_row_linear_fwd_partial(const void* Yq, const void* Btq, const float* y_scale_inv,
                                  const float* b_scale_inv, float* Zp_i, int64_t T, int64_t k,
                                  int64_t h, int64_t ld_y, int64_t ld_bt, int64_t ld_z,
                                  hipStream_t stream) {
  if (!Yq || !Btq || !y_scale_inv || !b_scale_inv || !Zp_i) return TP_ERR_NULL;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(h) || ld_z < h) return TP_ERR_SHAPE;
  if (!fp8_operand_ok(Yq, ld_y, k) || !fp8_operand_ok(Btq, ld_bt, k)) return TP_ERR_SHAPE;
  GemmParams p{};
  p.a = Yq;
  p.b = Btq;
  p.c = Zp_i;
  p.M = T;
  p.N = h;
  p.K = k;
  p.lda = ld_y;
  p.ldb = ld_bt;
  p.ldc = ld_z;
  p.epi = EPI_STORE;
  p.out_bf16 = 0;
  p.a_kcontig = p.b_kcontig = 1;
  p.f8 = 1;
  p.sa_inv = y_scale_inv;
  p.sb_inv = b_scale_inv;
  return run_gemm_fp8(p, false, 0, stream);
}

static int fp8_dgrad(const void* dOutq, const void* Wq, const float* dout_scale_inv,
                     const float* w_scale_inv, tp_fp8_format dout_fmt, const void* U, tp_act act,
                     void* dIn, int64_t T, int64_t k, int64_t n, int64_t ld_dout, int64_t ld_w,
                     int64_t ld_u, int64_t ld_din, tp_dtype out_dt, float* amax,
                     hipStream_t stream) {
  if (!dOutq || !Wq || !dout_scale_inv || !w_scale_inv || !dIn) return TP_ERR_NULL;
  if (!fmt_ok(dout_fmt) || !dtype_ok(out_dt)) return TP_ERR_DTYPE;
  if (!act_ok(act)) return TP_ERR_ACT;
  if (act != TP_ACT_NONE && !U) return TP_ERR_NULL;
  if (act != TP_ACT_NONE && out_dt != TP_BF16) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n) || ld_din < k) return TP_ERR_SHAPE;
  if (act != TP_ACT_NONE && ld_u < k) return TP_ERR_SHAPE;
  if (!fp8_operand_ok(dOutq, ld_dout, n) || !fp8_operand_ok(Wq, ld_w, n)) return TP_ERR_SHAPE;
  GemmParams p{};
  p.a = dOutq;
  p.b = Wq;
  p.c = dIn;
  p.u = U;
  p.M = T;
  p.N = k;
  p.K = n;
  p.lda = ld_dout;
  p.ldb = ld_w;
  p.ldc = ld_din;
  p.ldu = ld_u;
  p.epi = act != TP_ACT_NONE ? EPI_DACT : EPI_STORE;
  p.act = act == TP_ACT_GELU_TANH ? ACT_GELU : ACT_NONE;
  p.out_bf16 = out_dt == TP_BF16;
  p.a_kcontig = p.b_kcontig = 1;
  p.f8 = 1 + dout_fmt;  // dOut in dout_fmt, W in E4M3
  p.sa_inv = dout_scale_inv;
  p.sb_inv = w_scale_inv;
  p.amax = amax;
  return run_gemm_fp8(p, false, 0, stream);
}

int tp_fp8_linear_bwd_dgrad(const void* dOutq, const void* Wq, const float* dout_scale_inv,
                            const float* w_scale_inv, tp_fp8_format dout_fmt, const void* U, tp_act act,
                            void* dIn, int64_t T, int64_t k, int64_t n, int64_t ld_dout,
                            int64_t ld_w, int64_t ld_u, int64_t ld_din, tp_dtype out_dt,
                            hipStream_t stream) {
  return fp8_dgrad(dOutq, Wq, dout_scale_inv, w_scale_inv, dout_fmt, U, act, dIn, T, k, n,
                   ld_dout, ld_w, ld_u, ld_din, out_dt, nullptr, stream);
}

int tp_fp8_linear_bwd_dgrad_amax(const void* dOutq, const void* Wq, const float* dout_scale_inv,
                                 const float* w_scale_inv, tp_fp8_format dout_fmt, const void* U,
                                 void* dIn, int64_t T, int64_t k, int64_t n, int64_t ld_dout,
                                 int64_t ld_w, int64_t ld_u, int64_t ld_din, float* din_amax,
                                 hipStream_t stream) {
  if (!din_amax) return TP_ERR_NULL;
  if (fp8_amax_slot_count(T, k, n) == 0) return TP_ERR_SHAPE;
  return fp8_dgrad(dOutq, Wq, dout_scale_inv, w_scale_inv, dout_fmt, U, TP_ACT_GELU_TANH, dIn, T,
                   k, n, ld_dout, ld_w, ld_u, ld_din, TP_BF16, din_amax, stream);
}

int tp_fp8_amax_slots(int64_t M, int64_t N, int64_t K, int64_t* slots) {
  if (!slots) return TP_ERR_NULL;
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return TP_ERR_SHAPE;
  *slots = fp8_amax_slot_count(M, N, K);
  return *slots > 0 ? TP_OK : TP_ERR_SHAPE;
}

int tp_fp8_quantize_both_from_amax(const void* X, int64_t rows, int64_t cols, int64_t ld_x,
                                   tp_dtype dt, tp_fp8_format fmt, void* Q, int64_t ld_q, void* Qt,
                                   int64_t ld_qt, float* scale_inv, const float* amax,
                                   int64_t n_amax, hipStream_t stream) {
  if (!amax) return TP_ERR_NULL;
  if (n_amax < 1 || n_amax > 0x7fffffff || !aligned(amax, 4)) return TP_ERR_SHAPE;
  Fp8QuantParams q{};
  // the maxima are given: the parameter check's workspace is the amax array
  const int st = fp8_both_params(X, rows, cols, ld_x, dt, fmt, Q, ld_q, Qt, ld_qt, scale_inv,
                                 const_cast<float*>(amax), kFp8AmaxBlocks * sizeof(float), &q);
  if (st != TP_OK) return st;
  q.nblk = static_cast<int>(n_amax);
  return hip_status(launch_fp8_cast(q, stream));
}

int tp_fp8_linear_bwd_wgrad_workspace_size(int64_t T, int64_t k, int64_t n, size_t* bytes) {
  if (!bytes) return TP_ERR_NULL;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n)) return TP_ERR_SHAPE;
  *bytes = fp8_wgrad_split_bytes(T, k, n) + colsum_workspace_bytes(T, n);
  return TP_OK;
}

int tp_fp8_linear_bwd_wgrad(const void* Intq, const void* dOuttq, const float* in_scale_inv,
                            const float* dout_scale_inv, tp_fp8_format dout_fmt, float* dW,
                            const void* dOut, float* dbias, int64_t T, int64_t k, int64_t n,
                            int64_t ld_int, int64_t ld_doutt, int64_t ld_dw, int64_t ld_dout,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!Intq || !dOuttq || !in_scale_inv || !dout_scale_inv || !dW) return TP_ERR_NULL;
  if (dbias && !dOut) return TP_ERR_NULL;
  if (!fmt_ok(dout_fmt)) return TP_ERR_DTYPE;
  if (!dim_ok(T) || !dim_ok(k) || !dim_ok(n) || ld_dw < n) return TP_ERR_SHAPE;
  if (dbias && ld_dout < n) return TP_ERR_SHAPE;
  if (!fp8_operand_ok(Intq, ld_int, T) || !fp8_operand_ok(dOuttq, ld_doutt, T)) return TP_ERR_SHAPE;
  const size_t split_bytes = fp8_wgrad_split_bytes(T, k, n);
  const size_t cs_bytes = dbias ? colsum_workspace_bytes(T, n) : 0;
  if (split_bytes + cs_bytes > 0 && (!workspace || workspace_bytes < split_bytes + cs_bytes))
    return TP_ERR_WORKSPACE;
  GemmParams p{};
  p.a = Intq;
  p.b = dOuttq;
  p.c = dW;
  p.M = k;
  p.N = n;
  p.K = T;
  p.lda = ld_int;
  p.ldb = ld_doutt;
  p.ldc = ld_dw;
  p.epi = EPI_STORE;
  p.out_bf16 = 0;
  p.ws = static_cast<float*>(workspace);
  p.a_kcontig = p.b_kcontig = 1;
  p.f8 = 1 + 2 * dout_fmt;  // In^T in E4M3, dOut^T in dout_fmt
  p.sa_inv = in_scale_inv;
  p.sb_inv = dout_scale_inv;
  ColsumParams c{};
  c.src = dOut;
  c.T = T;
  c.N = n;
  c.ld = ld_dout;
  c.src_bf16 = 1;
  c.dbias = dbias;
  c.ws = dbias ? reinterpret_cast<float*>(static_cast<char*>(workspace) + split_bytes) : nullptr;
  return run_gemm_fp8(p, true, split_bytes, stream, dbias ? &c : nullptr);
}

int tp_gemm_plan(int64_t M, int64_t N, int64_t K, int allow_split, int* tile, int* splitk,
                 int64_t* k_chunk) {
  if (!dim_ok(M) || !dim_ok(N) || !dim_ok(K)) return TP_ERR_SHAPE;
  const SplitPlan plan = plan_gemm_bf16(M, N, K, allow_split != 0);
  if (tile) *tile = plan.tile;
  if (splitk) *splitk = plan.splitk;
  if (k_chunk) *k_chunk = plan.k_chunk;
  return TP_OK;
}

int tp_set_gemm_override(int tile, int splitk) {
  return set_gemm_override(tile, splitk) ? TP_OK : TP_ERR_SHAPE;
}

const char* tp_status_string(int status) {
  switch (status) {
    case TP_OK:
      return "TP_OK";
    case TP_ERR_NULL:
      return "TP_ERR_NULL: a required pointer is NULL";
    case TP_ERR_SHAPE:
      return "TP_ERR_SHAPE: bad dimension, leading dimension or shard count";
    case TP_ERR_DTYPE:
      return "TP_ERR_DTYPE: unknown or unsupported dtype";
    case TP_ERR_ACT:
      return "TP_ERR_ACT: unknown activation";
    case TP_ERR_WORKSPACE:
      return "TP_ERR_WORKSPACE: workspace missing or too small";
    case TP_ERR_SCRATCH:
      return "TP_ERR_SCRATCH: shape needs more than the library's static scratch";
    case TP_ERR_HIP:
      return "TP_ERR_HIP: a HIP launch failed";
    default:
      return "unknown tp_status";
  }
}

int tp_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
