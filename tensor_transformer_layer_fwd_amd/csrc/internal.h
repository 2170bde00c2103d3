// Internal interface between the C ABI (tp_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpmlp {

enum Epilogue : int {
  EPI_STORE = 0,     // C (+)= acc
  EPI_BIAS_ACT = 1,  // U = acc + bias; C = act(U); C2 = U (if C2)
  EPI_DACT = 2,      // C = acc * act'(Uin); C2 = act(Uin) (if C2: recompute)
};

enum Act : int { ACT_NONE = 0, ACT_GELU = 1 };

// Column-sum (bias gradient) request: dbias[n] (+)= sum_t src[t, n].
struct ColsumParams {
  const void* src;
  int64_t T, N, ld;
  int src_bf16;
  float* dbias;
  int accumulate;
  float* ws;  // partial sums [nchunks, N]
};

constexpr int kColsumRows = 64;  // rows summed per block in the first pass

// One GEMM C[M,N] = op(A)[M,K] * op(B)[K,N] with a fused epilogue.
//   a_kcontig: A stored [M,K] (true) or [K,M] (false), row stride lda
//   b_kcontig: B stored [N,K] (true) or [K,N] (false), row stride ldb
struct GemmParams {
  const void* a;
  const void* b;
  void* c;         // output [M,N], ldc; fp32 or bf16 (out_bf16)
  void* c2;        // EPI_BIAS_ACT: pre-activation U; EPI_DACT: recomputed act(Uin);
                   // row stride ldc2, dtype of c; may be null
  const void* bias;  // EPI_BIAS_ACT: [N], dtype of the operands; may be null
  const void* u;     // EPI_DACT: saved pre-activation [M,N], ldu, dtype of the operands
  // EPI_DACT on the pipelined kernel, nullable: column sums of the stored
  // (bf16) outputs over each block tile's BM rows, one row of N per tile row
  // (row stride N): the first pass of the bias gradient of the next layer down
  float* cs_part;
  int64_t M, N, K;
  int64_t lda, ldb, ldc, ldu, ldc2;
  int epi, act;
  int out_bf16;    // output dtype of c / c2
  int accumulate;  // EPI_STORE with fp32 output: C += acc
  // split-K: grid slice z covers K range [z*k_chunk, min(K,(z+1)*k_chunk)) and
  // writes raw fp32 partials to ws + z*M*N (row stride N); the fix-up kernel
  // then applies the epilogue.
  int splitk;
  int64_t k_chunk;
  float* ws;
  int a_kcontig, b_kcontig;
  // Column sums carried by this launch (weight gradients on the pipelined
  // kernel, fp32 epilogue): cs_blocks extra blocks after all tiles run the
  // cs_units pass-1 units of cs (cs_nchunks row chunks); the fix-up launch
  // then runs pass 2. cs_blocks = 0: none.
  ColsumParams cs;
  int cs_blocks, cs_units, cs_nchunks;
  // FP8 operands (both K-contiguous codes): f8 = 0 for bf16, else
  // 1 + fmt_a + 2 * fmt_b (fmt 0: E4M3, 1: E5M2); the accumulators are
  // multiplied by sa_inv[0] * sb_inv[0] before the epilogue.
  int f8;
  const float* sa_inv;
  const float* sb_inv;
  // bias + GeLU and GeLU' epilogues of the pipelined kernel: when set, each
  // wave stores the largest |stored bf16 value| of its part of the output
  // tile at amax[tile * waves + wave] (tile = tile row * tile columns + tile
  // column), for a quantiser that then needs no pass of its own over them
  float* amax;
  // XCDs the blocks go round-robin over (device_shape().xcds; set by the
  // launchers): each takes a run of consecutive tiles
  int xcds;
};

// Compute units and XCDs of the current device, queried once per device
// (hipDeviceAttributeMultiprocessorCount, hipDeviceAttributeNumberOfXccs).
// Without a device (a host-only process) the MI355X figures, 256 and 8.
struct DeviceShape {
  int cus, xcds;
};
DeviceShape device_shape();


// FP8 quantisation of X [rows, cols] (ld_x, bf16 or fp32) into codes Q
// (ld_q; [cols, rows] when transpose) with per-tensor scaling; scale_inv
// receives 1/s; partial holds kFp8AmaxBlocks floats of per-block maxima.
constexpr int kFp8AmaxBlocks = 1024;
struct Fp8QuantParams {
  const void* x;
  int64_t rows, cols, ld_x;
  int x_bf16;
  int fmt;  // 0: E4M3, 1: E5M2
  int transpose;
  uint8_t* q;
  int64_t ld_q;
  float* scale_inv;
  float* partial;
  int nblk;              // set by the launcher
  int vec_in, vec_out;   // 16-byte input loads / 8- or 16-byte code stores allowed
  // with transpose: also the codes of X itself ([rows, cols], ld_q_rows), or null
  uint8_t* q_rows;
  int64_t ld_q_rows;
  int vec_rows;          // 16-byte stores into q_rows allowed
};
int fp8_amax_blocks(int64_t rows, int64_t cols);
hipError_t launch_fp8_quantize(Fp8QuantParams p, hipStream_t s);
// The cast launch alone, with p.partial / p.nblk holding maxima the caller
// already has (amax slots of the producing GEMM's epilogue).
hipError_t launch_fp8_cast(Fp8QuantParams p, hipStream_t s);
// Up to kFp8MaxMulti tensors, each quantised with transpose (and optionally its
// own layout), in two launches; each tensor has its own partial array.
constexpr int kFp8MaxMulti = 6;
struct Fp8MultiParams {
  Fp8QuantParams t[kFp8MaxMulti];
  int first[kFp8MaxMulti + 1];  // first block of each tensor in the launch
  int n;
};
hipError_t launch_fp8_quantize_multi(const Fp8QuantParams* ps, int n, hipStream_t s);

// Attention core of one shard (forward): QKV [batch*seq, 3*heads*64] bf16 as
// [Q | K | V], C [batch*seq, heads*64] bf16, lse [batch, heads, seq] (or null).
struct AttnParams {
  const void* qkv;
  void* c;
  float* lse;
  int64_t batch, seq, heads, ld_qkv, ld_c;
  // heads per block of QKV columns: head h's Q, K and V are at columns
  // (h / group) * 3 * group * 64 + (h % group) * 64, + group * 64 and
  // + 2 * group * 64 (group = heads: one [Q | K | V] block; one block per
  // shard when several shards' heads run in one launch)
  int64_t group;
  int causal;
  float scale_log2;  // log2(e) / sqrt(head_dim)
};

// Attention core backward: dQKV [batch*seq, 3*heads*64] bf16 ([dQ | dK | dV])
// from QKV, the forward output C, its gradient dC and the forward lse; delta
// [batch, heads, seq] fp32 receives rowsum(dC * C).
struct AttnBwdParams {
  const void* qkv;
  const void* c;
  const void* dc;
  const float* lse;
  float* delta;
  void* dqkv;
  int64_t batch, seq, heads, ld_qkv, ld_c, ld_dc, ld_dqkv;
  int64_t group;  // heads per block of QKV (and dQKV) columns, as AttnParams
  int causal;
  float scale_log2;  // log2(e) / sqrt(head_dim)
};

// The row work of the MLP step of p shards in one persistent launch
// (mlp_step.hip): per XCD, a queue over the XCD's own token rows of every
// shard's fc1 forward (bias + GeLU) and fc2 forward partial, the sum over
// shards, every shard's fc2 dgrad (GeLU derivative) and fc1 dgrad partial, and
// the sum of the dX partials. The weight and bias gradients, which read every
// token row, are products of their own (tp_api.hip).
struct StepParams {
  // operands, row strides in elements (bf16 unless noted)
  const void* x;       // X [T, h], ld_x
  const void* a;       // A [h, p*F], ld_a (shard i: columns i*F ..)
  const void* bias_a;  // [p*F] or null
  const void* b;       // B [p*F, h], ld_b (shard i: rows i*F ..)
  const void* bias_b;  // [h] or null
  const void* dz;      // dZ [T, h], ld_dz
  void* u;             // U, Y, dU [T, p*F], ld_u (shard i: columns i*F ..)
  void* y;
  void* du;
  float* zp;           // Zp, dXp fp32 [p, T, h], compact
  float* dxp;
  void* z;             // Z [T, h], ld_z
  void* dx;            // dX [T, h], ld_dx
  int64_t T, h, F;
  int p;
  int64_t ld_x, ld_a, ld_b, ld_dz, ld_u, ld_z, ld_dx;
  // workspace
  unsigned* err;       // nonzero after a dependency wait gave up
  unsigned long long* clk;  // block 0: s_memtime and s_memrealtime, start and end
  unsigned* ctr;       // counters (mlp_step.hip)
  int xcds, rb, rbx;   // XCDs; token rows of a unit; its row blocks per XCD
  int units_a;         // queue length per XCD
  long long spin;      // polls before a dependency wait gives up
  int phases;          // 1: the forward units, 2: the backward units, 3: both
  int recompute;       // backward: fc2's data-gradient epilogue rebuilds Y = GeLU(U)
  int no_dx_sum;       // backward without the dX sum units (a later launch sums)
};
// Whether launch_mlp_rows supports these shapes (the bf16 tiles, one row slab
// per XCD); and the workspace it needs (0 when unsupported).
bool mlp_step_supported(int64_t T, int64_t h, int64_t F, int p);
size_t mlp_step_workspace_bytes(int64_t T, int64_t h, int64_t F, int p);
// Fills the shapes, queue length and workspace pointers of s (operands,
// phases and recompute set by the caller) and enqueues the launch.
hipError_t launch_mlp_rows(StepParams s, void* workspace, hipStream_t stream);
// The attention projections of p shards in one persistent launch over each
// XCD's own token rows (proj_step.hip): QKV_i = X W_i, the output projection's
// partial Zpa_i = C_i O_i and their sum Za, dC_i = dZa O_i^T, and the partial
// dXqp_i = dQKV_i W_i^T with its sum dXq. Layouts as tp_attn_proj_step's.
struct ProjParams {
  const void* x;     // X [T, h], ld_x
  const void* w;     // W [h, p*Q], ld_w (W_i: columns i*Q ..)
  const void* ow;    // Ow [p*O, h], ld_ow (O_i: rows i*O ..)
  const void* c;     // C [T, p*O], ld_c (C_i: columns i*O ..)
  const void* dz;    // dZa [T, h], ld_dz
  const void* dqkv;  // dQKV [T, p*Q], ld_dqkv
  void* qkv;         // QKV [T, p*Q], ld_qkv
  void* dc;          // dC [T, p*O], ld_dc
  float* zp;         // Zpa, dXqp fp32 [p, T, h], compact
  float* dxp;
  void* z;           // Za [T, h], ld_z
  void* dx;          // dXq [T, h], ld_dx
  int64_t T, h, Q, O;
  int p;
  int64_t ld_x, ld_w, ld_ow, ld_c, ld_dz, ld_dqkv, ld_qkv, ld_dc, ld_z, ld_dx;
  // the units the launch runs: kProjQkv (QKV_i), kProjOut (Zpa_i and Za),
  // kProjDc (dC_i), kProjDx (dXqp_i and dXq)
  int phases;
  // workspace (launch_proj_rows)
  unsigned* err;
  unsigned long long* clk;
  unsigned* ctr;
  int xcds, rb, rbx, units_a;
  long long spin;
  int no_dx_sum;      // with kProjDx: no dXq sum units (a later launch sums)
};
constexpr int kProjQkv = 1, kProjOut = 2, kProjDc = 4, kProjDx = 8;
bool proj_step_supported(int64_t T, int64_t h, int64_t Q, int64_t O, int p);
size_t proj_step_workspace_bytes(int64_t T, int64_t h, int64_t Q, int64_t O, int p);
hipError_t launch_proj_rows(ProjParams s, void* workspace, hipStream_t stream);

// Polls before a dependency wait of launch_mlp_rows gives up, for the calling
// thread: 0 restores the default (about 0.25 s), a negative value gives up at
// the first unsatisfied check.
void set_step_wait_limit(long long polls);
// The polls a dependency wait of the persistent launches takes before giving
// up (set_step_wait_limit's value for the calling thread, or the default).
long long step_wait_polls();

// Reduction over shards.
constexpr int kMaxPartials = 16;
struct ReduceParams {
  const float* parts[kMaxPartials];
  int p;
  const void* bias;
  void* out;
  int64_t T, N, ldp, ldo;
  int out_bf16;
};

struct BiasActParams {
  const void* u;
  const void* bias;
  void* y;
  int64_t T, N, ldu, ldy;
  int in_bf16, u_f32, out_bf16, act;
};

// bf16 GEMM kernels. The pipelined kernel needs M and N to be multiples of
// its tile, K of 64 and 16-byte aligned operands; the general kernel takes
// any shape, stride and alignment.
enum TileId : int {
  kGeneral128x128 = 0,  // general kernel, 128x128 tile
  kGeneral256x256 = 1,  // general kernel, 256x256 tile
  kPipe256x256 = 10,  // 8 waves (two per SIMD), 128x64 per wave
  kPipe256x128 = 11,  // 4 waves, 128x64 per wave
  kPipe128x256 = 12,  // 8 waves, 64x64 per wave
  kPipe128x128 = 13,  // 4 waves, 64x64 per wave
  kPipe256x192 = 14,  // 8 waves, 64x96 per wave
  kPipe128x192 = 15,  // 4 waves, 64x96 per wave
};

// Tile and split-K choice. It depends on the shape only, so the workspace-size
// query and the launch always agree; k_chunk is a multiple of 64.
struct SplitPlan {
  int tile;     // TileId for aligned operands
  int splitk;   // >= 1
  int64_t k_chunk;
};

SplitPlan plan_gemm_bf16(int64_t M, int64_t N, int64_t K, bool allow_split);
// FP8 products: M, N multiples of 128, K of 128 (k_chunk too); tile 0 if none fits.
SplitPlan plan_gemm_fp8(int64_t M, int64_t N, int64_t K, bool allow_split);
hipError_t launch_gemm_fp8(const GemmParams& p, const SplitPlan& plan, hipStream_t s);
int fp8_pipe_epilogue(const GemmParams& p);  // kEpiNone: not supported
// Forced tile / split for later plans (tile 0: none); false for invalid values.
bool set_gemm_override(int tile, int splitk);
int forced_tile();  // the calling thread's forced tile (0: none)
size_t colsum_workspace_bytes(int64_t T, int64_t N);

// Launch per plan: the planned pipelined tile when the operands allow it,
// otherwise the general kernel with the same split.
hipError_t launch_gemm_bf16(const GemmParams& p, const SplitPlan& plan, hipStream_t s);
// Whether launch_gemm_bf16 will run the pipelined kernel, and with which epilogue kind.
int gemm_pipe_epilogue(const GemmParams& p, const SplitPlan& plan);  // kEpiNone: general kernel
hipError_t launch_gemm_bf16_general(const GemmParams& p, const SplitPlan& plan, hipStream_t s);
// Epilogue kinds the pipelined kernel is compiled for (one kernel per kind):
// fp32 store (or split-K partial), bf16 store, bias + GeLU saving the
// pre-activation, and GeLU derivative from the saved pre-activation. All
// outputs 16-byte aligned with row strides a multiple of 8.
enum EpiKind : int { kEpiNone = -1, kEpiF32 = 0, kEpiBF16 = 1, kEpiBiasGelu = 2, kEpiDGelu = 3 };
int pipe_epilogue_kind(const GemmParams& p);  // kEpiNone: use the general kernel
hipError_t launch_gemm_bf16_pipe(const GemmParams& p, const SplitPlan& plan, int ek,
                                 hipStream_t s);
// The backward of one linear layer in one launch: the weight gradient pw (TN,
// fp32 epilogue, K slices and carried column-sum units set as for its own
// launch) and then the data gradient pd (NT, epilogue kind ekd), on the tiles
// of `kind` (below). The split-K fix-up is a launch of its own, or rides in a
// later paired launch.
// An earlier weight gradient finished by spare blocks of a paired launch: its
// split-K fix-up over nfix blocks (vector path, splitk_fixup_vec_ok), then ncs
// column-sum pass-2 units of its carried bias gradient. p NULL: none.
struct PairRider {
  const GemmParams* p = nullptr;
  int nfix = 0, ncs = 0;
  // pass 2 of a second bias gradient (partials in cs2.ws, cs2_nchunks rows of
  // cs2.N) over ncs2 units
  ColsumParams cs2{};
  int ncs2 = 0, cs2_nchunks = 0;
};
// Tiles of a paired backward launch: the weight gradient's (TN, fp32) and the
// data gradient's (NT), each with its own K-tile and stage count.
enum PairKind : int {
  kPairNone = 0,
  kPairSame128x128 = 1,       // both 128x128, 64-wide K-tiles, 3 stages
  kPairW128x128D128x192 = 2,  // weight 128x128 (32-wide, 4 stages), data 128x192 (64, 3)
  kPairSame256x192 = 3,       // both 256x192, 64-wide K-tiles, 2 stages (8 waves)
};
// The paired launch of one bf16 layer with input width k and output width n
// over T tokens: plan.tile holds the PairKind (kPairNone: the layer's products
// cannot pair), plan.splitk / k_chunk the weight gradient's K slices. Shapes
// only, so the workspace query and the call agree.
SplitPlan plan_pair(int64_t T, int64_t k, int64_t n);
// CUs a paired launch of plan `pl` leaves without a tile in its first round.
int pair_free_cus(const SplitPlan& pl, int64_t T, int64_t k, int64_t n);
hipError_t launch_gemm_bwd_pair(const GemmParams& pw, const GemmParams& pd, int kind, int ekd,
                                const PairRider& rider, hipStream_t s);
bool splitk_fixup_vec_ok(const GemmParams& p);
hipError_t launch_gemm_f32(const GemmParams& p, hipStream_t s);
hipError_t launch_splitk_fixup(const GemmParams& p, hipStream_t s);
hipError_t launch_colsum(const ColsumParams& p, hipStream_t s);
// Column-sum pass-1 units for a ColsumParams: row chunks, vector path usable.
int64_t colsum_chunks(const ColsumParams& p);
bool colsum_vec_ok(const ColsumParams& p);
hipError_t launch_colsum_pass2(const ColsumParams& p, int nchunks, hipStream_t s);
// Two weight gradients (TN, fp32) on the 128 x 128 tile in one launch, each
// with its carried column-sum pass-1 units (cs_blocks) after both products'
// tiles. Tiles of the combined list (product 0's, then product 1's) below
// `whole` run over all of K; the others (a remainder over the CUs) run after
// the column-sum units as sk blocks each, over K slices of K / sk rows, and
// store fp32 partials ([tile - whole][slice][128 x 128], compact), which
// launch_wgrad2_finish adds.
struct WgradSplit {
  float* part;
  int whole;  // tiles run over all of K (the combined tile count when sk = 0)
  int sk;     // K slices of each remaining tile; 0: none
};
// A sum over row partials that the stacked weight-gradient launch runs in
// blocks after its tiles: out = sum_i parts[i] (bf16 out, fp32 partials of
// `rows` x N, compact, shard i at i * rows * N); rows a multiple of 16.
struct RowSumParams {
  const float* parts;
  int p;
  void* out;
  int64_t rows, N, ld_out;
};
hipError_t launch_gemm_wgrad2(const GemmParams& p0, const GemmParams& p1, const WgradSplit& sp,
                              const RowSumParams* rs, hipStream_t s);
// After launch_gemm_wgrad2: the sums of the split tiles' K-slice partials
// into their outputs (slices in K order), and the column sums' pass 2 of the
// products with more than one row chunk (n0, n1 chunks; 1 or less: none).
hipError_t launch_wgrad2_finish(const GemmParams& p0, const GemmParams& p1, const WgradSplit& sp,
                                int n0, int n1, hipStream_t s);
hipError_t launch_reduce(const ReduceParams& p, hipStream_t s);
hipError_t launch_bias_act(const BiasActParams& p, hipStream_t s);
hipError_t launch_attention_fwd(const AttnParams& p, hipStream_t s);
hipError_t launch_attention_bwd(const AttnBwdParams& p, hipStream_t s);

}  // namespace tpmlp
