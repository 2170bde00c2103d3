/*
 * tp_mlp.h - C ABI of the tensor-parallel Transformer MLP / attention-projection
 * shard on one MI355X (gfx950).
 *
 * What is computed (page "Megatron", zzmblog.top):
 *   - section "Tensor Parallelism", subsection "mathematical principles": the
 *     first MLP weight A (h x 4h) is split by output columns, A = [A_1 .. A_p],
 *     so Y = [X A_1, .., X A_p] needs no exchange because X is replicated; the
 *     second weight B (4h x h) is split by input rows, B = [B_1; ..; B_p], so
 *     Z = Y_1 B_1 + .. + Y_p B_p, a sum over shards (an All-Reduce across GPUs).
 *   - section "Transformer-layer tensor parallelism": the attention QKV
 *     projection and the first MLP linear are column-split, the attention output
 *     projection and the second MLP linear are row-split.
 *   - the training-script listing on the same page sets activation_func "gelu";
 *     the tanh form of GeLU is used.
 * The backward products (dgrad, wgrad, bias gradients) are not on the pages;
 * they are the textbook derivatives of the forward definitions.
 *
 * One call computes one shard step. On one GPU the p shards of a layer run one
 * after another and tp_reduce_partials stands in for the All-Reduce.
 *
 * Conventions shared by every call:
 *   - Matrices are row-major. "ld" is the row stride in elements (>= the row
 *     width). Weights are stored [in, out]: A_i is h x n, B_i is k x h.
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library
 *     never allocates or frees memory and keeps no pointer after returning;
 *     scratch memory (split-K partials, column-sum partials) is the caller's
 *     workspace, sized by tp_linear_bwd_wgrad_workspace_size.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream).
 *     Outputs are valid after the caller synchronises with that stream.
 *   - dtype TP_BF16: operands are bf16, products accumulate in fp32; outputs
 *     are rounded to bf16 with round-to-nearest-even (NaN stays NaN) unless the
 *     call says fp32. dtype TP_F32: fp32 throughout.
 *   - Errors: arguments are validated on the host before anything is launched.
 *     A bad argument returns a negative tp_status and launches nothing. A failed
 *     launch returns TP_ERR_HIP; tp_last_hip_error() gives the hipError_t (kept
 *     per thread). Faults during execution surface at the caller's stream
 *     synchronisation. Nothing throws across this interface.
 *   - Sizes: every dimension must be >= 1 and < 2^31; any ld >= width is
 *     accepted. Pointers need only the alignment of their element type; 16-byte
 *     aligned pointers with ld a multiple of 8 take the vector-load path.
 *   - Results are deterministic: the same call on the same inputs gives the same
 *     bits (fixed summation orders, no floating-point atomics).
 *   - Calls are reentrant. The library's only mutable state is per thread:
 *     the last HIP error (tp_last_hip_error) and the tile override of
 *     tp_set_gemm_override (a tuning and test hook), plus a per-device cache
 *     of the device's CU and XCD counts, filled on first use. Tile and split
 *     choices depend on the shapes and on those counts, so a workspace query
 *     and the call it sizes agree when made on the same device and thread.
 */
#ifndef TP_MLP_H
#define TP_MLP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TP_OK = 0,
  TP_ERR_NULL = -1,      /* a required pointer is NULL */
  TP_ERR_SHAPE = -2,     /* a dimension < 1 or >= 2^31, an ld below the row width, p out of range */
  TP_ERR_DTYPE = -3,     /* unknown dtype or unsupported dtype combination */
  TP_ERR_ACT = -4,       /* unknown activation */
  TP_ERR_WORKSPACE = -5, /* workspace smaller than tp_linear_bwd_wgrad_workspace_size */
  TP_ERR_HIP = -6,       /* a HIP launch failed; see tp_last_hip_error() */
  TP_ERR_SCRATCH = -7    /* tp_linear_bwd_wgrad_noalloc: the shape needs more than
                            TP_NOALLOC_SCRATCH_BYTES of scratch */
} tp_status;

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype;

typedef enum { TP_ACT_NONE = 0, TP_ACT_GELU_TANH = 1 } tp_act;

/* FP8 code formats (OCP 8-bit floats): E4M3 (largest finite 448), E5M2 (57344) */
typedef enum { TP_FP8_E4M3 = 0, TP_FP8_E5M2 = 1 } tp_fp8_format;

/*
 * Column-parallel forward of shard i ("Megatron" page, "Tensor Parallelism /
 * mathematical principles", the column split Y = [X A_1, .., X A_p]; applied to
 * MLP fc1 and to the QKV projection per "Transformer-layer tensor parallelism").
 *
 *   U_i = X A_i + bias_i          (T x n; bias broadcast over rows)
 *   Y_i = act(U_i)                (T x n)
 *
 * X      [T, h], ld_x, dtype dt        replicated input
 * A_i    [h, n], ld_a, dtype dt        column shard of the weight (may be a view
 *                                      of the unsharded [h, p*n] weight)
 * bias_i [n], dtype dt, or NULL        column shard of the bias
 * Y_i    [T, n], ld_y, dtype dt        output
 * U_i    [T, n], ld_y, dtype dt, or NULL   pre-activation, saved for the
 *                                      backward; required when act != NONE
 *                                      (with act == NONE it receives Y_i's values)
 */
int tp_column_linear_fwd(const void* X, const void* A_i, const void* bias_i, void* Y_i,
                         void* U_i, int64_t T, int64_t h, int64_t n, int64_t ld_x,
                         int64_t ld_a, int64_t ld_y, tp_dtype dt, tp_act act, hipStream_t stream);

/*
 * Row-parallel forward partial of shard i ("Megatron" page, "Tensor
 * Parallelism / mathematical principles", one term Y_i B_i of
 * Z = Y_1 B_1 + .. + Y_p B_p; MLP fc2 and the attention output projection).
 *
 *   Zp_i = Y_i B_i                (T x h, fp32, no bias: the bias is added once
 *                                  after the sum, in tp_reduce_partials)
 *
 * Y_i  [T, k], ld_y, dtype dt
 * B_i  [k, h], ld_b, dtype dt          row shard of the weight (may be a view of
 *                                      the unsharded [p*k, h] weight)
 * Zp_i [T, h], ld_z, fp32
 */
int tp_row_linear_fwd_partial(const void* Y_i, const void* B_i, float* Zp_i, int64_t T,
                              int64_t k, int64_t h, int64_t ld_y, int64_t ld_b,
                              int64_t ld_z, tp_dtype dt, hipStream_t stream);

/*
 * Input gradient (dgrad) of Out = act(In W) for a weight stored [k, n]
 * (derivative of the forward definitions above; not on the pages).
 *
 *   dIn = (dOut W^T) * act'(U)     elementwise with the saved pre-activation U
 *   dIn = dOut W^T                 when act == NONE (U ignored, may be NULL)
 *
 * Row-parallel layer: dOut = dZ, W = B_i, U = U_i, act = GELU -> dU_i (out_dt = dt).
 * Column-parallel layer: dOut = dU_i, W = A_i, act = NONE -> partial dX_i
 * (out_dt = TP_F32), summed over shards by tp_reduce_partials.
 *
 * dOut [T, n], ld_dout, dtype dt
 * W    [k, n], ld_w, dtype dt
 * U    [T, k], ld_u, dtype dt (required when act != NONE)
 * dIn  [T, k], ld_din, dtype out_dt (TP_F32, or dt)
 */
int tp_linear_bwd_dgrad(const void* dOut, const void* W, const void* U, tp_act act, void* dIn,
                        int64_t T, int64_t k, int64_t n, int64_t ld_dout, int64_t ld_w,
                        int64_t ld_u, int64_t ld_din, tp_dtype dt, tp_dtype out_dt,
                        hipStream_t stream);

/*
 * Row-parallel dgrad with activation recompute. The "Megatron" page
 * ("activation recomputation", under its training optimisations) trades
 * compute for memory: activations that the forward does not keep are computed
 * again in the backward. With this call a step keeps only the pre-activation
 * U_i from the forward; Y_i = GeLU(U_i), which the fc2 weight gradient needs,
 * is recomputed in the epilogue of the fc2 dgrad, which loads U_i anyway:
 *
 *   dU_i = (dZ B_i^T) * GeLU'(U_i)     exactly as tp_linear_bwd_dgrad
 *   Y    = GeLU(U_i)                   from the stored (rounded) U_i
 *
 * Y is then the In operand of tp_linear_bwd_wgrad for B_i. Compared with the
 * forward's Y_i it differs by the rounding of U_i to dt before the GeLU.
 *
 * dOut, W, U, dIn as tp_linear_bwd_dgrad with act = TP_ACT_GELU_TANH (other
 * values: TP_ERR_ACT) and out_dt = dt
 * Y    [T, k], ld_y, dtype dt; must not overlap U or dIn
 */
int tp_linear_bwd_dgrad_recompute(const void* dOut, const void* W, const void* U, tp_act act,
                                  void* dIn, void* Y, int64_t T, int64_t k, int64_t n,
                                  int64_t ld_dout, int64_t ld_w, int64_t ld_u, int64_t ld_din,
                                  int64_t ld_y, tp_dtype dt, hipStream_t stream);

/*
 * Weight and bias gradients (wgrad) of Out = In W + c for a weight stored
 * [k, n] (derivative of the forward definitions; not on the pages).
 *
 *   dW    (+)= In^T dOut           (k x n, fp32)
 *   dbias (+)= sum over the T rows of dOut   (n, fp32; skipped when NULL)
 *
 * With accumulate != 0 both are added to the values already in dW / dbias;
 * otherwise they are overwritten.
 *
 * In   [T, k], ld_in, dtype dt
 * dOut [T, n], ld_dout, dtype dt
 * dW   [k, n], ld_dw, fp32
 * workspace: device scratch of at least tp_linear_bwd_wgrad_workspace_size()
 *            bytes for the same (T, k, n, dt); may be NULL when that size is 0.
 *            Its contents on entry are ignored. One workspace must not be
 *            shared by calls that may run at the same time.
 */
int tp_linear_bwd_wgrad(const void* In, const void* dOut, float* dW, float* dbias, int64_t T,
                        int64_t k, int64_t n, int64_t ld_in, int64_t ld_dout, int64_t ld_dw,
                        int accumulate, tp_dtype dt, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/* Scratch bytes tp_linear_bwd_wgrad needs for (T, k, n, dt); pure host function. */
int tp_linear_bwd_wgrad_workspace_size(int64_t T, int64_t k, int64_t n, tp_dtype dt,
                                       size_t* bytes);

/* Bytes of the library's own device scratch array behind
 * tp_linear_bwd_wgrad_noalloc (one such array per GPU). */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * tp_linear_bwd_wgrad for callers that cannot allocate device memory: code
 * recorded under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, layouts, results and kernels as
 * tp_linear_bwd_wgrad, less the workspace: the split-K partials and the
 * column-sum partials live in a scratch array of TP_NOALLOC_SCRATCH_BYTES
 * that the library holds in static device memory on every GPU it is loaded
 * on, until the process ends. Nothing is allocated or freed by this call.
 *
 * The array used is the one of the current device (hipGetDevice); stream must
 * belong to that device. The first call on a device looks up that device's
 * address of the array once. No byte of the array needs to hold any value on
 * entry: every byte the kernels read was written earlier by the same call.
 *
 * Calls that may overlap on one GPU race on its array: serialise them (one
 * stream, or events). Returns TP_ERR_SCRATCH, launching nothing, when
 * tp_linear_bwd_wgrad_workspace_size(T, k, n, dt) exceeds
 * TP_NOALLOC_SCRATCH_BYTES, and the errors of tp_linear_bwd_wgrad otherwise.
 */
int tp_linear_bwd_wgrad_noalloc(const void* In, const void* dOut, float* dW, float* dbias,
                                int64_t T, int64_t k, int64_t n, int64_t ld_in, int64_t ld_dout,
                                int64_t ld_dw, int accumulate, tp_dtype dt, hipStream_t stream);

/*
 * The whole backward of one linear layer of the shard, the data gradient and
 * the weight gradient of the same forward product (derivatives of the
 * column- and row-parallel products of the "Megatron" page, "Tensor
 * Parallelism / mathematical principles"; the pages do not write the backward
 * out):
 *
 *   dIn   = (dOut W^T) [* act'(U)]    as tp_linear_bwd_dgrad
 *   dW    (+)= In^T dOut, dbias (+)= column sums of dOut
 *                                     as tp_linear_bwd_wgrad
 *
 * Same arguments, layouts and dtypes as those two calls made one after the
 * other. dIn is bitwise equal to tp_linear_bwd_dgrad's; dW and dbias equal
 * tp_linear_bwd_wgrad's to within fp32 summation order (the weight gradient's
 * tile and K slices may differ). For bf16 operands whose products both
 * fit one of the pipelined tiles 128x192, 128x128 or 256x192 (16-byte aligned
 * operands, row strides a multiple of 8, T a multiple of 64, k and n tile
 * multiples), both products run in one launch, the weight gradient's blocks
 * first, which saves one kernel's start and drain; otherwise the two calls
 * run. dIn and dW must not overlap any input. workspace: at least
 * tp_linear_bwd_workspace_size() bytes for the same (T, k, n, dt) (a smaller
 * one that still fits tp_linear_bwd_wgrad runs the two calls); contents on
 * entry ignored; not shared by calls that may run at the same time. Errors as
 * the two calls; every check of both runs before the first launch.
 */
int tp_linear_bwd(const void* dOut, const void* W, const void* U, tp_act act, const void* In,
                  void* dIn, float* dW, float* dbias, int64_t T, int64_t k, int64_t n,
                  int64_t ld_dout, int64_t ld_w, int64_t ld_u, int64_t ld_in, int64_t ld_din,
                  int64_t ld_dw, int accumulate, tp_dtype dt, tp_dtype out_dt, void* workspace,
                  size_t workspace_bytes, hipStream_t stream);

/* Scratch bytes tp_linear_bwd needs for (T, k, n, dt); pure host function. */
int tp_linear_bwd_workspace_size(int64_t T, int64_t k, int64_t n, tp_dtype dt, size_t* bytes);

/*
 * How tp_linear_bwd runs a bf16 layer of this shape (pure host function, for
 * tuning, tests and measurement). Writes the pairing: 0 (no paired kernel
 * fits: the two calls run), 1 (one launch, both products on 128x128 tiles),
 * 2 (one launch, weight gradient on 128x128 and data gradient on 128x192
 * tiles), 3 (one launch, both on 256x192 tiles); and the weight gradient's
 * number of K slices in that launch (1 when pairing is 0). A paired call is
 * one kernel launch unless splitk > 1 (a fix-up launch sums the slices) or
 * dbias is requested over more than one row block (a second pass sums the
 * column partials). Shape only: the call pairs when its operands also meet
 * the alignment stated for tp_linear_bwd. Returns TP_ERR_SHAPE for a
 * dimension < 1; either output pointer may be NULL.
 */
int tp_linear_bwd_plan(int64_t T, int64_t k, int64_t n, int* pairing, int* splitk);

/*
 * The backward of one shard's MLP block ("Megatron" page, "Tensor
 * Parallelism / mathematical principles": the column-parallel fc1 with GeLU,
 * then the row-parallel fc2; derivatives not on the pages), without the sum
 * of the dX partials over shards (tp_reduce_partials):
 *
 *   fc2: dU_i = (dZ B_i^T) * GeLU'(U_i); dB_i (+)= Y_i^T dZ; db (+)= colsum(dZ)
 *   fc1: dXp_i = dU_i A_i^T (fp32 partial); dA_i (+)= X^T dU_i;
 *        da_i (+)= colsum(dU_i)
 *
 * Same results as tp_linear_bwd for fc2 (act GeLU, out dtype dt) followed by
 * tp_linear_bwd for fc1 (act none, out TP_F32): dU_i and dXp_i bitwise, the
 * weight and bias gradients to within fp32 summation order (da_i is summed
 * per data-gradient tile of 128 or 256 rows, then over the tiles in order). Where both layers pair (see
 * tp_linear_bwd) it makes two launches (plus fc1's own fix-up if fc1's
 * weight gradient splits K): fc2's data-gradient epilogue also writes the
 * column partial sums of dU_i, and fc2's split-K fix-up, the last pass of db
 * and of da_i run in spare blocks of fc1's paired launch, on the CUs fc1's
 * data gradient leaves while its weight gradient still runs; otherwise the
 * two tp_linear_bwd calls run.
 *
 * dZ [T,h], X [T,h], A_i [h,F] (ld_a), B_i [F,h] (ld_b), U_i and Y_i [T,F]:
 * dtype dt. dU_i [T,F] dtype dt (written, then read by fc1). dB_i [F,h]
 * (ld_db), dA_i [h,F] (ld_da), dXp_i [T,h] (ld_dxp), db [h], da_i [F]: fp32;
 * db and da_i nullable. No output may overlap an input or another output.
 * workspace: at least tp_mlp_bwd_workspace_size() bytes; contents on entry
 * ignored; not shared by calls that may run at the same time. Errors as
 * tp_linear_bwd; every check of both layers runs before the first launch.
 */
int tp_mlp_bwd(const void* dZ, const void* X, const void* A_i, const void* B_i, const void* U_i,
               const void* Y_i, void* dU_i, float* dB_i, float* db, float* dXp_i, float* dA_i,
               float* da_i, int64_t T, int64_t h, int64_t F, int64_t ld_dz, int64_t ld_x,
               int64_t ld_a, int64_t ld_b, int64_t ld_u, int64_t ld_y, int64_t ld_du,
               int64_t ld_dxp, int64_t ld_db, int64_t ld_da, int accumulate, tp_dtype dt,
               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Scratch bytes tp_mlp_bwd needs for (T, h, F, dt); pure host function. */
int tp_mlp_bwd_workspace_size(int64_t T, int64_t h, int64_t F, tp_dtype dt, size_t* bytes);

/*
 * The whole MLP step of all p shards of a layer on this device: every
 * shard's column-parallel fc1 (bias + GeLU) and row-parallel fc2 partial, the
 * sum Z = Y_1 B_1 + .. + Y_p B_p + b that stands in for the All-Reduce
 * ("Megatron" page, "Tensor Parallelism / mathematical principles"), then every
 * shard's backward (as tp_mlp_bwd) and the sum of the dX partials. The
 * results are those of the per-product calls above, shard by shard.
 *
 * Layouts (bf16 = dt, fp32 as noted; shard i is a column or row block):
 *   X   [T, h], ld_x            A  [h, p*F], ld_a (A_i: columns i*F ..)
 *   a   [p*F] or NULL           B  [p*F, h], ld_b (B_i: rows i*F ..)
 *   b   [h] or NULL             dZ [T, h], ld_dz
 *   U, Y, dU  [T, p*F], ld_u    (U_i, Y_i, dU_i: columns i*F ..)
 *   Zp, dXp   fp32 [p, T, h]    compact (shard i at i*T*h, row stride h)
 *   Z, dX     [T, h], ld_z / ld_dx
 *   dB  fp32 [p*F, h], ld_db (dB_i: rows i*F ..)   db fp32 [h] or NULL
 *   dA  fp32 [h, p*F], ld_da (dA_i: columns i*F ..) da fp32 [p*F] or NULL
 * Weight and bias gradients are overwritten. db = column sums of dZ and
 * da_i = column sums of dU_i are computed only where their pointer is set.
 *
 * bf16, with the shapes tp_mlp_step_plan reports as fused (T a multiple of
 * 128 x the device's XCD count, h and F of 128, 16-byte aligned operands and
 * row strides), runs the forward, both sums and the data gradients in one
 * persistent launch over each XCD's own token rows, then the weight and bias
 * gradients of all shards as two products over the stacked shards
 * (dB = Y^T dZ, dA = X^T dU, as tp_linear_bwd_wgrad). Any other shape or
 * dtype runs the same step as the per-product calls.
 *
 * workspace: at least tp_mlp_step_workspace_size bytes, 256-byte aligned,
 * ZEROED BEFORE ITS FIRST USE (it holds the queue's counters, which every
 * call leaves zeroed again, ahead of the weight gradients' scratch). It belongs to tp_mlp_step calls alone: no other
 * call may use it as scratch between them (that would leave the counters
 * nonzero), and tp_mlp_step calls that share it must not overlap (enqueue them
 * on one stream). Its first 32-bit word is nonzero after a call
 * in which a dependency wait gave up (tp_set_wait_limit); that call's results
 * are then invalid, and the word stays set until the caller clears it.
 * Bytes 64..95 hold four 64-bit counters of the persistent launch's block 0:
 * the shader clock and the 100 MHz real-time clock at its start, then at its
 * end.
 */
int tp_mlp_step(const void* X, const void* A, const void* a, const void* B, const void* b,
                const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                float* db, float* dA, float* da, float* dXp, void* dX, int64_t T, int64_t h,
                int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b, int64_t ld_dz,
                int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db, int64_t ld_da,
                tp_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The two halves of tp_mlp_step, same arguments: tp_mlp_step_rows computes
 * the forward, both sums and the data gradients (U, Y, Zp, Z, dU, dXp, dX;
 * the persistent launch), tp_mlp_step_wgrad the weight and bias gradients
 * (dB, db, dA, da; the two products) from the Y and dU the first left.
 * Calling rows then wgrad on one stream is tp_mlp_step.
 */
int tp_mlp_step_rows(const void* X, const void* A, const void* a, const void* B, const void* b,
                     const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                     float* db, float* dA, float* da, float* dXp, void* dX, int64_t T,
                     int64_t h, int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b,
                     int64_t ld_dz, int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db,
                     int64_t ld_da, tp_dtype dt, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);
int tp_mlp_step_wgrad(const void* X, const void* A, const void* a, const void* B, const void* b,
                      const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                      float* db, float* dA, float* da, float* dXp, void* dX, int64_t T,
                      int64_t h, int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b,
                      int64_t ld_dz, int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db,
                      int64_t ld_da, tp_dtype dt, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * The forward and the backward of tp_mlp_step as two calls, same arguments,
 * for a caller that runs other layers between them (the "Megatron" page,
 * "Tensor Parallelism / mathematical principles", for the step; its training
 * optimisations, activation recomputation, for `recompute`).
 * tp_mlp_step_fwd computes U, Y, Zp and Z (the forward units of the
 * persistent launch); tp_mlp_step_bwd computes dU, dXp, dX and the weight and
 * bias gradients from the saved X, U, dZ and the weights (the backward units,
 * then the two products). With recompute = 0 tp_mlp_step_bwd reads the Y the
 * forward left; with recompute nonzero Y is only transient between the calls
 * (its memory may be reused) and tp_mlp_step_bwd rebuilds Y_i = GeLU(U_i)
 * from the saved bf16 U_i in fc2's data-gradient epilogue (as
 * tp_linear_bwd_dgrad_recompute) before dB reads it. Forward then backward
 * with recompute = 0 on one stream give tp_mlp_step's results bit for bit.
 * The workspace rules are tp_mlp_step's (both calls share one workspace).
 */
int tp_mlp_step_fwd(const void* X, const void* A, const void* a, const void* B, const void* b,
                    const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                    float* db, float* dA, float* da, float* dXp, void* dX, int64_t T, int64_t h,
                    int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b, int64_t ld_dz,
                    int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db, int64_t ld_da,
                    tp_dtype dt, void* workspace, size_t workspace_bytes, hipStream_t stream);
int tp_mlp_step_bwd(const void* X, const void* A, const void* a, const void* B, const void* b,
                    const void* dZ, void* U, void* Y, float* Zp, void* Z, void* dU, float* dB,
                    float* db, float* dA, float* da, float* dXp, void* dX, int64_t T, int64_t h,
                    int64_t F, int p, int64_t ld_x, int64_t ld_a, int64_t ld_b, int64_t ld_dz,
                    int64_t ld_u, int64_t ld_z, int64_t ld_dx, int64_t ld_db, int64_t ld_da,
                    int recompute, tp_dtype dt, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * The attention projections of all p shards of a layer on this device
 * ("Megatron" page, "Transformer-layer tensor parallelism": the QKV
 * projection is column-parallel and the output projection row-parallel, the
 * sum over shards standing in for the All-Reduce; the backward is the
 * derivative of the same definitions):
 *   QKV_i = X W_i                      (stage 1)
 *   Zpa_i = C_i O_i, Za = sum_i Zpa_i   (stage 2)
 *   dC_i  = dZa O_i^T                  (stage 4)
 *   dXqp_i = dQKV_i W_i^T, dXq = sum_i dXqp_i   (stage 8)
 *   dO_i = C_i^T dZa, dW_i = X^T dQKV_i (stage 16, fp32, overwritten)
 * `stages` is any nonempty sum of those bits; the stages run in that order.
 * C_i and dQKV_i are inputs: the attention core's output and input gradient
 * (tp_attention_fwd / tp_attention_bwd), so a caller with the core runs stage
 * 1, the core, stage 2; then stage 4, the core's backward, stages 8 + 16.
 * Without it all five stages are one call.
 *
 * Layouts (bf16 = dt, fp32 as noted; shard i is a column or row block):
 *   X [T, h], ld_x            W [h, p*Q], ld_w (W_i: columns i*Q ..)
 *   Ow [p*O, h], ld_ow (O_i: rows i*O ..)
 *   C [T, p*O], ld_c          dZa [T, h], ld_dz      dQKV [T, p*Q], ld_dqkv
 *   QKV [T, p*Q], ld_qkv      dC [T, p*O], ld_dc
 *   Zpa, dXqp fp32 [p, T, h] compact (shard i at i*T*h, row stride h)
 *   Za [T, h], ld_za          dXq [T, h], ld_dxq
 *   dOw fp32 [p*O, h], ld_dow (dO_i: rows i*O ..)
 *   dW  fp32 [h, p*Q], ld_dw  (dW_i: columns i*Q ..)
 * Pointers a stage does not touch may be NULL.
 *
 * bf16 with the shapes tp_attn_proj_step_plan reports as fused (T a multiple
 * of 128 x the device's XCD count; h, Q, O of 128; 16-byte aligned operands
 * and row strides) runs stages 1, 2, 4 and 8 in one persistent launch over
 * each XCD's own token rows (the MLP step's queue, with no dependency between
 * the products and the sums waiting for every shard's partials), and stage 16
 * as two products over the stacked shards (as tp_mlp_step's weight
 * gradients). Any other shape or dtype runs the same stages as the
 * per-product calls. The results are those of the per-product calls.
 *
 * workspace: at least tp_attn_proj_step_workspace_size bytes, 256-byte
 * aligned, zeroed before its first use, with the same rules as tp_mlp_step's
 * (its counters are left zeroed by every call; calls sharing it do not
 * overlap; its first 32-bit word is nonzero after a call in which a sum's
 * wait gave up).
 */
int tp_attn_proj_step(const void* X, const void* W, const void* Ow, const void* C,
                      const void* dZa, const void* dQKV, void* QKV, float* Zpa, void* Za,
                      void* dC, float* dOw, float* dW, float* dXqp, void* dXq, int64_t T,
                      int64_t h, int64_t Q, int64_t O, int p, int64_t ld_x, int64_t ld_w,
                      int64_t ld_ow, int64_t ld_c, int64_t ld_dz, int64_t ld_dqkv, int64_t ld_qkv,
                      int64_t ld_dc, int64_t ld_za, int64_t ld_dxq, int64_t ld_dow, int64_t ld_dw,
                      int stages, tp_dtype dt, void* workspace, size_t workspace_bytes,
                      hipStream_t stream);
/* Workspace bytes of tp_attn_proj_step (pure host function). */
int tp_attn_proj_step_workspace_size(int64_t T, int64_t h, int64_t Q, int64_t O, int p,
                                     tp_dtype dt, size_t* bytes);
/* *fused = 1 where tp_attn_proj_step runs the persistent launch for these
 * shapes (alignment aside), else 0. */
int tp_attn_proj_step_plan(int64_t T, int64_t h, int64_t Q, int64_t O, int p, tp_dtype dt,
                           int* fused);

/* Workspace bytes of tp_mlp_step for these shapes (the larger of the fused
 * path's and the per-product path's needs); pure host function. */
int tp_mlp_step_workspace_size(int64_t T, int64_t h, int64_t F, int p, tp_dtype dt,
                               size_t* bytes);

/* Whether tp_mlp_step runs these shapes in the persistent launch and the two
 * stacked weight-gradient products (*fused = 1, given aligned operands) or as
 * per-product calls (0). */
int tp_mlp_step_plan(int64_t T, int64_t h, int64_t F, int p, tp_dtype dt, int* fused);

/*
 * Test hook: the number of polls after which a dependency wait of
 * tp_mlp_step's persistent launch gives up (setting the workspace's error
 * word), for calls made by the calling thread. 0 restores the default (about
 * a quarter of a second); a negative value gives up at the first check that
 * finds the dependency unmet. Every block still runs to its end.
 */
int tp_set_wait_limit(int64_t polls);

/*
 * Sum over shards, the one-GPU stand-in for the All-Reduce ("Megatron" page,
 * "Tensor Parallelism / mathematical principles": the row-split partials Y_i B_i
 * are summed across GPUs; "Transformer-layer tensor parallelism": one such sum
 * after the attention output projection and one after the MLP).
 *
 *   out = partials[0] + partials[1] + .. + partials[p-1] + bias
 *
 * summed in fp32 in the order i = 0 .. p-1, the bias (if any) added last, then
 * rounded once to out_dt. Also used for the backward sum of the partial dX_i.
 *
 * partials  HOST array of p DEVICE pointers, each [T, h] fp32 with row stride ld_p
 * p         1 .. 16
 * bias      [h], dtype out_dt, or NULL
 * out       [T, h], ld_out, dtype out_dt; may alias partials[0] when
 *           out_dt == TP_F32 and ld_out == ld_p
 */
int tp_reduce_partials(const float* const* partials, int p, const void* bias, void* out,
                       int64_t T, int64_t h, int64_t ld_p, int64_t ld_out, tp_dtype out_dt,
                       hipStream_t stream);

/*
 * Standalone bias + activation pass: Y = act(U + bias), elementwise.
 * The fused epilogue of tp_column_linear_fwd does the same work inside the
 * GEMM. On its own the pass is HBM-bound. With bias NULL it rebuilds
 * Y = GeLU(U) from a stored U for activation recompute.
 *
 * U    [T, n], ld_u, dtype in_dt
 * bias [n], dtype in_dt, or NULL
 * Y    [T, n], ld_y, dtype out_dt
 * act  TP_ACT_GELU_TANH or TP_ACT_NONE (then Y = U + bias)
 */
int tp_bias_act(const void* U, const void* bias, void* Y, int64_t T, int64_t n, int64_t ld_u,
                int64_t ld_y, tp_dtype in_dt, tp_dtype out_dt, tp_act act, hipStream_t stream);

/*
 * Attention core of one shard, forward. The "Megatron" page ("Transformer-
 * layer tensor parallelism") splits the QKV projection by output columns, so a
 * shard holds whole heads and attends with them alone, between its QKV
 * projection and its row-split output projection; the page's optimisation
 * list recommends a fused attention kernel. For each of `batch` sequences of
 * `seq` tokens (tokens sequence-major) and each of the shard's `heads` heads:
 *
 *   C   = softmax(Q K^T / sqrt(head_dim) [causal: position q sees keys <= q]) V
 *   lse = log of each query's softmax normaliser (natural log)
 *
 * QKV   [batch*seq, 3*heads*head_dim] bf16, row stride ld_qkv: the Q, K and V
 *       thirds, each head-major (head j at columns j*head_dim .. of its third)
 * C     [batch*seq, heads*head_dim] bf16, row stride ld_c, head-major
 * lse   [batch, heads, seq] fp32, or NULL
 * causal  nonzero: mask keys after the query (a GPT decoder)
 *
 * bf16 only (TP_ERR_DTYPE). head_dim must be 64, QKV 16-byte aligned with
 * ld_qkv a multiple of 8, and C 8-byte aligned with ld_c a multiple of 4
 * (TP_ERR_SHAPE otherwise).
 */
int tp_attention_fwd(const void* QKV, void* C, float* lse, int64_t batch, int64_t seq,
                     int64_t heads, int64_t head_dim, int64_t ld_qkv, int64_t ld_c, int causal,
                     tp_dtype dt, hipStream_t stream);

/*
 * Attention core of one shard, backward: the gradient of the forward above
 * with respect to QKV, given the gradient dC of its output (in a shard this is
 * the dgrad of the row-split output projection). With P the softmax weights,
 * recomputed from Q, K and lse:
 *
 *   delta[q] = sum_d dC[q,d] C[q,d]
 *   dV = P^T dC,  dS = P * (dC V^T - delta),  dQ = dS K / sqrt(head_dim),
 *   dK = dS^T Q / sqrt(head_dim)
 *
 * QKV, C, lse, causal  exactly as passed to / written by tp_attention_fwd
 * dC    [batch*seq, heads*head_dim] bf16, row stride ld_dc
 * delta [batch, heads, seq] fp32 workspace owned by the caller, overwritten
 * dQKV  [batch*seq, 3*heads*head_dim] bf16, row stride ld_dqkv, laid out like
 *       QKV; columns 0 .. 3*heads*head_dim of every row are written. It must
 *       not overlap any input.
 *
 * Each output element is computed by one thread in a fixed order (no atomics):
 * results are bitwise reproducible. bf16 only (TP_ERR_DTYPE); lse and delta
 * must not be NULL (TP_ERR_NULL). head_dim must be 64, QKV, C and dC 16-byte
 * aligned with row strides a multiple of 8, dQKV 8-byte aligned with ld_dqkv a
 * multiple of 4 (TP_ERR_SHAPE otherwise).
 */
int tp_attention_bwd(const void* QKV, const void* C, const void* dC, const float* lse,
                     float* delta, void* dQKV, int64_t batch, int64_t seq, int64_t heads,
                     int64_t head_dim, int64_t ld_qkv, int64_t ld_c, int64_t ld_dc,
                     int64_t ld_dqkv, int causal, tp_dtype dt, hipStream_t stream);

/*
 * The attention core of `shards` shards in one launch, forward and backward:
 * every shard as tp_attention_fwd / tp_attention_bwd with `heads` heads, the
 * shards side by side in the layouts tp_attn_proj_step stacks them in:
 *   QKV, dQKV [batch*seq, shards*3*heads*head_dim]: shard s's [Q | K | V]
 *             block is columns s*3*heads*head_dim ..
 *   C, dC     [batch*seq, shards*heads*head_dim]: shard s's heads are
 *             columns s*heads*head_dim ..
 *   lse, delta [batch, shards*heads, seq] fp32
 * The results equal the per-shard calls bit for bit (each shard's heads run
 * the same kernels in the same order); one launch fills the device where one
 * shard's heads would not. Arguments and errors as the single-shard calls,
 * with shards in 1 .. 16 (TP_ERR_SHAPE otherwise).
 */
int tp_attention_fwd_shards(const void* QKV, void* C, float* lse, int64_t batch, int64_t seq,
                            int64_t heads, int64_t shards, int64_t head_dim, int64_t ld_qkv,
                            int64_t ld_c, int causal, tp_dtype dt, hipStream_t stream);
int tp_attention_bwd_shards(const void* QKV, const void* C, const void* dC, const float* lse,
                            float* delta, void* dQKV, int64_t batch, int64_t seq, int64_t heads,
                            int64_t shards, int64_t head_dim, int64_t ld_qkv, int64_t ld_c,
                            int64_t ld_dc, int64_t ld_dqkv, int causal, tp_dtype dt,
                            hipStream_t stream);

/*
 * FP8 variant of the shard GEMMs. The "Megatron" page ("mixed-precision
 * training") trains in FP8 besides FP16/BF16, and the "Megatron-LM
 * quick-start" page ("performance optimisation") recommends it; neither fixes
 * the format or the scaling. Here: OCP E4M3 for weights and activations,
 * E4M3 or E5M2 for gradients, each tensor with its own current scale
 * s = fmax / amax(tensor). The GEMMs run on gfx950's FP8 matrix cores
 * (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulation) and multiply the
 * accumulators by the two 1/s factors before their epilogue. Both operands of
 * every FP8 product are K-contiguous codes, so the quantiser writes X or X^T
 * as each product needs it.
 *
 * Shapes: every M, N and K of an FP8 product must be a multiple of 128, the
 * code operands 16-byte aligned with row strides (ld, in codes = bytes) a
 * multiple of 16 (TP_ERR_SHAPE otherwise). Scale factors are device fp32
 * scalars written by tp_fp8_quantize.
 */

/* Bytes of workspace tp_fp8_quantize needs (per-block maxima; 4 KiB). */
int tp_fp8_quantize_workspace_size(int64_t rows, int64_t cols, size_t* bytes);

/*
 * Per-tensor current scaling of X [rows, cols] (ld_x, dtype dt):
 *   s = fmax / max|X| in fp32 (1 when X is all zeros),
 *   code = nearest value of `fmt`, ties to even, of clamp(x * s, -fmax, fmax),
 *   scale_inv[0] = 1 / s (device fp32 scalar, for the GEMMs).
 * Q receives the codes of X ([rows, cols], ld_q >= cols) or, with transpose,
 * of X^T ([cols, rows], ld_q >= rows). The maximum is order-independent, so
 * the result is reproducible. X must hold finite values. Two launches.
 */
int tp_fp8_quantize(const void* X, int64_t rows, int64_t cols, int64_t ld_x, tp_dtype dt, tp_fp8_format fmt,
                    int transpose, void* Q, int64_t ld_q, float* scale_inv, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/*
 * Both layouts at once: the codes of X into Q ([rows, cols], ld_q >= cols) and
 * of X^T into Qt ([cols, rows], ld_qt >= rows), with one scale, from one read
 * of X (two launches in all). The codes equal those of two tp_fp8_quantize
 * calls.
 */
int tp_fp8_quantize_both(const void* X, int64_t rows, int64_t cols, int64_t ld_x, tp_dtype dt,
                         tp_fp8_format fmt, void* Q, int64_t ld_q, void* Qt, int64_t ld_qt,
                         float* scale_inv, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * tp_fp8_quantize_both for n tensors (1 <= n <= 6) in two launches in all
 * instead of 2n: one for every tensor's per-block maxima, one for every
 * tensor's codes. Tensor i has its own scale and takes its arguments from
 * entry i of each array. The arrays are HOST arrays of n entries; the pointers
 * they hold are DEVICE pointers. Codes and scales are bitwise equal to n
 * tp_fp8_quantize_both calls. No output may overlap another tensor's input or
 * output. workspace: at least tp_fp8_quantize_multi_workspace_size(n) bytes
 * (tensor i's maxima in its i-th slice), 4-byte aligned, contents on entry
 * ignored. Every tensor is checked as tp_fp8_quantize_both checks it before
 * the first launch, and the first failing check's status is returned.
 * TP_ERR_SHAPE for n outside 1..6.
 */
int tp_fp8_quantize_both_multi(int n, const void* const* X, const int64_t* rows,
                               const int64_t* cols, const int64_t* ld_x, const int* dt,
                               const int* fmt, void* const* Q, const int64_t* ld_q,
                               void* const* Qt, const int64_t* ld_qt, float* const* scale_inv,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace tp_fp8_quantize_both_multi needs for n tensors (n * 4 KiB). */
int tp_fp8_quantize_multi_workspace_size(int n, size_t* bytes);

/*
 * FP8 column-parallel forward: Y_i = act(X A_i + a_i) with U_i saved, as
 * tp_column_linear_fwd, from Xq = codes of X [T, h] (E4M3) and Atq = codes of
 * A_i^T [n, h] (E4M3, quantised with transpose). Y_i, U_i and bias_i bf16.
 * act TP_ACT_NONE requires bias_i and U_i NULL (a plain bf16 store).
 */
int tp_fp8_column_linear_fwd(const void* Xq, const void* Atq, const float* x_scale_inv,
                             const float* a_scale_inv, const void* bias_i, void* Y_i, void* U_i,
                             int64_t T, int64_t h, int64_t n, int64_t ld_x, int64_t ld_at,
                             int64_t ld_y, tp_act act, hipStream_t stream);

/*
 * tp_fp8_column_linear_fwd with act TP_ACT_GELU_TANH that also leaves the
 * maxima of |Y_i| the quantisation of Y_i needs ("Megatron" page, mixed-precision
 * training: FP8 with per-tensor current scaling): each wave of the epilogue
 * stores the largest |stored bf16 value| of its part of an output tile into
 * one float of y_amax, tp_fp8_amax_slots(T, n, h) of them in all (every slot is
 * written; nothing needs clearing). tp_fp8_quantize_both_from_amax then
 * quantises Y_i in one launch with the same codes and scale as
 * tp_fp8_quantize_both. TP_ERR_SHAPE where no FP8 tile fits the shape.
 */
int tp_fp8_column_linear_fwd_amax(const void* Xq, const void* Atq, const float* x_scale_inv,
                                  const float* a_scale_inv, const void* bias_i, void* Y_i,
                                  void* U_i, int64_t T, int64_t h, int64_t n, int64_t ld_x,
                                  int64_t ld_at, int64_t ld_y, float* y_amax,
                                  hipStream_t stream);

/*
 * Slots of the maxima the _amax products write for an M x N output of
 * K-long products (one per wave of each output tile of the planned FP8 tile);
 * pure host function. TP_ERR_SHAPE where no FP8 tile fits.
 */
int tp_fp8_amax_slots(int64_t M, int64_t N, int64_t K, int64_t* slots);

/*
 * tp_fp8_quantize_both with the maxima of |X| already given (the amax slots
 * of the product that wrote X, n_amax of them): the codes of X and X^T and
 * 1/s in one launch, equal to tp_fp8_quantize_both's when the slots cover X.
 */
int tp_fp8_quantize_both_from_amax(const void* X, int64_t rows, int64_t cols, int64_t ld_x,
                                   tp_dtype dt, tp_fp8_format fmt, void* Q, int64_t ld_q, void* Qt,
                                   int64_t ld_qt, float* scale_inv, const float* amax,
                                   int64_t n_amax, hipStream_t stream);

/*
 * FP8 row-parallel forward partial: Zp_i = Y_i B_i (fp32 [T, h]) from
 * Yq = codes of Y_i [T, k] (E4M3) and Btq = codes of B_i^T [h, k] (E4M3).
 */
int tp_fp8_row_linear_fwd_partial(const void* Yq, const void* Btq, const float* y_scale_inv,
                                  const float* b_scale_inv, float* Zp_i, int64_t T, int64_t k,
                                  int64_t h, int64_t ld_y, int64_t ld_bt, int64_t ld_z,
                                  hipStream_t stream);

/*
 * FP8 dgrad: dIn = (dOut W^T) [* act'(U)] as tp_linear_bwd_dgrad, from
 * dOutq = codes of dOut [T, n] (dout_fmt) and Wq = codes of the weight as
 * stored, [k, n] (E4M3). act TP_ACT_GELU_TANH needs U (bf16 [T, k]) and
 * out_dt TP_BF16; act NONE writes dIn in out_dt (TP_F32 for a dX partial).
 */
int tp_fp8_linear_bwd_dgrad(const void* dOutq, const void* Wq, const float* dout_scale_inv,
                            const float* w_scale_inv, tp_fp8_format dout_fmt, const void* U, tp_act act,
                            void* dIn, int64_t T, int64_t k, int64_t n, int64_t ld_dout,
                            int64_t ld_w, int64_t ld_u, int64_t ld_din, tp_dtype out_dt,
                            hipStream_t stream);

/*
 * tp_fp8_linear_bwd_dgrad with act TP_ACT_GELU_TANH and a bf16 dIn, that also
 * leaves the maxima of |dIn| in din_amax (tp_fp8_amax_slots(T, k, n) floats),
 * as tp_fp8_column_linear_fwd_amax does for Y_i.
 */
int tp_fp8_linear_bwd_dgrad_amax(const void* dOutq, const void* Wq, const float* dout_scale_inv,
                                 const float* w_scale_inv, tp_fp8_format dout_fmt, const void* U,
                                 void* dIn, int64_t T, int64_t k, int64_t n, int64_t ld_dout,
                                 int64_t ld_w, int64_t ld_u, int64_t ld_din, float* din_amax,
                                 hipStream_t stream);

/* Workspace bytes of tp_fp8_linear_bwd_wgrad (split-K partials and bias sums). */
int tp_fp8_linear_bwd_wgrad_workspace_size(int64_t T, int64_t k, int64_t n, size_t* bytes);

/*
 * FP8 wgrad: dW = In^T dOut (fp32 [k, n], overwritten) from Intq = codes of
 * In^T [k, T] (E4M3) and dOuttq = codes of dOut^T [n, T] (dout_fmt), both
 * quantised with transpose. K = T may be split, with partials in the
 * workspace and a fixed-order fix-up. With dbias non-NULL, dbias = column sums
 * of the unquantised dOut (bf16 [T, n], ld_dout), as tp_linear_bwd_wgrad.
 */
int tp_fp8_linear_bwd_wgrad(const void* Intq, const void* dOuttq, const float* in_scale_inv,
                            const float* dout_scale_inv, tp_fp8_format dout_fmt, float* dW,
                            const void* dOut, float* dbias, int64_t T, int64_t k, int64_t n,
                            int64_t ld_int, int64_t ld_doutt, int64_t ld_dw, int64_t ld_dout,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Which GEMM kernel configuration the library uses for a bf16 product
 * C[M,N] = op(A)[M,K] op(B)[K,N] of this shape (pure host function, for
 * tuning and tests). allow_split != 0 for the weight-gradient products, which
 * may split K. Writes the tile id (0: general kernel, any shape; 10: 256x256,
 * 11: 256x128, 12: 128x256, 13: 128x128, 14: 256x192, 15: 128x192 pipelined
 * kernels, used when M and N are multiples of the tile, K of 64 and both
 * operands are 16-byte aligned with row strides a multiple of 8), the number
 * of K slices, and the K extent of each slice. Any output pointer may be NULL.
 */
int tp_gemm_plan(int64_t M, int64_t N, int64_t K, int allow_split, int* tile, int* splitk,
                 int64_t* k_chunk);

/*
 * Tuning and test hook: every later bf16 product whose shape the pipelined
 * tile `tile` (10..15, as for tp_gemm_plan) supports uses that tile, and a
 * weight-gradient product (the only kind that may split K) uses `splitk` K
 * slices when K is a multiple of 64 * splitk. tile = 0 restores the library's
 * own choice. The override belongs to the calling thread: it changes the plans
 * (and so the workspace queries) of calls made by that thread only, and other
 * threads keep the library's choice. Returns TP_ERR_SHAPE for an unknown tile
 * id or a splitk outside 1..16.
 */
int tp_set_gemm_override(int tile, int splitk);

/* Human-readable name of a tp_status value (never NULL). */
const char* tp_status_string(int status);

/* hipError_t of the last TP_ERR_HIP returned on the calling thread (0 if none). */
int tp_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TP_MLP_H */
