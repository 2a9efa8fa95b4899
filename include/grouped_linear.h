/*
 * grouped_linear.h -- C ABI of the MI355X (gfx950) grouped-linear library.
 *
 * The method (page "transformer_engine/pytorch/ops/basic/grouped_linear.py",
 * GroupedLinear class docstring): a token matrix x [T, K] is split along its rows
 * into num_groups consecutive blocks of m_splits[g] rows (zeros allowed), and
 * block g goes through its own linear layer, y_g = x_g W_g^T + b_g -- the same as
 * torch.split, one torch.nn.Linear per split, torch.cat.  The backward pass
 * (same page, fuser_backward) is dgrad dx_g = dy_g W_g, wgrad dW_g = dy_g^T x_g
 * (optionally added into an fp32 main_grad) and bias grad db_g = column sums of
 * dy_g.
 *
 * Notation: G = num_groups, K = in_features, N = out_features, T = total_rows =
 * sum of m_splits.  All matrices are dense row-major: x [T,K], y/dy [T,N],
 * dx [T,K], W [G,N,K] (or G separate [N,K]), b/db [G,N] (or G separate [N]),
 * dW/main_grad [G,N,K] (or G separate [N,K]).
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument is a DEVICE pointer owned by the caller, except the
 *    stream and the deferred-wgrad queue handle.  The library allocates no device
 *    memory, keeps no pointer after return (except the records of a deferred-wgrad
 *    queue, until they run) and never synchronises the host (gl_read_status is the
 *    one exception).  Work is enqueued on `stream` in call order.
 *  - Weights (and biases, wgrad outputs) come in one of two forms: a stacked
 *    buffer (`w`) or a DEVICE array of G per-group pointers (`w_ptrs`); exactly one
 *    of the two must be non-NULL (page "Improve device-init grouped linear module
 *    with single grouped weight support": single stacked weight or discrete
 *    per-group weights).  For biases both NULL means "no bias".
 *  - Buffers must be 16-byte aligned, and for bf16 K and N must be multiples of 8
 *    so every row starts on a 16-byte boundary, and at most 2^22 (GL_ERR_SHAPE
 *    otherwise; the MXFP8 forward and dgrad take the same 2^22 bound).
 *  - Output buffers may have more rows than T (`y_rows`, `dx_rows` >= T).  Kernels
 *    store into rows [0, T) alone; every row from T to the end of the buffer keeps
 *    whatever it held before the call (page "[PyTorch] Add optional caller-provided
 *    output/grad-input buffers to GroupedLinear and fused grouped MLP", Changes).
 *  - Return value: GL_OK (0) or a negative GL_ERR_* code.  On any host-detected
 *    error nothing is launched and nothing is written; gl_last_error() gives a
 *    message (thread-local).
 *  - Split sizes live on the device.  gl_offsets validates them there: a negative
 *    size or a sum different from total_rows sets the status word in the
 *    workspace, and every later kernel that reads that workspace then exits
 *    without writing anything.  gl_read_status() reports the word.
 */
#ifndef GROUPED_LINEAR_H
#define GROUPED_LINEAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  GL_F16 goes wherever GL_BF16 does except the MXFP8 quantizers
 * (whose source is bf16, as on the pages).  The enum is int-sized, and any int a
 * caller passes is a value of it (GL_DTYPE_INT_RANGE_ widens its range to all of
 * int), so an unknown code is rejected with GL_ERR_DTYPE rather than being
 * undefined behaviour in C++. */
typedef enum gl_dtype {
  GL_F32 = 0,
  GL_BF16 = 1,
  GL_F16 = 2,
  GL_E4M3 = 3,
  GL_DTYPE_INT_RANGE_ = 0x7fffffff
} gl_dtype;

enum {
  GL_OK = 0,
  GL_ERR_ARG = -1,         /* bad size, NULL or misaligned pointer, both/neither weight forms */
  GL_ERR_DTYPE = -2,       /* element type not valid for this call */
  GL_ERR_SHAPE = -3,       /* output capacity < total_rows, K/N alignment, K % 32 for MXFP8 */
  GL_ERR_UNSUPPORTED = -4, /* reserved: recognised but not provided by the library */
  GL_ERR_HIP = -5,         /* a HIP runtime call failed */
  GL_ERR_HOST_MEMORY = -6  /* a deferred-wgrad queue could not allocate its host record */
};

/* Status word bits written by gl_offsets (read back with gl_read_status). */
enum {
  GL_STATUS_NEGATIVE_SPLIT = 1, /* some m_splits[g] < 0 */
  GL_STATUS_SUM_MISMATCH = 2,   /* sum of m_splits != total_rows */
  GL_STATUS_WORKSPACE = 4,      /* a later call named a workspace built for other G / T */
  GL_STATUS_DEVICE_CHECK = 8    /* device-check build only (libgrouped_linear_checked.so): a
                                   kernel decoded a work item outside its launch's bounds (a
                                   workspace changed after the offsets call, or a defect) and
                                   skipped it without touching memory */
};

/*
 * Bytes of device workspace a call sequence over num_groups groups needs: the
 * offsets, the per-group row-tile tables and the status word (a few KiB), plus a
 * fixed area of 256 fp32 partial tiles of 256 x 256 and their arrival counters
 * (64 MiB + 1 KiB) where a GEMM launch whose last round of tiles would leave most
 * CUs idle splits those tiles over the contraction.  The split result is the same
 * on every run (partials are added in a fixed order).  One workspace serves one
 * call sequence at a time: calls that use the same workspace must not overlap
 * (same stream, or ordered by events).
 */
size_t gl_workspace_size(int num_groups);

/*
 * Split-offset scan (page "Single parameter for GroupedLinear module", Greptile
 * summary and the common.cu row of its files table: an exclusive prefix sum with a
 * leading zero, one kernel instead of cumsum + cat).
 *   m_splits   device int64[num_groups], row count of each group (zeros allowed)
 *   total_rows rows of x / dy; the splits must add up to it
 *   workspace  device buffer of gl_workspace_size(num_groups) bytes; receives the
 *              offsets int64[G+1] (off[0] = 0, off[g+1] = off[g] + m[g]), the
 *              per-group row-tile tables the GEMMs schedule from, and the status word.
 * One small kernel; reads m_splits once.  The workspace then serves every later
 * call of the same step (forward, dgrad, wgrad, bgrad) with the same G and T.
 */
int gl_offsets(const int64_t *m_splits, int num_groups, int64_t total_rows, void *workspace,
               hipStream_t stream);

/* Device address of the int64[G+1] offsets inside a workspace (no device access). */
const int64_t *gl_workspace_offsets(const void *workspace);

/* Synchronises `stream`, then copies the status word to *status (0 = valid splits). */
int gl_read_status(const void *workspace, int *status, hipStream_t stream);

/*
 * Grouped forward y[r,:] = x[r,:] W_g^T + b_g for the rows r of group g (page
 * "transformer_engine/pytorch/ops/basic/grouped_linear.py", class docstring and
 * fuser_forward "Perform GEMMs").
 *   in_dtype   GL_F32, GL_BF16, or GL_E4M3 (MXFP8: x and W are E4M3 codes with one
 *              E8M0 scale byte per 32 consecutive elements of a row, as produced by
 *              gl_group_quantize_mxfp8)
 *   out_dtype  equals in_dtype for GL_F32 / GL_BF16; GL_BF16 or GL_F32 for GL_E4M3
 *   x          [T, K] (elements of in_dtype); x_scale [T, K/32] bytes (E4M3 only, else NULL)
 *   w / w_ptrs stacked [G, N, K] or device array of G pointers to [N, K];
 *   w_scale / w_scale_ptrs  [G, N, K/32] or G pointers to [N, K/32] (E4M3 only)
 *   bias / bias_ptrs  [G, N] or G pointers to [N], type out_dtype; both NULL = no bias
 *   y          [y_rows, N] of out_dtype, y_rows >= T; rows >= T are never written
 * Accumulation is fp32 (MFMA); the bias is added to the fp32 sum before the single
 * rounding to out_dtype.
 */
int gl_forward(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows,
               gl_dtype in_dtype, gl_dtype out_dtype, const void *x, const uint8_t *x_scale,
               const void *w, const void *const *w_ptrs, const uint8_t *w_scale,
               const uint8_t *const *w_scale_ptrs, const void *bias, const void *const *bias_ptrs,
               void *y, int64_t y_rows, const void *workspace, hipStream_t stream);

/*
 * Grouped dgrad dx[r,:] = dy[r,:] W_g for the rows r of group g (page
 * "transformer_engine/pytorch/ops/basic/grouped_linear.py", fuser_backward
 * "Perform dgrad GEMMs", layout NN).
 *   dtype  GL_F32 or GL_BF16 for dy, W and dx
 *   dy [T, N]; w / w_ptrs as in gl_forward; dx [dx_rows, K], dx_rows >= T, rows >= T
 *   untouched (the caller-provided dgrad buffer of the caller-buffer pull request).
 */
int gl_dgrad(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows,
             gl_dtype dtype, const void *dy, const void *w, const void *const *w_ptrs, void *dx,
             int64_t dx_rows, const void *workspace, hipStream_t stream);

/*
 * Grouped wgrad dW_g = dy_g^T x_g, contracted over the m_splits[g] rows of group g
 * (page "transformer_engine/pytorch/ops/basic/grouped_linear.py", fuser_backward
 * "Perform wgrad GEMMs", layout NT; accumulate follows the main_grad fusion in
 * "Initialize grad weight buffers").
 *   in_dtype   GL_F32 or GL_BF16 for x [T, K] and dy [T, N]
 *   out_dtype  GL_BF16 or GL_F32 for dW (GL_F32 for an fp32 main_grad)
 *   dw / dw_ptrs  stacked [G, N, K] or device array of G pointers to [N, K]
 *   accumulate 0: dW_g is overwritten (an empty group writes zeros);
 *              1: dW_g += dy_g^T x_g (an empty group is not touched at all).
 * Every element of dW is produced by one work item in a fixed summation order, so
 * results are deterministic (no atomics).
 */
int gl_wgrad(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows,
             gl_dtype in_dtype, gl_dtype out_dtype, const void *x, const void *dy, void *dw,
             void *const *dw_ptrs, int accumulate, const void *workspace, hipStream_t stream);

/*
 * Bias grad db_g = sum over the rows of group g of dy (page
 * "transformer_engine/pytorch/ops/basic/grouped_linear.py", fuser_backward: a
 * column sum per split of the grad output).  fp32 accumulation in a fixed order;
 * an empty group gets zeros.
 *   dtype  GL_F32 or GL_BF16 for dy [T, N] and db
 *   db / db_ptrs  stacked [G, N] or device array of G pointers to [N]
 */
int gl_bgrad(int num_groups, int64_t out_features, int64_t total_rows, gl_dtype dtype,
             const void *dy, void *db, void *const *db_ptrs, const void *workspace,
             hipStream_t stream);

/*
 * gl_wgrad and gl_bgrad of the same dy in one call, dy read once (page
 * "transformer_engine/pytorch/ops/basic/grouped_linear.py", fuser_backward: the
 * bias gradient and the wgrad GEMMs both consume the grad output).  For bf16 / fp16
 * inputs the wgrad tiles of one column of in_features per group also add up their dy
 * stages while those sit in LDS, so no separate pass over dy runs; for fp32 inputs
 * the bias gradient is a second launch.  Arguments as gl_wgrad, plus
 *   db_dtype       GL_F32 or in_dtype
 *   db / db_ptrs   stacked [G, N] or device array of G pointers to [N]; every group
 *                  gets its column sums (zeros for an empty group, also when
 *                  accumulate leaves that group's main_grad untouched)
 * fp32 accumulation in a fixed order (deterministic).  For bf16 inputs each step adds
 * two rows with one fp32 dot instruction, whose add may differ from round-to-nearest
 * by about one ulp, so db may differ from gl_bgrad's in the last bits; exact whenever
 * the partial sums are representable (integer-valued inputs).
 */
int gl_wgrad_bgrad(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows,
                   gl_dtype in_dtype, gl_dtype out_dtype, gl_dtype db_dtype, const void *x, const void *dy,
                   void *dw, void *const *dw_ptrs, int accumulate, void *db, void *const *db_ptrs,
                   const void *workspace, hipStream_t stream);

/*
 * Rowwise MXFP8 quantization of a bf16 [rows, cols] matrix (page
 * "transformer_engine/pytorch/ops/basic/grouped_linear.py", _quantize_weights_mxfp8:
 * E4M3 data with one scale per 32 elements along the inner dimension; the scale
 * rule is OCP MX v1.0): per block of 32 consecutive elements of a row, shared
 * exponent e = floor(log2(amax)) - 8 clamped to [-127, 127] (all-zero block: -127),
 * scale byte = e + 127, codes = E4M3 round-to-nearest-even of v * 2^-e saturated
 * to +-448, signed zeros kept; a block holding Inf/NaN gets scale 0xFF and codes
 * 0x7F | sign.  Blocks never straddle rows, so stacked activations [T, K] and
 * stacked weights [G*N, K] are both one call, independent of m_splits.
 *   src  bf16 [rows, cols], cols % 32 == 0;  data  uint8 [rows, cols];
 *   scale  uint8 [rows, cols / 32] (compact, row-major, no padding)
 */
int gl_group_quantize_mxfp8(const void *src, int64_t rows, int64_t cols, uint8_t *data,
                            uint8_t *scale, hipStream_t stream);

/*
 * ---------------------------------------------------------------- MXFP8 backward
 * The quantized backward pass (page "transformer_engine/pytorch/ops/basic/
 * grouped_linear.py", op_forward and fuser_backward: dgrad runs on the grad output
 * quantized rowwise and the weights quantized columnwise; wgrad on the input and
 * the grad output quantized columnwise, each split on its own) contracts over
 * out_features in dgrad and over token rows in wgrad, so those operands carry
 * blocks of 32 along the rows.  This library stores columnwise codes transposed, so
 * a block's 32 codes are contiguous (the scale rule is the rowwise one, OCP MX v1.0):
 *   activations [T, C] split into groups -> codes [C, ld] and scales [C, ld / 32];
 *     group g's rows occupy columns [poff[g], poff[g] + m_g) with
 *     poff[g] = 128 * sum_{h<g} ceil(m_h / 128); its rows up to the next multiple
 *     of 128 are zero codes with scale byte 0; a group's last block may hold fewer
 *     than 32 rows (the zero padding leaves its amax unchanged).
 *   weights [G, N, K] -> codes [G, K, N] and scales [G, K, N / 32].
 */

/* Smallest row length ld of the transposed columnwise activation layout that fits
 * any split of total_rows rows into num_groups groups: T + 127 G rounded up to 128
 * (-1 for invalid sizes). */
int64_t gl_colwise_ld(int num_groups, int64_t total_rows);

/*
 * Columnwise MXFP8 group quantization of bf16 activations src [total_rows, cols]
 * (x or dy) into the transposed layout above, with the groups of the workspace
 * written by gl_offsets.  ld: a multiple of 128, at least gl_colwise_ld and at most
 * 2^23; cols % 4 == 0.  Columns past the last group's padding are not written.
 * src and data_t 16-byte aligned.  Split sizes found invalid by gl_offsets:
 * nothing is written.
 */
int gl_group_quantize_mxfp8_colwise(const void *src, int64_t cols, int num_groups, int64_t total_rows,
                                    const void *workspace, uint8_t *data_t, uint8_t *scale_t, int64_t ld,
                                    hipStream_t stream);

/*
 * Both usages of one bf16 tensor in one pass (page "transformer_engine/pytorch/ops/
 * basic/grouped_linear.py": a quantizer can make rowwise and columnwise data of the
 * same tensor; the quantized backward uses dy rowwise for dgrad and columnwise for
 * wgrad): data [total_rows, cols] / scale [total_rows, cols / 32] exactly as
 * gl_group_quantize_mxfp8 makes them, and data_t / scale_t exactly as
 * gl_group_quantize_mxfp8_colwise makes them.  cols % 32 == 0; src, data and data_t
 * 16-byte aligned; ld as for gl_group_quantize_mxfp8_colwise.  The input is read
 * once when scale_t is 4-byte aligned, else the two quantizations run as separate
 * launches.  Split sizes found invalid by gl_offsets: nothing is written.
 */
int gl_group_quantize_mxfp8_rowwise_colwise(const void *src, int64_t cols, int num_groups, int64_t total_rows,
                                            const void *workspace, uint8_t *data, uint8_t *scale, uint8_t *data_t,
                                            uint8_t *scale_t, int64_t ld, hipStream_t stream);

/*
 * Split-offset scan and rowwise MXFP8 quantization of the activations in one launch
 * (page "Single parameter for GroupedLinear module", review comments: compute the
 * tensor offsets in the same kernel rather than a separate cumsum; the grouped
 * MXFP8 forward quantizes x per split, page "Improve device-init grouped linear
 * module with single grouped weight support").  Exactly gl_offsets followed by
 * gl_group_quantize_mxfp8(x, total_rows, in_features, ...): the workspace gets the
 * offsets, tile tables and status word, and x [T, K] (bf16, K % 32 == 0) its codes
 * x_data [T, K] and scales x_scale [T, K / 32].  Rowwise blocks never straddle
 * rows, so the quantization is written even when the splits are found invalid
 * (the status word then stops every later kernel).  x and x_data 16-byte aligned.
 */
int gl_offsets_quantize_mxfp8(const int64_t *m_splits, int num_groups, int64_t total_rows, void *workspace,
                              const void *x, int64_t in_features, uint8_t *x_data, uint8_t *x_scale,
                              hipStream_t stream);

/*
 * gl_offsets_quantize_mxfp8 plus the columnwise codes of x for the wgrad (as
 * gl_group_quantize_mxfp8_colwise makes them, into x_data_t [K, ld] / x_scale_t
 * [K, ld / 32]), reading x once: with fewer than 64 groups and a 4-byte aligned
 * x_scale_t, one launch in which every workgroup derives the group offsets from
 * m_splits itself while the first also writes the workspace; otherwise the two
 * launches one after the other.  ld as for gl_group_quantize_mxfp8_colwise.
 * Invalid splits: the workspace's status word is set (which stops every later
 * kernel) and the codes are not to be used; the one-launch form writes none.
 */
int gl_offsets_quantize_mxfp8_rowwise_colwise(const int64_t *m_splits, int num_groups, int64_t total_rows,
                                              void *workspace, const void *x, int64_t in_features,
                                              uint8_t *x_data, uint8_t *x_scale, uint8_t *x_data_t,
                                              uint8_t *x_scale_t, int64_t ld, hipStream_t stream);

/*
 * The MXFP8 weight workspace, refreshed in one launch and skippable on the device
 * (page "Improve device-init grouped linear module with single grouped weight
 * support": group_quantize writes into a cached output in place and takes a
 * noop_flag, so a captured graph can replay the weight quantization without new
 * pointers).  w: stacked bf16 [G, N, K], K % 32 == 0, 16-byte aligned.
 *   data, scale      rowwise codes [G, N, K] and scales [G, N, K / 32] (the forward
 *                    operand, as gl_group_quantize_mxfp8 of w viewed as [G*N, K])
 *   data_t, scale_t  columnwise codes [G, K, N] and scales [G, K, N / 32] (the dgrad
 *                    operand, as gl_quantize_mxfp8_colwise_weights), or both NULL;
 *                    needs N % 32 == 0
 *   noop_flag        device int32, or NULL: when it holds a nonzero value at run
 *                    time nothing is written and the workspace keeps its contents
 */
int gl_quantize_mxfp8_weights(const void *w, int num_groups, int64_t out_features, int64_t in_features,
                              uint8_t *data, uint8_t *scale, uint8_t *data_t, uint8_t *scale_t,
                              const int32_t *noop_flag, hipStream_t stream);

/*
 * Columnwise MXFP8 of stacked bf16 weights w [G, N, K] (blocks of 32 along N, the
 * dgrad contraction) into codes [G, K, N] and scales [G, K, N / 32]; N % 32 == 0,
 * K % 4 == 0.
 */
int gl_quantize_mxfp8_colwise_weights(const void *w, int num_groups, int64_t out_features, int64_t in_features,
                                      uint8_t *data_t, uint8_t *scale_t, hipStream_t stream);

/*
 * MXFP8 grouped dgrad dx = deq(dy) deq(W_g) (page "transformer_engine/pytorch/ops/
 * basic/grouped_linear.py", fuser_backward "Perform dgrad GEMMs" on quantized
 * operands), fp32 accumulation.
 *   dy, dy_scale   rowwise codes [T, N] and scales [T, N / 32] (gl_group_quantize_mxfp8)
 *   w_t, w_t_scale columnwise weight codes [G, K, N] and scales [G, K, N / 32]
 *   out_dtype      GL_BF16 or GL_F32 for dx [dx_rows, K], dx_rows >= T, rows >= T untouched
 *   N % 128 == 0, K % 8 == 0.
 */
int gl_dgrad_mxfp8(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows,
                   gl_dtype out_dtype, const uint8_t *dy, const uint8_t *dy_scale, const uint8_t *w_t,
                   const uint8_t *w_t_scale, void *dx, int64_t dx_rows, const void *workspace, hipStream_t stream);

/*
 * MXFP8 grouped wgrad dW_g (+)= deq(dy_g)^T deq(x_g) (page "transformer_engine/
 * pytorch/ops/basic/grouped_linear.py", fuser_backward "Perform wgrad GEMMs" on
 * quantized operands), fp32 accumulation, from columnwise codes in the transposed
 * group layout: dy_t [N, ld] / dy_t_scale [N, ld / 32], x_t [K, ld] / x_t_scale
 * [K, ld / 32] (gl_group_quantize_mxfp8_colwise with the same workspace and ld).
 * dw / dw_ptrs, out_dtype and accumulate as in gl_wgrad (an empty group: zeros, or
 * untouched when accumulating).  K % 8 == 0, N % 8 == 0.
 */
int gl_wgrad_mxfp8(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows, gl_dtype out_dtype,
                   const uint8_t *dy_t, const uint8_t *dy_t_scale, const uint8_t *x_t, const uint8_t *x_t_scale,
                   int64_t ld, void *dw, void *const *dw_ptrs, int accumulate, const void *workspace,
                   hipStream_t stream);

/*
 * Grouped MLP: FC1 -> SwiGLU -> FC2 over the same splits (page "[PyTorch] Add
 * optional caller-provided output/grad-input buffers to GroupedLinear and fused
 * grouped MLP": a fused op of two grouped linear layers and an activation, whose
 * FC2 output and FC1 grad-input may be caller buffers of which only the packed
 * valid rows are written).  The pages do not name the activation; it is SwiGLU on
 * the two halves of FC1's output h [T, 2F]: a = silu(h[:, :F]) * h[:, F:], with
 * silu(v) = v / (1 + exp(-v)), computed in fp32 and rounded once to dtype.
 *
 * gl_swiglu_forward: a [T, F] from h [T, 2F].  gl_swiglu_backward: dh [T, 2F] from
 * h and the upstream gradient da [T, F] (dh_g = da * u * s (1 + g (1 - s)),
 * dh_u = da * g * s, s = sigmoid(g)).  dtype GL_F32, GL_BF16 or GL_F16; F a multiple
 * of 8 (16-bit) or 4 (fp32); buffers 16-byte aligned.
 */
int gl_swiglu_forward(int64_t total_rows, int64_t ffn_features, gl_dtype dtype, const void *h, void *a,
                      hipStream_t stream);
int gl_swiglu_backward(int64_t total_rows, int64_t ffn_features, gl_dtype dtype, const void *h, const void *da,
                       void *dh, hipStream_t stream);

/*
 * Grouped MLP forward: h = FC1(x) (+ b1), a = SwiGLU(h), y = FC2(a) (+ b2).
 *   x [T, K]; w1 / w1_ptrs [G, 2F, K] or G x [2F, K]; b1 / b1_ptrs [G, 2F] or NULL;
 *   w2 / w2_ptrs [G, N, F] or G x [N, F]; b2 / b2_ptrs [G, N] or NULL
 *   h [T, 2F], a [T, F]: caller buffers, kept for the backward
 *   y [y_rows, N], y_rows >= T: rows >= T are never written
 * All tensors of dtype (GL_F32, GL_BF16 or GL_F16).  Every step is checked before
 * any kernel is launched; the rules of gl_forward apply to both GEMMs.
 */
int gl_grouped_mlp_forward(int num_groups, int64_t in_features, int64_t ffn_features, int64_t out_features,
                           int64_t total_rows, gl_dtype dtype, const void *x, const void *w1,
                           const void *const *w1_ptrs, const void *b1, const void *const *b1_ptrs, const void *w2,
                           const void *const *w2_ptrs, const void *b2, const void *const *b2_ptrs, void *h, void *a,
                           void *y, int64_t y_rows, const void *workspace, hipStream_t stream);

/*
 * Grouped MLP backward, given the forward's x, h, a and the grad output dy [T, N]:
 *   FC2: dW2_g (+)= dy_g^T a_g and db2 (fused, one pass over dy); da = dy W2_g
 *   SwiGLU: dh from h and da
 *   FC1: dW1_g (+)= dh_g^T x_g and db1 (fused); dx = dh W1_g
 *   da [T, F], dh [T, 2F]: caller scratch; dx [dx_rows, K], dx_rows >= T, rows >= T
 *   never written; dw1 / dw2 stacked or per-group, of wgrad_dtype (GL_F32 or dtype),
 *   accumulate as in gl_wgrad; db1 / db2 of dtype, stacked or per-group, both forms
 *   NULL to skip a bias gradient.  Every step is checked before any is launched.
 */
int gl_grouped_mlp_backward(int num_groups, int64_t in_features, int64_t ffn_features, int64_t out_features,
                            int64_t total_rows, gl_dtype dtype, gl_dtype wgrad_dtype, const void *x, const void *w1,
                            const void *const *w1_ptrs, const void *w2, const void *const *w2_ptrs, const void *h,
                            const void *a, const void *dy, void *da, void *dh, void *dx, int64_t dx_rows, void *dw1,
                            void *const *dw1_ptrs, void *db1, void *const *db1_ptrs, void *dw2,
                            void *const *dw2_ptrs, void *db2, void *const *db2_ptrs, int accumulate,
                            const void *workspace, hipStream_t stream);

/*
 * Deferred weight gradients (page "transformer_engine/pytorch/ops/basic/
 * grouped_linear.py", delay_wgrad_compute and backward_dw): the backward pass puts
 * its wgrad call in a queue instead of running it, and a later call runs the
 * oldest put call, so the weight-gradient GEMMs can be scheduled after the rest of
 * the backward (for instance behind another layer's dgrad or a communication).
 *
 * A queue is a host object (host memory only, not thread-safe: one thread at a
 * time).  gl_wgrad_queue_put takes the arguments of gl_wgrad_bgrad without the
 * stream (db and db_ptrs both NULL: plain gl_wgrad, db_dtype ignored), and
 * gl_wgrad_queue_put_mxfp8 those of gl_wgrad_mxfp8.  Every check of that entry
 * point runs at put time, with the same errors; on an error nothing is queued.
 * A put or create that cannot allocate its host record returns GL_ERR_HOST_MEMORY.
 * Nothing is launched and no device memory is read by a put.  The queue keeps the
 * pointers: the caller keeps every buffer, pointer array and the workspace alive
 * and unchanged until the call has run, and the workspace must still hold the
 * offsets of the same splits (gl_offsets on it in between changes what runs).
 *
 * gl_wgrad_queue_run_next launches the oldest queued call on `stream` (nothing if
 * the queue is empty); gl_wgrad_queue_flush launches all of them in put order.  A
 * launched call leaves the queue whatever its result; if a launch fails, flush
 * drops the calls after it and returns the error.  gl_wgrad_queue_size returns the
 * number of queued calls (>= 0), gl_wgrad_queue_clear drops them without running,
 * gl_wgrad_queue_destroy frees the queue (queued calls are dropped; NULL is a
 * no-op).
 */
typedef struct gl_wgrad_queue gl_wgrad_queue;
int gl_wgrad_queue_create(gl_wgrad_queue **queue);
int gl_wgrad_queue_destroy(gl_wgrad_queue *queue);
int gl_wgrad_queue_put(gl_wgrad_queue *queue, int num_groups, int64_t in_features, int64_t out_features,
                       int64_t total_rows, gl_dtype in_dtype, gl_dtype out_dtype, gl_dtype db_dtype, const void *x,
                       const void *dy, void *dw, void *const *dw_ptrs, int accumulate, void *db,
                       void *const *db_ptrs, const void *workspace);
int gl_wgrad_queue_put_mxfp8(gl_wgrad_queue *queue, int num_groups, int64_t in_features, int64_t out_features,
                             int64_t total_rows, gl_dtype out_dtype, const uint8_t *dy_t, const uint8_t *dy_t_scale,
                             const uint8_t *x_t, const uint8_t *x_t_scale, int64_t ld, void *dw,
                             void *const *dw_ptrs, int accumulate, const void *workspace);
int gl_wgrad_queue_size(const gl_wgrad_queue *queue);
int gl_wgrad_queue_run_next(gl_wgrad_queue *queue, hipStream_t stream);
int gl_wgrad_queue_flush(gl_wgrad_queue *queue, hipStream_t stream);
int gl_wgrad_queue_clear(gl_wgrad_queue *queue);

/*
 * Allocation-free grouped forward, for callers that cannot allocate device memory
 * or hand the library a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  It is gl_offsets followed by gl_forward
 * (same arguments, same results, same host checks and errors), except that the
 * offsets, tile tables, status word and split area live in a file-scope device
 * array of the library instead of a caller workspace:
 *   - at most GL_NOALLOC_MAX_GROUPS groups (more: GL_ERR_SHAPE); the array is
 *     about 16.4 MiB (the tables for that many groups plus GL_NOALLOC_SPLIT_SLOTS
 *     fp32 partial tiles of 256 x 256), held on every device the library runs this
 *     call on until the process ends;
 *   - nothing is allocated: no hipMalloc, no library allocation;
 *   - every call on one device shares that device's array and leaves its contents
 *     behind; each call rewrites what it reads (the scan zeroes the split
 *     counters), so calls in sequence are independent, but calls that overlap on
 *     one device (different streams, not ordered by events) race;
 *   - split sizes found invalid on the device make the forward write nothing;
 *     there is no status word for the caller to read.
 * The split area is smaller than a workspace's, so the tail-round split of a
 * launch may use fewer parts than gl_forward does (results then differ by fp32
 * summation order only).
 */
#define GL_NOALLOC_MAX_GROUPS 16384
#define GL_NOALLOC_SPLIT_SLOTS 64
int gl_forward_noalloc(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows,
                       gl_dtype in_dtype, gl_dtype out_dtype, const int64_t *m_splits, const void *x,
                       const uint8_t *x_scale, const void *w, const void *const *w_ptrs, const uint8_t *w_scale,
                       const uint8_t *const *w_scale_ptrs, const void *bias, const void *const *bias_ptrs, void *y,
                       int64_t y_rows, hipStream_t stream);

/* Message of the last error on this thread ("" if none). */
const char *gl_last_error(void);

/* Library identification string. */
const char *gl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GROUPED_LINEAR_H */
