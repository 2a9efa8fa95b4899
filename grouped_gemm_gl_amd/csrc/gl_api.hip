// Host entry points of the C ABI declared in include/grouped_linear.h.
//
// Each entry point validates its arguments on the host before anything is
// enqueued (the reference layer raises before allocating or launching: page
// "transformer_engine/pytorch/ops/basic/grouped_linear.py", constructor and
// fuser_forward checks; caller buffers are validated by shape/dtype/contiguity on
// page "[PyTorch] Add optional caller-provided output/grad-input buffers ...").  On
// an error nothing is launched and the message is kept per thread.
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <deque>
#include <mutex>
#include <new>

#include "../../include/grouped_linear.h"
#include "gl_common.hpp"

namespace gl {
hipError_t launch_offsets(const int64_t *m_splits, int G, int64_t total_rows, void *ws, int split_slots,
                          hipStream_t stream);
hipError_t launch_forward_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *x, const uint16_t *w,
                               const uint16_t *const *w_ptrs, const void *bias, const void *const *bias_ptrs,
                               uint16_t *y, int f16, const void *ws, hipStream_t s);
hipError_t launch_dgrad_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *dy, const uint16_t *w,
                             const uint16_t *const *w_ptrs, uint16_t *dx, int f16, const void *ws, hipStream_t s);
hipError_t launch_wgrad_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *x, const uint16_t *dy,
                             void *dw, void *const *dw_ptrs, int out_f32, int accumulate, int f16, void *db,
                             void *const *db_ptrs, int db_f32, const void *ws, hipStream_t s);
hipError_t launch_forward_mxfp8(int G, int64_t K, int64_t N, int64_t T, const uint8_t *xq, const uint8_t *xs,
                                const uint8_t *wq, const uint8_t *const *wq_ptrs, const uint8_t *ws_scale,
                                const uint8_t *const *ws_scale_ptrs, const void *bias,
                                const void *const *bias_ptrs, void *y, int out_f32, const void *ws,
                                hipStream_t s);
hipError_t launch_forward_f32(int G, int64_t K, int64_t N, int64_t T, const float *x, const float *w,
                              const float *const *w_ptrs, const float *bias, const float *const *bias_ptrs,
                              float *y, const void *ws, hipStream_t s);
hipError_t launch_dgrad_f32(int G, int64_t K, int64_t N, int64_t T, const float *dy, const float *w,
                            const float *const *w_ptrs, float *dx, const void *ws, hipStream_t s);
hipError_t launch_wgrad_f32(int G, int64_t K, int64_t N, int64_t T, const float *x, const float *dy, float *dw,
                            float *const *dw_ptrs, int accumulate, const void *ws, hipStream_t s);
hipError_t launch_bgrad(int G, int64_t N, int64_t T, int el, const void *dy, void *db, void *const *db_ptrs,
                        const void *ws, hipStream_t s);
hipError_t launch_quantize_mxfp8(const uint16_t *src, int64_t rows, int64_t cols, uint8_t *data, uint8_t *scale,
                                 hipStream_t s);
hipError_t launch_quantize_mxfp8_colwise(const uint16_t *src, int64_t cols, int G, int64_t total_rows,
                                         const void *ws, uint8_t *data, uint8_t *scale, int64_t ld, hipStream_t s);
hipError_t launch_quantize_mxfp8_colwise_weights(const uint16_t *w, int G, int64_t N, int64_t K, uint8_t *data,
                                                 uint8_t *scale, hipStream_t s);
hipError_t launch_quantize_mxfp8_rowwise_colwise(const uint16_t *src, int64_t cols, int G, int64_t total_rows,
                                                 const void *ws, uint8_t *row_data, uint8_t *row_scale,
                                                 uint8_t *data, uint8_t *scale, int64_t ld, hipStream_t s);
hipError_t launch_offsets_quantize_mxfp8_rowwise_colwise(const int64_t *m_splits, int G, int64_t total_rows,
                                                         void *ws, const uint16_t *src, int64_t cols,
                                                         uint8_t *row_data, uint8_t *row_scale, uint8_t *data,
                                                         uint8_t *scale, int64_t ld, hipStream_t s);
hipError_t launch_offsets_quantize_mxfp8(const int64_t *m_splits, int G, int64_t total_rows, void *ws,
                                         const uint16_t *src, int64_t cols, uint8_t *data, uint8_t *scale,
                                         hipStream_t s);
hipError_t launch_quantize_mxfp8_weights(const uint16_t *w, int G, int64_t N, int64_t K, uint8_t *data,
                                         uint8_t *scale, uint8_t *data_t, uint8_t *scale_t, const int32_t *noop,
                                         hipStream_t s);
hipError_t launch_swiglu_fwd(int el, int64_t T, int64_t F, const void *h, void *a, hipStream_t s);
hipError_t launch_swiglu_bwd(int el, int64_t T, int64_t F, const void *h, const void *da, void *dh, hipStream_t s);
hipError_t launch_wgrad_mxfp8(int G, int64_t K, int64_t N, int64_t T, const uint8_t *dyt, const uint8_t *dyt_s,
                              const uint8_t *xt, const uint8_t *xt_s, int64_t ld, void *dw, void *const *dw_ptrs,
                              int out_f32, int accumulate, const void *ws, hipStream_t s);
}  // namespace gl

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return GL_OK;
}

int hip_result(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(GL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Sizes shared by every GEMM entry point.
int check_sizes(int G, int64_t K, int64_t N, int64_t T) {
  if (G <= 0) return fail(GL_ERR_ARG, "Invalid number of groups (%d)", G);
  if (K <= 0) return fail(GL_ERR_ARG, "Invalid input size (%lld)", (long long)K);
  if (N <= 0) return fail(GL_ERR_ARG, "Invalid output size (%lld)", (long long)N);
  if (T < 0) return fail(GL_ERR_ARG, "Invalid total_rows (%lld)", (long long)T);
  if (T > INT32_MAX || (int64_t)G * 256 > INT32_MAX)
    return fail(GL_ERR_SHAPE, "sizes exceed the 32-bit work-item range");
  return GL_OK;
}

int check_float_dtype(gl_dtype d, const char *what) {
  if (d != GL_F32 && d != GL_BF16 && d != GL_F16)
    return fail(GL_ERR_DTYPE, "%s: dtype must be GL_F32, GL_BF16 or GL_F16", what);
  return GL_OK;
}

bool is16(gl_dtype d) { return d == GL_BF16 || d == GL_F16; }

int check_one_form(const void *stacked, const void *ptrs, const char *what, bool optional) {
  if (stacked && ptrs) return fail(GL_ERR_ARG, "%s: pass either the stacked buffer or the pointer array, not both", what);
  if (!optional && !stacked && !ptrs) return fail(GL_ERR_ARG, "%s: missing (stacked buffer or pointer array)", what);
  if (stacked && !aligned16(stacked)) return fail(GL_ERR_ARG, "%s: buffer not 16-byte aligned", what);
  if (ptrs && ((uintptr_t)ptrs & 7u)) return fail(GL_ERR_ARG, "%s: pointer array not 8-byte aligned", what);
  return GL_OK;
}

int check_buf(const void *p, int64_t T, const char *what) {
  if (T == 0) return GL_OK;
  if (!p) return fail(GL_ERR_ARG, "%s is NULL", what);
  if (!aligned16(p)) return fail(GL_ERR_ARG, "%s not 16-byte aligned", what);
  return GL_OK;
}

// The GEMMs address a 256-row stage of an operand with 32-bit byte offsets from
// the stage's base, so a row may hold at most 2^22 elements (bf16, fp16; MXFP8
// codes are bounded the same way).
constexpr int64_t kMaxBf16Dim = (int64_t)1 << 22;

int check_bf16_dims(gl_dtype d, int64_t K, int64_t N) {
  if (is16(d) && (K % 8 || N % 8))
    return fail(GL_ERR_SHAPE, "bf16/fp16 need in_features and out_features that are multiples of 8 (got %lld, %lld)",
                (long long)K, (long long)N);
  if (is16(d) && (K > kMaxBf16Dim || N > kMaxBf16Dim))
    return fail(GL_ERR_SHAPE, "bf16/fp16 in_features and out_features must be at most %lld (got %lld, %lld)",
                (long long)kMaxBf16Dim, (long long)K, (long long)N);
  return GL_OK;
}

}  // namespace

#define GL_TRY(expr)          \
  do {                        \
    int _rc = (expr);         \
    if (_rc != GL_OK) return _rc; \
  } while (0)

extern "C" {

size_t gl_workspace_size(int num_groups) { return num_groups > 0 ? gl::ws_bytes(num_groups) : 0; }

const int64_t *gl_workspace_offsets(const void *workspace) {
  return workspace ? (const int64_t *)((const char *)workspace + gl::ws_offsets_byte(0)) : nullptr;
}

const char *gl_last_error(void) { return g_err; }

const char *gl_version(void) { return "grouped_gemm_gl_amd 0.1 (gfx950)"; }

int gl_offsets(const int64_t *m_splits, int num_groups, int64_t total_rows, void *workspace, hipStream_t stream) {
  if (num_groups <= 0) return fail(GL_ERR_ARG, "Invalid number of groups (%d)", num_groups);
  if (total_rows < 0) return fail(GL_ERR_ARG, "Invalid total_rows (%lld)", (long long)total_rows);
  if (!m_splits) return fail(GL_ERR_ARG, "m_splits is NULL");
  if ((uintptr_t)m_splits & 7u) return fail(GL_ERR_ARG, "m_splits not 8-byte aligned");
  if (!workspace || !aligned16(workspace)) return fail(GL_ERR_ARG, "workspace NULL or not 16-byte aligned");
  return hip_result(gl::launch_offsets(m_splits, num_groups, total_rows, workspace, gl::kSplitSlots, stream),
                    "gl_offsets");
}

int gl_read_status(const void *workspace, int *status, hipStream_t stream) {
  if (!workspace || !status) return fail(GL_ERR_ARG, "workspace or status is NULL");
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_result(e, "gl_read_status");
  int32_t st = 0;
  e = hipMemcpy(&st, workspace, sizeof(st), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_result(e, "gl_read_status");
  *status = st;
  return ok();
}

}  // extern "C"

namespace {
// The entry points' checks, then (launch) the kernels; with launch false only the
// checks run, so a composite call can check every step before it launches any.
int forward_impl(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows, gl_dtype in_dtype,
                 gl_dtype out_dtype, const void *x, const uint8_t *x_scale, const void *w, const void *const *w_ptrs,
                 const uint8_t *w_scale, const uint8_t *const *w_scale_ptrs, const void *bias,
                 const void *const *bias_ptrs, void *y, int64_t y_rows, const void *workspace, hipStream_t stream,
                 bool launch) {
  const int G = num_groups;
  const int64_t K = in_features, N = out_features, T = total_rows;
  GL_TRY(check_sizes(G, K, N, T));
  if (!workspace) return fail(GL_ERR_ARG, "workspace is NULL");
  if (y_rows < T) return fail(GL_ERR_SHAPE, "output buffer has %lld rows, needs at least %lld", (long long)y_rows,
                              (long long)T);
  GL_TRY(check_one_form(w, w_ptrs, "weight", false));
  GL_TRY(check_one_form(bias, bias_ptrs, "bias", true));
  GL_TRY(check_buf(x, T, "x"));
  GL_TRY(check_buf(y, T, "y"));
  if (in_dtype == GL_E4M3) {
    if (out_dtype != GL_BF16 && out_dtype != GL_F32)
      return fail(GL_ERR_DTYPE, "MXFP8 forward: out_dtype must be GL_BF16 or GL_F32");
    if (K % 128) return fail(GL_ERR_SHAPE, "MXFP8 forward needs in_features %% 128 == 0 (got %lld)", (long long)K);
    if (N % 8) return fail(GL_ERR_SHAPE, "MXFP8 forward needs out_features %% 8 == 0 (got %lld)", (long long)N);
    if (K > kMaxBf16Dim || N > kMaxBf16Dim)
      return fail(GL_ERR_SHAPE, "MXFP8 in_features and out_features must be at most %lld (got %lld, %lld)",
                  (long long)kMaxBf16Dim, (long long)K, (long long)N);
    if (T > 0 && (!x_scale || ((uintptr_t)x_scale & 3u))) return fail(GL_ERR_ARG, "x_scale NULL or not 4-byte aligned");
    if ((w != nullptr) != (w_scale != nullptr) || (w_ptrs != nullptr) != (w_scale_ptrs != nullptr))
      return fail(GL_ERR_ARG, "weight scales must come in the same form as the weights");
    if (w_scale && ((uintptr_t)w_scale & 3u)) return fail(GL_ERR_ARG, "w_scale not 4-byte aligned");
    if (T == 0 || !launch) return ok();
    return hip_result(gl::launch_forward_mxfp8(G, K, N, T, (const uint8_t *)x, x_scale, (const uint8_t *)w,
                                               (const uint8_t *const *)w_ptrs, w_scale, w_scale_ptrs, bias,
                                               bias_ptrs, y, out_dtype == GL_F32, workspace, stream),
                      "gl_forward");
  }
  GL_TRY(check_float_dtype(in_dtype, "gl_forward"));
  if (out_dtype != in_dtype)
    return fail(GL_ERR_DTYPE, "gl_forward: out_dtype must equal in_dtype for fp32/bf16/fp16");
  if (x_scale || w_scale || w_scale_ptrs) return fail(GL_ERR_ARG, "scales are only for GL_E4M3 inputs");
  GL_TRY(check_bf16_dims(in_dtype, K, N));
  if (T == 0 || !launch) return ok();
  hipError_t e;
  if (is16(in_dtype))
    e = gl::launch_forward_bf16(G, K, N, T, (const uint16_t *)x, (const uint16_t *)w,
                                (const uint16_t *const *)w_ptrs, bias, bias_ptrs, (uint16_t *)y, in_dtype == GL_F16,
                                workspace, stream);
  else
    e = gl::launch_forward_f32(G, K, N, T, (const float *)x, (const float *)w, (const float *const *)w_ptrs,
                               (const float *)bias, (const float *const *)bias_ptrs, (float *)y, workspace, stream);
  return hip_result(e, "gl_forward");
}

int dgrad_impl(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows, gl_dtype dtype,
               const void *dy, const void *w, const void *const *w_ptrs, void *dx, int64_t dx_rows,
               const void *workspace, hipStream_t stream, bool launch) {
  const int G = num_groups;
  const int64_t K = in_features, N = out_features, T = total_rows;
  GL_TRY(check_sizes(G, K, N, T));
  GL_TRY(check_float_dtype(dtype, "gl_dgrad"));
  GL_TRY(check_bf16_dims(dtype, K, N));
  if (!workspace) return fail(GL_ERR_ARG, "workspace is NULL");
  if (dx_rows < T) return fail(GL_ERR_SHAPE, "dgrad buffer has %lld rows, needs at least %lld", (long long)dx_rows,
                               (long long)T);
  GL_TRY(check_one_form(w, w_ptrs, "weight", false));
  GL_TRY(check_buf(dy, T, "dy"));
  GL_TRY(check_buf(dx, T, "dx"));
  if (T == 0 || !launch) return ok();
  hipError_t e;
  if (is16(dtype))
    e = gl::launch_dgrad_bf16(G, K, N, T, (const uint16_t *)dy, (const uint16_t *)w, (const uint16_t *const *)w_ptrs,
                              (uint16_t *)dx, dtype == GL_F16, workspace, stream);
  else
    e = gl::launch_dgrad_f32(G, K, N, T, (const float *)dy, (const float *)w, (const float *const *)w_ptrs,
                             (float *)dx, workspace, stream);
  return hip_result(e, "gl_dgrad");
}

// gl_wgrad, and with db / db_ptrs set also the bias gradient of the same dy.
int wgrad_impl(const char *who, int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows,
               gl_dtype in_dtype, gl_dtype out_dtype, const void *x, const void *dy, void *dw, void *const *dw_ptrs,
               int accumulate, bool with_db, gl_dtype db_dtype, void *db, void *const *db_ptrs,
               const void *workspace, hipStream_t stream, bool launch = true) {
  const int G = num_groups;
  const int64_t K = in_features, N = out_features, T = total_rows;
  GL_TRY(check_sizes(G, K, N, T));
  GL_TRY(check_float_dtype(in_dtype, "gl_wgrad"));
  GL_TRY(check_float_dtype(out_dtype, "gl_wgrad"));
  if (out_dtype != GL_F32 && out_dtype != in_dtype)
    return fail(GL_ERR_DTYPE, "gl_wgrad: the weight gradient is fp32 or the input type");
  GL_TRY(check_bf16_dims(in_dtype, K, N));
  if (!workspace) return fail(GL_ERR_ARG, "workspace is NULL");
  GL_TRY(check_one_form(dw, dw_ptrs, "weight gradient", false));
  GL_TRY(check_buf(x, T, "x"));
  GL_TRY(check_buf(dy, T, "dy"));
  if (accumulate != 0 && accumulate != 1) return fail(GL_ERR_ARG, "accumulate must be 0 or 1");
  if (with_db) {
    if (db_dtype != GL_F32 && db_dtype != in_dtype)
      return fail(GL_ERR_DTYPE, "%s: the bias gradient is fp32 or the input type", who);
    GL_TRY(check_one_form(db, db_ptrs, "bias gradient", false));
    if (!is16(in_dtype) && N % 4) return fail(GL_ERR_SHAPE, "%s needs out_features %% 4 == 0 for fp32", who);
  }
  if (!launch) return ok();
  hipError_t e;
  if (is16(in_dtype)) {
    e = gl::launch_wgrad_bf16(G, K, N, T, (const uint16_t *)x, (const uint16_t *)dy, dw, dw_ptrs,
                              out_dtype == GL_F32, accumulate, in_dtype == GL_F16, with_db ? db : nullptr,
                              with_db ? db_ptrs : nullptr, db_dtype == GL_F32, workspace, stream);
  } else {
    e = gl::launch_wgrad_f32(G, K, N, T, (const float *)x, (const float *)dy, (float *)dw, (float *const *)dw_ptrs,
                             accumulate, workspace, stream);
    // fp32: the bias gradient is its own (HBM-bound) launch
    if (e == hipSuccess && with_db) e = gl::launch_bgrad(G, N, T, 1, dy, db, db_ptrs, workspace, stream);
  }
  return hip_result(e, who);
}
}  // namespace

extern "C" {

int gl_forward(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows, gl_dtype in_dtype,
               gl_dtype out_dtype, const void *x, const uint8_t *x_scale, const void *w, const void *const *w_ptrs,
               const uint8_t *w_scale, const uint8_t *const *w_scale_ptrs, const void *bias,
               const void *const *bias_ptrs, void *y, int64_t y_rows, const void *workspace,
               hipStream_t stream) {
  return forward_impl(num_groups, in_features, out_features, total_rows, in_dtype, out_dtype, x, x_scale, w, w_ptrs,
                      w_scale, w_scale_ptrs, bias, bias_ptrs, y, y_rows, workspace, stream, true);
}

int gl_dgrad(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows, gl_dtype dtype,
             const void *dy, const void *w, const void *const *w_ptrs, void *dx, int64_t dx_rows,
             const void *workspace, hipStream_t stream) {
  return dgrad_impl(num_groups, in_features, out_features, total_rows, dtype, dy, w, w_ptrs, dx, dx_rows, workspace,
                    stream, true);
}

int gl_wgrad(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows, gl_dtype in_dtype,
             gl_dtype out_dtype, const void *x, const void *dy, void *dw, void *const *dw_ptrs, int accumulate,
             const void *workspace, hipStream_t stream) {
  return wgrad_impl("gl_wgrad", num_groups, in_features, out_features, total_rows, in_dtype, out_dtype, x, dy, dw,
                    dw_ptrs, accumulate, false, GL_F32, nullptr, nullptr, workspace, stream);
}

int gl_wgrad_bgrad(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows, gl_dtype in_dtype,
                   gl_dtype out_dtype, gl_dtype db_dtype, const void *x, const void *dy, void *dw,
                   void *const *dw_ptrs, int accumulate, void *db, void *const *db_ptrs, const void *workspace,
                   hipStream_t stream) {
  return wgrad_impl("gl_wgrad_bgrad", num_groups, in_features, out_features, total_rows, in_dtype, out_dtype, x, dy,
                    dw, dw_ptrs, accumulate, true, db_dtype, db, db_ptrs, workspace, stream);
}

int gl_bgrad(int num_groups, int64_t out_features, int64_t total_rows, gl_dtype dtype, const void *dy, void *db,
             void *const *db_ptrs, const void *workspace, hipStream_t stream) {
  const int G = num_groups;
  const int64_t N = out_features, T = total_rows;
  GL_TRY(check_sizes(G, 8, N, T));
  GL_TRY(check_float_dtype(dtype, "gl_bgrad"));
  if (N % (is16(dtype) ? 8 : 4))
    return fail(GL_ERR_SHAPE, "gl_bgrad needs out_features %% %d == 0", is16(dtype) ? 8 : 4);
  if (!workspace) return fail(GL_ERR_ARG, "workspace is NULL");
  GL_TRY(check_one_form(db, db_ptrs, "bias gradient", false));
  GL_TRY(check_buf(dy, T, "dy"));
  return hip_result(gl::launch_bgrad(G, N, T, dtype == GL_F32 ? 1 : dtype == GL_F16 ? 2 : 0, dy, db, db_ptrs, workspace,
                                     stream),
                    "gl_bgrad");
}

int gl_group_quantize_mxfp8(const void *src, int64_t rows, int64_t cols, uint8_t *data, uint8_t *scale,
                            hipStream_t stream) {
  if (rows < 0 || cols <= 0) return fail(GL_ERR_ARG, "Invalid shape (%lld, %lld)", (long long)rows, (long long)cols);
  if (cols % 32) return fail(GL_ERR_SHAPE, "cols must be a multiple of 32 (got %lld)", (long long)cols);
  if (rows == 0) return ok();
  if (!src || !data || !scale) return fail(GL_ERR_ARG, "src, data or scale is NULL");
  if (!aligned16(src) || !aligned16(data)) return fail(GL_ERR_ARG, "src and data must be 16-byte aligned");
  return hip_result(gl::launch_quantize_mxfp8((const uint16_t *)src, rows, cols, data, scale, stream),
                    "gl_group_quantize_mxfp8");
}

}  // extern "C"

int64_t gl_colwise_ld(int num_groups, int64_t total_rows) {
  if (num_groups <= 0 || total_rows < 0) return -1;
  const int64_t need = total_rows + 127 * (int64_t)num_groups;
  return (need + 127) / 128 * 128;
}

namespace {
// The columnwise layout's row length: room for every group's padded rows, and few
// enough that a 256-row GEMM stage stays within 32-bit byte offsets.
int check_colwise_ld(int G, int64_t T, int64_t ld) {
  if (ld % 128 || ld < gl_colwise_ld(G, T))
    return fail(GL_ERR_SHAPE, "ld must be a multiple of 128 and at least %lld (got %lld)",
                (long long)gl_colwise_ld(G, T), (long long)ld);
  if (ld > ((int64_t)1 << 23)) return fail(GL_ERR_SHAPE, "ld must be at most 2^23 (got %lld)", (long long)ld);
  return GL_OK;
}
}  // namespace

int gl_group_quantize_mxfp8_colwise(const void *src, int64_t cols, int num_groups, int64_t total_rows,
                                    const void *workspace, uint8_t *data_t, uint8_t *scale_t, int64_t ld,
                                    hipStream_t stream) {
  const int G = num_groups;
  if (G <= 0 || total_rows < 0 || cols <= 0)
    return fail(GL_ERR_ARG, "Invalid sizes (groups %d, rows %lld, cols %lld)", G, (long long)total_rows,
                (long long)cols);
  if (cols % 4) return fail(GL_ERR_SHAPE, "cols must be a multiple of 4 (got %lld)", (long long)cols);
  GL_TRY(check_colwise_ld(G, total_rows, ld));
  if (!workspace) return fail(GL_ERR_ARG, "workspace is NULL");
  if (total_rows == 0) return ok();
  if (!src || !data_t || !scale_t) return fail(GL_ERR_ARG, "src, data_t or scale_t is NULL");
  if (!aligned16(src) || !aligned16(data_t)) return fail(GL_ERR_ARG, "src and data_t must be 16-byte aligned");
  return hip_result(gl::launch_quantize_mxfp8_colwise((const uint16_t *)src, cols, G, total_rows, workspace, data_t,
                                                      scale_t, ld, stream),
                    "gl_group_quantize_mxfp8_colwise");
}

int gl_group_quantize_mxfp8_rowwise_colwise(const void *src, int64_t cols, int num_groups, int64_t total_rows,
                                            const void *workspace, uint8_t *data, uint8_t *scale, uint8_t *data_t,
                                            uint8_t *scale_t, int64_t ld, hipStream_t stream) {
  const int G = num_groups;
  if (G <= 0 || total_rows < 0 || cols <= 0)
    return fail(GL_ERR_ARG, "Invalid sizes (groups %d, rows %lld, cols %lld)", G, (long long)total_rows,
                (long long)cols);
  if (cols % 32) return fail(GL_ERR_SHAPE, "cols must be a multiple of 32 (got %lld)", (long long)cols);
  if (total_rows * (cols / 32) / 256 >= ((int64_t)1 << 31))
    return fail(GL_ERR_SHAPE, "src too large for one launch (%lld x %lld)", (long long)total_rows, (long long)cols);
  GL_TRY(check_colwise_ld(G, total_rows, ld));
  if (!workspace) return fail(GL_ERR_ARG, "workspace is NULL");
  if (total_rows == 0) return ok();
  if (!src || !data || !scale || !data_t || !scale_t) return fail(GL_ERR_ARG, "a buffer is NULL");
  if (!aligned16(src) || !aligned16(data) || !aligned16(data_t))
    return fail(GL_ERR_ARG, "src, data and data_t must be 16-byte aligned");
  return hip_result(gl::launch_quantize_mxfp8_rowwise_colwise((const uint16_t *)src, cols, G, total_rows, workspace,
                                                              data, scale, data_t, scale_t, ld, stream),
                    "gl_group_quantize_mxfp8_rowwise_colwise");
}

int gl_offsets_quantize_mxfp8_rowwise_colwise(const int64_t *m_splits, int num_groups, int64_t total_rows,
                                              void *workspace, const void *x, int64_t in_features,
                                              uint8_t *x_data, uint8_t *x_scale, uint8_t *x_data_t,
                                              uint8_t *x_scale_t, int64_t ld, hipStream_t stream) {
  const int G = num_groups;
  const int64_t K = in_features;
  if (G <= 0) return fail(GL_ERR_ARG, "Invalid number of groups (%d)", G);
  if (total_rows < 0 || K <= 0) return fail(GL_ERR_ARG, "Invalid shape (%lld, %lld)", (long long)total_rows, (long long)K);
  if (K % 32) return fail(GL_ERR_SHAPE, "in_features must be a multiple of 32 (got %lld)", (long long)K);
  if (total_rows * (K / 32) / 256 >= ((int64_t)1 << 31))
    return fail(GL_ERR_SHAPE, "x too large for one launch (%lld x %lld)", (long long)total_rows, (long long)K);
  GL_TRY(check_colwise_ld(G, total_rows, ld));
  if (!m_splits || ((uintptr_t)m_splits & 7u)) return fail(GL_ERR_ARG, "m_splits NULL or not 8-byte aligned");
  if (!workspace || !aligned16(workspace)) return fail(GL_ERR_ARG, "workspace NULL or not 16-byte aligned");
  if (total_rows > 0) {
    if (!x || !x_data || !x_scale || !x_data_t || !x_scale_t) return fail(GL_ERR_ARG, "a buffer is NULL");
    if (!aligned16(x) || !aligned16(x_data) || !aligned16(x_data_t))
      return fail(GL_ERR_ARG, "x, x_data and x_data_t must be 16-byte aligned");
  }
  return hip_result(gl::launch_offsets_quantize_mxfp8_rowwise_colwise(m_splits, G, total_rows, workspace,
                                                                      (const uint16_t *)x, K, x_data, x_scale,
                                                                      x_data_t, x_scale_t, ld, stream),
                    "gl_offsets_quantize_mxfp8_rowwise_colwise");
}

int gl_offsets_quantize_mxfp8(const int64_t *m_splits, int num_groups, int64_t total_rows, void *workspace,
                              const void *x, int64_t in_features, uint8_t *x_data, uint8_t *x_scale,
                              hipStream_t stream) {
  const int64_t K = in_features;
  if (num_groups <= 0) return fail(GL_ERR_ARG, "Invalid number of groups (%d)", num_groups);
  if (total_rows < 0 || K <= 0)
    return fail(GL_ERR_ARG, "Invalid shape (%lld, %lld)", (long long)total_rows, (long long)K);
  if (K % 32) return fail(GL_ERR_SHAPE, "in_features must be a multiple of 32 (got %lld)", (long long)K);
  if (total_rows * (K / 32) / 256 >= ((int64_t)1 << 31))
    return fail(GL_ERR_SHAPE, "x too large for one launch (%lld x %lld)", (long long)total_rows, (long long)K);
  if (!m_splits || ((uintptr_t)m_splits & 7u)) return fail(GL_ERR_ARG, "m_splits NULL or not 8-byte aligned");
  if (!workspace || !aligned16(workspace)) return fail(GL_ERR_ARG, "workspace NULL or not 16-byte aligned");
  if (total_rows > 0) {
    if (!x || !x_data || !x_scale) return fail(GL_ERR_ARG, "x, x_data or x_scale is NULL");
    if (!aligned16(x) || !aligned16(x_data)) return fail(GL_ERR_ARG, "x and x_data must be 16-byte aligned");
  }
  return hip_result(gl::launch_offsets_quantize_mxfp8(m_splits, num_groups, total_rows, workspace,
                                                      (const uint16_t *)x, K, x_data, x_scale, stream),
                    "gl_offsets_quantize_mxfp8");
}

int gl_quantize_mxfp8_weights(const void *w, int num_groups, int64_t out_features, int64_t in_features,
                              uint8_t *data, uint8_t *scale, uint8_t *data_t, uint8_t *scale_t,
                              const int32_t *noop_flag, hipStream_t stream) {
  const int G = num_groups;
  const int64_t N = out_features, K = in_features;
  if (G <= 0 || N <= 0 || K <= 0)
    return fail(GL_ERR_ARG, "Invalid sizes (groups %d, N %lld, K %lld)", G, (long long)N, (long long)K);
  if (K % 32) return fail(GL_ERR_SHAPE, "in_features must be a multiple of 32 (got %lld)", (long long)K);
  if (!w || !data || !scale) return fail(GL_ERR_ARG, "w, data or scale is NULL");
  if (!aligned16(w) || !aligned16(data)) return fail(GL_ERR_ARG, "w and data must be 16-byte aligned");
  if ((data_t == nullptr) != (scale_t == nullptr)) return fail(GL_ERR_ARG, "give both data_t and scale_t, or neither");
  if (data_t) {
    if (N % 32) return fail(GL_ERR_SHAPE, "columnwise codes need out_features %% 32 == 0 (got %lld)", (long long)N);
    if (!aligned16(data_t)) return fail(GL_ERR_ARG, "data_t must be 16-byte aligned");
  }
  if (noop_flag && ((uintptr_t)noop_flag & 3u)) return fail(GL_ERR_ARG, "noop_flag must be 4-byte aligned");
  return hip_result(gl::launch_quantize_mxfp8_weights((const uint16_t *)w, G, N, K, data, scale, data_t, scale_t,
                                                      noop_flag, stream),
                    "gl_quantize_mxfp8_weights");
}

int gl_quantize_mxfp8_colwise_weights(const void *w, int num_groups, int64_t out_features, int64_t in_features,
                                      uint8_t *data_t, uint8_t *scale_t, hipStream_t stream) {
  const int G = num_groups;
  const int64_t N = out_features, K = in_features;
  if (G <= 0 || N <= 0 || K <= 0)
    return fail(GL_ERR_ARG, "Invalid sizes (groups %d, N %lld, K %lld)", G, (long long)N, (long long)K);
  if (N % 32) return fail(GL_ERR_SHAPE, "out_features must be a multiple of 32 (got %lld)", (long long)N);
  if (K % 4) return fail(GL_ERR_SHAPE, "in_features must be a multiple of 4 (got %lld)", (long long)K);
  if (!w || !data_t || !scale_t) return fail(GL_ERR_ARG, "w, data_t or scale_t is NULL");
  if ((uintptr_t)w & 7u) return fail(GL_ERR_ARG, "w must be 8-byte aligned");
  if (!aligned16(data_t)) return fail(GL_ERR_ARG, "data_t must be 16-byte aligned");
  return hip_result(gl::launch_quantize_mxfp8_colwise_weights((const uint16_t *)w, G, N, K, data_t, scale_t, stream),
                    "gl_quantize_mxfp8_colwise_weights");
}

int gl_dgrad_mxfp8(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows,
                   gl_dtype out_dtype, const uint8_t *dy, const uint8_t *dy_scale, const uint8_t *w_t,
                   const uint8_t *w_t_scale, void *dx, int64_t dx_rows, const void *workspace, hipStream_t stream) {
  const int G = num_groups;
  const int64_t K = in_features, N = out_features, T = total_rows;
  GL_TRY(check_sizes(G, K, N, T));
  if (out_dtype != GL_BF16 && out_dtype != GL_F32)
    return fail(GL_ERR_DTYPE, "gl_dgrad_mxfp8: out_dtype must be GL_BF16 or GL_F32");
  if (N % 128) return fail(GL_ERR_SHAPE, "MXFP8 dgrad needs out_features %% 128 == 0 (got %lld)", (long long)N);
  if (K % 8) return fail(GL_ERR_SHAPE, "MXFP8 dgrad needs in_features %% 8 == 0 (got %lld)", (long long)K);
  if (K > kMaxBf16Dim || N > kMaxBf16Dim)
    return fail(GL_ERR_SHAPE, "MXFP8 in_features and out_features must be at most %lld (got %lld, %lld)",
                (long long)kMaxBf16Dim, (long long)K, (long long)N);
  if (!workspace) return fail(GL_ERR_ARG, "workspace is NULL");
  if (dx_rows < T) return fail(GL_ERR_SHAPE, "dgrad buffer has %lld rows, needs at least %lld", (long long)dx_rows,
                               (long long)T);
  if (!w_t || !w_t_scale) return fail(GL_ERR_ARG, "w_t or w_t_scale is NULL");
  if (!aligned16(w_t) || ((uintptr_t)w_t_scale & 3u)) return fail(GL_ERR_ARG, "w_t / w_t_scale misaligned");
  GL_TRY(check_buf(dy, T, "dy"));
  GL_TRY(check_buf(dx, T, "dx"));
  if (T > 0 && (!dy_scale || ((uintptr_t)dy_scale & 3u))) return fail(GL_ERR_ARG, "dy_scale NULL or misaligned");
  if (T == 0) return ok();
  // dx = dy W_g: the MXFP8 forward kernel with contraction N and B = W_g^T [K, N]
  return hip_result(gl::launch_forward_mxfp8(G, N, K, T, dy, dy_scale, w_t, nullptr, w_t_scale, nullptr, nullptr,
                                             nullptr, dx, out_dtype == GL_F32, workspace, stream),
                    "gl_dgrad_mxfp8");
}

namespace {
int wgrad_mxfp8_impl(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows,
                     gl_dtype out_dtype, const uint8_t *dy_t, const uint8_t *dy_t_scale, const uint8_t *x_t,
                     const uint8_t *x_t_scale, int64_t ld, void *dw, void *const *dw_ptrs, int accumulate,
                     const void *workspace, hipStream_t stream, bool launch = true) {
  const int G = num_groups;
  const int64_t K = in_features, N = out_features, T = total_rows;
  GL_TRY(check_sizes(G, K, N, T));
  if (out_dtype != GL_BF16 && out_dtype != GL_F32)
    return fail(GL_ERR_DTYPE, "gl_wgrad_mxfp8: out_dtype must be GL_BF16 or GL_F32");
  if (K % 8 || N % 8)
    return fail(GL_ERR_SHAPE, "MXFP8 wgrad needs in/out_features that are multiples of 8 (got %lld, %lld)",
                (long long)K, (long long)N);
  GL_TRY(check_colwise_ld(G, T, ld));
  if (!workspace) return fail(GL_ERR_ARG, "workspace is NULL");
  GL_TRY(check_one_form(dw, dw_ptrs, "weight gradient", false));
  if (accumulate != 0 && accumulate != 1) return fail(GL_ERR_ARG, "accumulate must be 0 or 1");
  if (!dy_t || !x_t || !dy_t_scale || !x_t_scale) return fail(GL_ERR_ARG, "codes or scales are NULL");
  if (!aligned16(dy_t) || !aligned16(x_t) || ((uintptr_t)dy_t_scale & 3u) || ((uintptr_t)x_t_scale & 3u))
    return fail(GL_ERR_ARG, "codes must be 16-byte and scales 4-byte aligned");
  if (!launch) return ok();
  return hip_result(gl::launch_wgrad_mxfp8(G, K, N, T, dy_t, dy_t_scale, x_t, x_t_scale, ld, dw, dw_ptrs,
                                           out_dtype == GL_F32, accumulate, workspace, stream),
                    "gl_wgrad_mxfp8");
}
}  // namespace

extern "C" {

int gl_wgrad_mxfp8(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows, gl_dtype out_dtype,
                   const uint8_t *dy_t, const uint8_t *dy_t_scale, const uint8_t *x_t, const uint8_t *x_t_scale,
                   int64_t ld, void *dw, void *const *dw_ptrs, int accumulate, const void *workspace,
                   hipStream_t stream) {
  return wgrad_mxfp8_impl(num_groups, in_features, out_features, total_rows, out_dtype, dy_t, dy_t_scale, x_t,
                          x_t_scale, ld, dw, dw_ptrs, accumulate, workspace, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ grouped MLP --

namespace {
// in1 is the backward's upstream gradient (need_in1), unused in the forward
int swiglu_check(const char *who, int64_t T, int64_t F, gl_dtype dtype, const void *in0, const void *in1,
                 const void *out, bool need_in1) {
  if (T < 0 || F <= 0) return fail(GL_ERR_ARG, "%s: invalid sizes (T %lld, F %lld)", who, (long long)T, (long long)F);
  GL_TRY(check_float_dtype(dtype, who));
  const int v = is16(dtype) ? 8 : 4;
  if (F % v) return fail(GL_ERR_SHAPE, "%s: F must be a multiple of %d (got %lld)", who, v, (long long)F);
  if (F > ((int64_t)1 << 22)) return fail(GL_ERR_SHAPE, "%s: F must be at most 2^22", who);
  if (T == 0) return GL_OK;
  if (!in0 || !out || (need_in1 && !in1)) return fail(GL_ERR_ARG, "%s: a buffer is NULL", who);
  if (!aligned16(in0) || !aligned16(out) || (in1 && !aligned16(in1)))
    return fail(GL_ERR_ARG, "%s: buffers must be 16-byte aligned", who);
  return GL_OK;
}
int sw_el(gl_dtype d) { return d == GL_F32 ? 1 : d == GL_F16 ? 2 : 0; }
}  // namespace

extern "C" {

int gl_swiglu_forward(int64_t total_rows, int64_t F, gl_dtype dtype, const void *h, void *a, hipStream_t stream) {
  GL_TRY(swiglu_check("gl_swiglu_forward", total_rows, F, dtype, h, nullptr, a, false));
  if (total_rows == 0) return ok();
  return hip_result(gl::launch_swiglu_fwd(sw_el(dtype), total_rows, F, h, a, stream), "gl_swiglu_forward");
}

int gl_swiglu_backward(int64_t total_rows, int64_t F, gl_dtype dtype, const void *h, const void *da, void *dh,
                       hipStream_t stream) {
  GL_TRY(swiglu_check("gl_swiglu_backward", total_rows, F, dtype, h, da, dh, true));
  if (total_rows == 0) return ok();
  return hip_result(gl::launch_swiglu_bwd(sw_el(dtype), total_rows, F, h, da, dh, stream), "gl_swiglu_backward");
}

int gl_grouped_mlp_forward(int num_groups, int64_t in_features, int64_t ffn_features, int64_t out_features,
                           int64_t total_rows, gl_dtype dtype, const void *x, const void *w1,
                           const void *const *w1_ptrs, const void *b1, const void *const *b1_ptrs, const void *w2,
                           const void *const *w2_ptrs, const void *b2, const void *const *b2_ptrs, void *h, void *a,
                           void *y, int64_t y_rows, const void *workspace, hipStream_t stream) {
  const int G = num_groups;
  const int64_t K = in_features, F = ffn_features, N = out_features, T = total_rows;
  // every step is checked before any is launched
  GL_TRY(check_float_dtype(dtype, "gl_grouped_mlp_forward"));
  GL_TRY(swiglu_check("gl_grouped_mlp_forward", T, F, dtype, h, nullptr, a, false));
  GL_TRY(forward_impl(G, K, 2 * F, T, dtype, dtype, x, nullptr, w1, w1_ptrs, nullptr, nullptr, b1, b1_ptrs, h, T,
                      workspace, stream, false));
  GL_TRY(forward_impl(G, F, N, T, dtype, dtype, a, nullptr, w2, w2_ptrs, nullptr, nullptr, b2, b2_ptrs, y, y_rows,
                      workspace, stream, false));
  if (T == 0) return ok();
  GL_TRY(forward_impl(G, K, 2 * F, T, dtype, dtype, x, nullptr, w1, w1_ptrs, nullptr, nullptr, b1, b1_ptrs, h, T,
                      workspace, stream, true));
  GL_TRY(hip_result(gl::launch_swiglu_fwd(sw_el(dtype), T, F, h, a, stream), "gl_grouped_mlp_forward"));
  return forward_impl(G, F, N, T, dtype, dtype, a, nullptr, w2, w2_ptrs, nullptr, nullptr, b2, b2_ptrs, y, y_rows,
                      workspace, stream, true);
}

int gl_grouped_mlp_backward(int num_groups, int64_t in_features, int64_t ffn_features, int64_t out_features,
                            int64_t total_rows, gl_dtype dtype, gl_dtype wgrad_dtype, const void *x, const void *w1,
                            const void *const *w1_ptrs, const void *w2, const void *const *w2_ptrs, const void *h,
                            const void *a, const void *dy, void *da, void *dh, void *dx, int64_t dx_rows, void *dw1,
                            void *const *dw1_ptrs, void *db1, void *const *db1_ptrs, void *dw2,
                            void *const *dw2_ptrs, void *db2, void *const *db2_ptrs, int accumulate,
                            const void *workspace, hipStream_t stream) {
  const int G = num_groups;
  const int64_t K = in_features, F = ffn_features, N = out_features, T = total_rows;
  const bool bias1 = db1 || db1_ptrs, bias2 = db2 || db2_ptrs;
  GL_TRY(check_float_dtype(dtype, "gl_grouped_mlp_backward"));
  GL_TRY(swiglu_check("gl_grouped_mlp_backward", T, F, dtype, h, da, dh, true));
  auto fc2_wgrad = [&](bool launch) {
    return wgrad_impl("gl_grouped_mlp_backward (FC2 wgrad)", G, F, N, T, dtype, wgrad_dtype, a, dy, dw2, dw2_ptrs,
                      accumulate, bias2, dtype, db2, db2_ptrs, workspace, stream, launch);
  };
  auto fc2_dgrad = [&](bool launch) {
    return dgrad_impl(G, F, N, T, dtype, dy, w2, w2_ptrs, da, T, workspace, stream, launch);
  };
  auto fc1_wgrad = [&](bool launch) {
    return wgrad_impl("gl_grouped_mlp_backward (FC1 wgrad)", G, K, 2 * F, T, dtype, wgrad_dtype, x, dh, dw1,
                      dw1_ptrs, accumulate, bias1, dtype, db1, db1_ptrs, workspace, stream, launch);
  };
  auto fc1_dgrad = [&](bool launch) {
    return dgrad_impl(G, K, 2 * F, T, dtype, dh, w1, w1_ptrs, dx, dx_rows, workspace, stream, launch);
  };
  GL_TRY(fc2_wgrad(false));
  GL_TRY(fc2_dgrad(false));
  GL_TRY(fc1_wgrad(false));
  GL_TRY(fc1_dgrad(false));
  GL_TRY(fc2_wgrad(true));  // also runs for T == 0: empty groups' weight and bias gradients
  GL_TRY(fc2_dgrad(true));
  if (T > 0) GL_TRY(hip_result(gl::launch_swiglu_bwd(sw_el(dtype), T, F, h, da, dh, stream), "gl_grouped_mlp_backward"));
  GL_TRY(fc1_wgrad(true));
  return fc1_dgrad(true);
}

}  // extern "C"

// ------------------------------------------------------------ deferred wgrad --
//
// The layer of page "transformer_engine/pytorch/ops/basic/grouped_linear.py" can
// delay its weight-gradient GEMMs (delay_wgrad_compute): the backward stores the
// wgrad call with its operands, and backward_dw later takes the oldest stored call
// and runs it.  Here the stored call is a host record of the C arguments, checked
// in full when it is put, so running it can only fail in the HIP launch.

struct gl_wgrad_queue {
  struct Entry {
    bool mx;  // gl_wgrad_mxfp8 form, else gl_wgrad / gl_wgrad_bgrad form
    int G;
    int64_t K, N, T;
    gl_dtype in_dtype, out_dtype, db_dtype;
    const void *x, *dy;
    void *dw;
    void *const *dw_ptrs;
    int accumulate;
    bool with_db;
    void *db;
    void *const *db_ptrs;
    const uint8_t *dy_t, *dy_t_scale, *x_t, *x_t_scale;
    int64_t ld;
    const void *workspace;
  };
  std::deque<Entry> pending;
};

namespace {
int run_entry(const gl_wgrad_queue::Entry &e, hipStream_t stream) {
  if (e.mx)
    return wgrad_mxfp8_impl(e.G, e.K, e.N, e.T, e.out_dtype, e.dy_t, e.dy_t_scale, e.x_t, e.x_t_scale, e.ld, e.dw,
                            e.dw_ptrs, e.accumulate, e.workspace, stream);
  return wgrad_impl(e.with_db ? "gl_wgrad_bgrad" : "gl_wgrad", e.G, e.K, e.N, e.T, e.in_dtype, e.out_dtype, e.x,
                    e.dy, e.dw, e.dw_ptrs, e.accumulate, e.with_db, e.db_dtype, e.db, e.db_ptrs, e.workspace,
                    stream);
}

// No C++ exception may cross the C ABI: a record that cannot be stored is an error.
int enqueue(gl_wgrad_queue *queue, const gl_wgrad_queue::Entry &e) {
  try {
    queue->pending.push_back(e);
  } catch (const std::bad_alloc &) {
    return fail(GL_ERR_HOST_MEMORY, "out of host memory");
  }
  return ok();
}
}  // namespace

extern "C" {

int gl_wgrad_queue_create(gl_wgrad_queue **queue) {
  if (!queue) return fail(GL_ERR_ARG, "queue is NULL");
  *queue = new (std::nothrow) gl_wgrad_queue();
  if (!*queue) return fail(GL_ERR_HOST_MEMORY, "out of host memory");
  return ok();
}

int gl_wgrad_queue_destroy(gl_wgrad_queue *queue) {
  delete queue;
  return ok();
}

int gl_wgrad_queue_put(gl_wgrad_queue *queue, int num_groups, int64_t in_features, int64_t out_features,
                       int64_t total_rows, gl_dtype in_dtype, gl_dtype out_dtype, gl_dtype db_dtype, const void *x,
                       const void *dy, void *dw, void *const *dw_ptrs, int accumulate, void *db,
                       void *const *db_ptrs, const void *workspace) {
  if (!queue) return fail(GL_ERR_ARG, "queue is NULL");
  gl_wgrad_queue::Entry e{};
  e.mx = false;
  e.G = num_groups;
  e.K = in_features;
  e.N = out_features;
  e.T = total_rows;
  e.in_dtype = in_dtype;
  e.out_dtype = out_dtype;
  e.db_dtype = db_dtype;
  e.x = x;
  e.dy = dy;
  e.dw = dw;
  e.dw_ptrs = dw_ptrs;
  e.accumulate = accumulate;
  e.with_db = db || db_ptrs;
  e.db = db;
  e.db_ptrs = db_ptrs;
  e.workspace = workspace;
  GL_TRY(wgrad_impl(e.with_db ? "gl_wgrad_bgrad" : "gl_wgrad", e.G, e.K, e.N, e.T, e.in_dtype, e.out_dtype, e.x,
                    e.dy, e.dw, e.dw_ptrs, e.accumulate, e.with_db, e.db_dtype, e.db, e.db_ptrs, e.workspace,
                    nullptr, false));
  return enqueue(queue, e);
}

int gl_wgrad_queue_put_mxfp8(gl_wgrad_queue *queue, int num_groups, int64_t in_features, int64_t out_features,
                             int64_t total_rows, gl_dtype out_dtype, const uint8_t *dy_t, const uint8_t *dy_t_scale,
                             const uint8_t *x_t, const uint8_t *x_t_scale, int64_t ld, void *dw,
                             void *const *dw_ptrs, int accumulate, const void *workspace) {
  if (!queue) return fail(GL_ERR_ARG, "queue is NULL");
  GL_TRY(wgrad_mxfp8_impl(num_groups, in_features, out_features, total_rows, out_dtype, dy_t, dy_t_scale, x_t,
                          x_t_scale, ld, dw, dw_ptrs, accumulate, workspace, nullptr, false));
  gl_wgrad_queue::Entry e{};
  e.mx = true;
  e.G = num_groups;
  e.K = in_features;
  e.N = out_features;
  e.T = total_rows;
  e.out_dtype = out_dtype;
  e.dy_t = dy_t;
  e.dy_t_scale = dy_t_scale;
  e.x_t = x_t;
  e.x_t_scale = x_t_scale;
  e.ld = ld;
  e.dw = dw;
  e.dw_ptrs = dw_ptrs;
  e.accumulate = accumulate;
  e.workspace = workspace;
  return enqueue(queue, e);
}

int gl_wgrad_queue_size(const gl_wgrad_queue *queue) {
  if (!queue) return fail(GL_ERR_ARG, "queue is NULL");
  return (int)queue->pending.size();
}

int gl_wgrad_queue_run_next(gl_wgrad_queue *queue, hipStream_t stream) {
  if (!queue) return fail(GL_ERR_ARG, "queue is NULL");
  if (queue->pending.empty()) return ok();
  const gl_wgrad_queue::Entry e = queue->pending.front();
  queue->pending.pop_front();
  return run_entry(e, stream);
}

int gl_wgrad_queue_flush(gl_wgrad_queue *queue, hipStream_t stream) {
  if (!queue) return fail(GL_ERR_ARG, "queue is NULL");
  while (!queue->pending.empty()) {
    const gl_wgrad_queue::Entry e = queue->pending.front();
    queue->pending.pop_front();
    const int rc = run_entry(e, stream);
    if (rc != GL_OK) {
      const size_t dropped = queue->pending.size();
      queue->pending.clear();
      if (dropped) {
        char msg[sizeof(g_err)];
        snprintf(msg, sizeof(msg), "%s (%zu later calls dropped)", g_err, dropped);
        return fail(rc, "%s", msg);
      }
      return rc;
    }
  }
  return ok();
}

int gl_wgrad_queue_clear(gl_wgrad_queue *queue) {
  if (!queue) return fail(GL_ERR_ARG, "queue is NULL");
  queue->pending.clear();
  return ok();
}

}  // extern "C"

// ------------------------------------------------------ allocation-free forward
// gl_forward_noalloc: the offsets and the forward's split area live in `scratch`, a
// file-scope device array of fixed size, instead of a caller workspace.  Host code
// never passes the array's name to a kernel (on the host it is a stand-in, not a
// device address): the device address comes from hipGetSymbolAddress, once per
// device, and is kept per device.
namespace {
constexpr int kNoallocSlots = GL_NOALLOC_SPLIT_SLOTS;
constexpr size_t kNoallocBytes = gl::ws_bytes_slots(GL_NOALLOC_MAX_GROUPS, kNoallocSlots);
static_assert(kNoallocBytes <= ((size_t)17 << 20), "the allocation-free forward's scratch stays small");
}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call
// per device, with that device current).
int scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_result(e, "gl_forward_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(GL_ERR_UNSUPPORTED, "gl_forward_noalloc: device %d beyond the %d devices it serves", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_result(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                                   "gl_forward_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GL_OK;
}
}  // namespace

extern "C" {

int gl_forward_noalloc(int num_groups, int64_t in_features, int64_t out_features, int64_t total_rows,
                       gl_dtype in_dtype, gl_dtype out_dtype, const int64_t *m_splits, const void *x,
                       const uint8_t *x_scale, const void *w, const void *const *w_ptrs, const uint8_t *w_scale,
                       const uint8_t *const *w_scale_ptrs, const void *bias, const void *const *bias_ptrs, void *y,
                       int64_t y_rows, hipStream_t stream) {
  if (num_groups > GL_NOALLOC_MAX_GROUPS)
    return fail(GL_ERR_SHAPE, "gl_forward_noalloc: %d groups exceed its maximum of %d (use gl_forward with a "
                "workspace)", num_groups, GL_NOALLOC_MAX_GROUPS);
  if (num_groups <= 0) return fail(GL_ERR_ARG, "Invalid number of groups (%d)", num_groups);
  if (!m_splits) return fail(GL_ERR_ARG, "m_splits is NULL");
  if ((uintptr_t)m_splits & 7u) return fail(GL_ERR_ARG, "m_splits not 8-byte aligned");
  // every argument check of gl_forward, before anything is enqueued (a stand-in
  // workspace pointer: these checks only test it for NULL)
  GL_TRY(forward_impl(num_groups, in_features, out_features, total_rows, in_dtype, out_dtype, x, x_scale, w, w_ptrs,
                      w_scale, w_scale_ptrs, bias, bias_ptrs, y, y_rows, m_splits, stream, false));
  if (total_rows == 0) return ok();
  void *ws = nullptr;
  GL_TRY(scratch_address(&ws));
  // the scan rewrites the header and tables and zeroes the split counters, so
  // nothing of the previous call's contents is read
  GL_TRY(hip_result(gl::launch_offsets(m_splits, num_groups, total_rows, ws, kNoallocSlots, stream),
                    "gl_forward_noalloc"));
  return forward_impl(num_groups, in_features, out_features, total_rows, in_dtype, out_dtype, x, x_scale, w, w_ptrs,
                      w_scale, w_scale_ptrs, bias, bias_ptrs, y, y_rows, ws, stream, true);
}

}  // extern "C"
