// Persistent grouped GEMM for the MXFP8 forward on gfx950: y = deq(xq) deq(wq)^T (+ b)
// with the scaled fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4), fp32 accumulation.
//
// The operands are the outputs of the MXFP8 group quantizer (page "Improve
// device-init grouped linear module with single grouped weight support", the
// grouped MXFP8 weight workspace; OCP MX E4M3 codes with one E8M0 scale per 32
// codes along K): codes xq [T, K] and wq [N, K] per group, scales [rows, K/32].
//
// Same tile machinery as the bf16 kernel (gl_gemm_tile.hpp): 256x256 outputs per
// workgroup, 8 waves of 128x64, a 2-stage LDS ring filled by direct buffer->LDS
// loads with the K-major layout.  Codes travel as 2-byte units, so a 128-byte stage
// row is 128 codes = 4 scale blocks and one stage is two 64-code MFMA steps.
// Alongside each stage every A and B row's 4 scale bytes (one dword) are loaded
// straight into a small LDS area: waves 0-3 load the A rows' dwords, waves 4-7
// the B rows'.  Each lane then passes its row's byte for the step's block to the
// MFMA (lane l of a 32x32x64 operand holds row l % 32 of block l / 32).
#include "gl_gemm_tile.hpp"

namespace gl {

namespace gemm {

// One 4-byte direct load per lane per stage: the scale dword of one tile row.
struct ScaleStream {
  const char *base;  // scale row 0 of the tile
  uint32_t off;      // this lane's row offset (rows past the tile's extent clamp)

  __device__ __forceinline__ void init(const uint8_t *rows, int64_t ld, int rv, int r) {
    base = (const char *)rows;
    off = (uint32_t)((int64_t)(r < rv ? r : rv - 1) * ld);
  }
  __device__ __forceinline__ void issue(int t, uint32_t *dst) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_at(base + 4 * t), (GL_LDS void *)dst, 4, off, 0, 0, 0);
  }
};

// MODE_ROWS: forward (and dgrad on transposed columnwise weight codes);
// MODE_KCONTR: wgrad on transposed columnwise codes of dy and x.
template <int MODE>
__global__ __launch_bounds__(kThreads) void gemm_mxfp8_kernel(Params p) {
  // One LDS object: the stage ring, then the scale dwords of every tile row
  // [kS][A, B][256].  (A second __shared__ array makes the compiler wait for every
  // outstanding direct-to-LDS load before each LDS read.)
  __shared__ __attribute__((aligned(1024))) char lds[kS * kStageBytes + kS * 2 * 256 * 4];
  uint32_t(*lds_sc)[2][256] = (uint32_t(*)[2][256])(lds + kS * kStageBytes);

  const WsView ws = ws_view(p.ws, p.G);
  if (!ws_usable(ws.hdr, p.G, p.T)) return;
  const int64_t *__restrict__ off = ws.off;
  const int32_t *__restrict__ pre = ws.pre[tile_rows_index(kBM)];
  const int32_t *__restrict__ cpre = ws.pre[tile_rows_index(128)];

  const int total = MODE == MODE_ROWS ? pre[p.G] * p.tiles_j : p.G * p.tiles_i * p.tiles_j;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int grid = gridDim.x, b = blockIdx.x;
  const int first = (grid & 7) == 0 ? (b & 7) * (grid >> 3) + (b >> 3) : b;

  for (int w = first; w < total; w += grid) {
    const Tile t = decode_tile<true, true, MODE>(p, off, pre, w, cpre);
    if (MODE == MODE_KCONTR && p.accumulate && t.g_rows == 0) continue;  // main_grad untouched
    // every stage is complete: K % 128 == 0 in row mode, padded groups otherwise
    const int nk = (int)(t.pmax / kBK);

    Stream<true> sa, sb;
    sa.init(t.a_base, p.lda, t.a_rv, wave, lane);
    sb.init(t.b_base, p.ldb, t.b_rv, wave, lane);
    ScaleStream ss;
    if (MODE == MODE_ROWS) {
      if (wave < 4) {
        ss.init(p.a_scale + (t.g_off + (int64_t)t.it * kBM) * p.scale_ld, p.scale_ld, t.a_rv, wave * 64 + lane);
      } else {
        const uint8_t *bs = p.b_scale ? p.b_scale + (int64_t)t.g * p.cols_j * p.scale_ld : p.b_scale_ptrs[t.g];
        ss.init(bs + (int64_t)t.jt * kBN * p.scale_ld, p.scale_ld, t.b_rv, (wave - 4) * 64 + lane);
      }
    } else {  // scale columns of the group start at 4 per padded 128-element tile
      const int64_t c0 = 4 * (int64_t)cpre[t.g];
      if (wave < 4)
        ss.init(p.a_scale + (int64_t)t.it * kBM * p.scale_ld + c0, p.scale_ld, t.a_rv, wave * 64 + lane);
      else
        ss.init(p.b_scale + (int64_t)t.jt * kBN * p.scale_ld + c0, p.scale_ld, t.b_rv, (wave - 4) * 64 + lane);
    }
    auto stage_ptr = [&](int s) { return lds + (s % kS) * kStageBytes; };
    auto issue = [&](int s) {
      char *st = stage_ptr(s);
      sa.issue_full(s, st, wave);
      sb.issue_full(s, st + kOpBytes, wave);
      ss.issue(s, &lds_sc[s % kS][wave >> 2][(wave & 3) * 64]);
    };

    f32x16_t acc[kNI][kNJ];
#pragma unroll
    for (int ii = 0; ii < kNI; ++ii)
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[ii][jj][q] = 0.f;

    // One 64-code step: the two B fragments first, then the A fragments one at a
    // time (32-byte fragments leave no room for a second fragment set).
    auto step_mx = [&](int s, int st_, const uint32_t *scl) {
      const char *ta = stage_ptr(s), *tb = ta + kOpBytes;
      const int sh = 8 * (2 * st_ + (lane >> 5));  // this lane's scale block in the step
      i32x8_t bfr[kNJ];
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj) bfr[jj] = frag_mx(tb, wn * kWTN + jj * 32, st_, lane);
#pragma unroll
      for (int ii = 0; ii < kNI; ++ii) {
        const i32x8_t af = frag_mx(ta, wm * kWTM + ii * 32, st_, lane);
#pragma unroll
        for (int jj = 0; jj < kNJ; ++jj)
          acc[ii][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              bfr[jj], af, acc[ii][jj], 0, 0, 0, (int)(scl[kNI + jj] >> sh), 0, (int)(scl[ii] >> sh));
      }
    };

    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    if (nk > 0) {
      issue(0);
      wait_vm0();
      __builtin_amdgcn_s_barrier();
    }
    for (int kt = 0; kt < nk; ++kt) {
      // the stage kt + 1 loads go into the slot stage kt - 1 used, freed by the
      // barrier that ended stage kt - 1
      if (kt + 1 < nk) issue(kt + 1);
      fence();
      uint32_t sc[kNI + kNJ];  // scale dwords of this lane's A and B rows for stage kt
#pragma unroll
      for (int ii = 0; ii < kNI; ++ii) sc[ii] = lds_sc[kt % kS][0][wm * kWTM + ii * 32 + (lane & 31)];
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj) sc[kNI + jj] = lds_sc[kt % kS][1][wn * kWTN + jj * 32 + (lane & 31)];
      step_mx(kt, 0, sc);
      step_mx(kt, 1, sc);
      fence();
      wait_vm0();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
    }
    // the wgrad's short contractions make its 1 GiB output the larger cost: there
    // the tile goes out through LDS as whole lines
    if (MODE != MODE_ROWS && !p.out_f32 && !p.accumulate)
      store_tile_lds<MODE, false>(p, t, acc, wm, wn, lane, lds);
    else
      store_tile<MODE>(p, t, acc, wm, wn, lane);
  }
}

}  // namespace gemm

// MXFP8 forward: y = deq(xq) deq(wq)^T (+ b).  Codes travel as two-byte units, so
// the loads see K/2 units per row; K % 128 == 0 keeps every stage whole and the
// per-stage scale dwords aligned.
hipError_t launch_forward_mxfp8(int G, int64_t K, int64_t N, int64_t T, const uint8_t *xq, const uint8_t *xs,
                                const uint8_t *wq, const uint8_t *const *wq_ptrs, const uint8_t *ws_scale,
                                const uint8_t *const *ws_scale_ptrs, const void *bias,
                                const void *const *bias_ptrs, void *y, int out_f32, const void *ws,
                                hipStream_t s) {
  using namespace gemm;
  Params p{};
  p.A = (const uint16_t *)xq; p.lda = K / 2;
  p.B = (const uint16_t *)wq; p.B_ptrs = (const uint16_t *const *)wq_ptrs; p.b_gstride = N * K / 2; p.ldb = K / 2;
  p.C = y; p.ldc = N;
  p.bias = bias; p.bias_ptrs = bias_ptrs;
  p.ws = ws; p.G = G; p.T = T;
  p.cols_j = N; p.P = K / 2;
  p.tiles_j = (int)((N + kBN - 1) / kBN);
  p.out_f32 = out_f32;
  p.a_scale = xs; p.b_scale = ws_scale; p.b_scale_ptrs = ws_scale_ptrs; p.scale_ld = K / 32;
  const int64_t max_items = ((T + kBM - 1) / kBM + G) * p.tiles_j;
  hipLaunchKernelGGL(gemm_mxfp8_kernel<MODE_ROWS>, dim3(persistent_grid(max_items)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// MXFP8 wgrad: dW_g (+)= deq(dy_g)^T deq(x_g) from columnwise codes stored transposed,
// dyt [N, ld] and xt [K, ld] (group g's rows from column 128 * pre128[g], zero-padded
// to whole 128-row tiles), scales [N, ld/32] and [K, ld/32].  A[i=n][p] = dyt, B[j=k][p]
// = xt, both K-major.
hipError_t launch_wgrad_mxfp8(int G, int64_t K, int64_t N, int64_t T, const uint8_t *dyt, const uint8_t *dyt_s,
                              const uint8_t *xt, const uint8_t *xt_s, int64_t ld, void *dw, void *const *dw_ptrs,
                              int out_f32, int accumulate, const void *ws, hipStream_t s) {
  using namespace gemm;
  Params p{};
  p.A = (const uint16_t *)dyt; p.lda = ld / 2;
  p.B = (const uint16_t *)xt; p.ldb = ld / 2;
  p.C = dw; p.C_ptrs = dw_ptrs; p.c_gstride = N * K; p.ldc = K;
  p.ws = ws; p.G = G; p.T = T;
  p.rows_i = N; p.cols_j = K;
  p.tiles_i = (int)((N + kBM - 1) / kBM);
  p.tiles_j = (int)((K + kBN - 1) / kBN);
  p.accumulate = accumulate;
  p.out_f32 = out_f32;
  p.a_scale = dyt_s; p.b_scale = xt_s; p.scale_ld = ld / 32;
  const int64_t max_items = (int64_t)G * p.tiles_i * p.tiles_j;
  hipLaunchKernelGGL(gemm_mxfp8_kernel<MODE_KCONTR>, dim3(persistent_grid(max_items)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace gl
