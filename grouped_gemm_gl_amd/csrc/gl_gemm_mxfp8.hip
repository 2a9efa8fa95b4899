// Persistent grouped GEMM for the MXFP8 forward on gfx950: y = deq(xq) deq(wq)^T (+ b)
// with the scaled fp8 MFMA (v_mfma_scale_f32_16x16x128_f8f6f4), fp32 accumulation.
//
// The operands are the outputs of the MXFP8 group quantizer (page "Improve
// device-init grouped linear module with single grouped weight support", the
// grouped MXFP8 weight workspace; OCP MX E4M3 codes with one E8M0 scale per 32
// codes along K): codes xq [T, K] and wq [N, K] per group, scales [rows, K/32].
//
// Same tile machinery as the bf16 kernel (gl_gemm_tile.hpp): 256x256 outputs per
// workgroup, 8 waves of 128x64, a 2-stage LDS ring filled by direct buffer->LDS
// loads with the K-major layout.  Codes travel as 2-byte units, so a 128-byte stage
// row is 128 codes = 4 scale blocks = one 16x16x128 MFMA step.
//
// Scales: a stage needs each A and B row's 4 scale bytes (one dword).  They go
// straight into a small LDS area beside the ring, waves 0-3 loading the A rows',
// waves 4-7 the B rows': one 4-byte load per row per stage, or, in the wgrad when
// both scale tensors allow it (16-byte aligned rows), one 16-byte load per row for
// the dwords of four consecutive stages, two such chunks alternating.  The wgrad's
// short contractions make its per-stage costs weigh more, and there the chunks are
// measured 5% faster; in the forward they were not faster.  Each lane passes one
// byte of its row's dword to the MFMA: the instruction takes the scale of row r's
// block b from lane r + 16 b.
#include "gl_gemm_tile.hpp"

namespace gl {

namespace gemm {

// Scale loads of one tile row (a lane's row; rows past the tile's extent clamp).
struct ScaleStream {
  const char *base;  // scale row 0 of the tile, at the tile's first contraction dword
  uint32_t off;      // this lane's row offset

  template <bool UNIFORM>
  __device__ __forceinline__ void init(const uint8_t *rows, int64_t ld, int rv, int r) {
    base = UNIFORM ? uniform_ptr((const char *)rows) : (const char *)rows;
    off = (uint32_t)((int64_t)(r < rv ? r : rv - 1) * ld);
  }
  // dword t of the row
  __device__ __forceinline__ void issue4(int t, uint32_t *dst) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_at(base + 4 * t), (GL_LDS void *)dst, 4, off, 0, 0, 0);
  }
  // dwords 4c .. 4c + 3 of the row (16-byte aligned)
  __device__ __forceinline__ void issue16(int c, uint32_t *dst) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_at(base + 16 * c), (GL_LDS void *)dst, 16, off, 0, 0, 0);
  }
};

// 16x16x128 scaled-MFMA operand fragment of a 128-code K-major stage row.  Lane l
// holds row l % 16 and, in each 64-code half of the stage, the 16 codes at 16 (l /
// 16): the instruction works as two 16x16x64 halves, as the 32x32x64 form works as
// two 32x32x32 halves.
__device__ __forceinline__ i32x8_t frag16_mx(const char *st, int row0, int lane) {
  const int r = row0 + (lane & 15), g = lane >> 4;
  const i32x4_t lo = *(const i32x4_t *)(st + r * kRowB + ((g ^ swz_k(r)) << 4));
  const i32x4_t hi = *(const i32x4_t *)(st + r * kRowB + (((4 + g) ^ swz_k(r)) << 4));
  return (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// MODE_ROWS: forward (and dgrad on transposed columnwise weight codes);
// MODE_KCONTR: wgrad on transposed columnwise codes of dy and x.  S16: scales in
// 16-byte chunks of four stages.
template <int MODE, bool S16>
__global__ __launch_bounds__(kThreads) void gemm_mxfp8_kernel(Params p) {
  // One LDS object: the stage ring, then the scale area.  (A second __shared__
  // array makes the compiler wait for every outstanding direct-to-LDS load before
  // each LDS read.)  Scale area: 16-byte chunks [2][A, B][256 rows][4 dwords], or
  // per-stage dwords [kS][A, B][256 rows].
  constexpr int kScaleBytes = 2 * 2 * 256 * 16;
  __shared__ __attribute__((aligned(1024))) char lds[kS * kStageBytes + kScaleBytes];
  uint32_t(*sc16)[2][256][4] = (uint32_t(*)[2][256][4])(lds + kS * kStageBytes);
  uint32_t(*sc4)[2][256] = (uint32_t(*)[2][256])(lds + kS * kStageBytes);
  using L = AccLayout<Acc16>;

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
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  for (int w = first; w < total; w += grid) {
    const Tile t = decode_tile<true, true, MODE>(p, off, pre, w, cpre);
    if (!device_check(t.ok, p.ws)) continue;
    if (MODE == MODE_KCONTR && p.accumulate && t.g_rows == 0) continue;  // main_grad untouched
    // every stage is complete: K % 128 == 0 in row mode, padded groups otherwise
    const int nk = (int)(t.pmax / kBK);
    const int kbeg = 0, kend = nk;

    Stream<true> sa, sb;
    // row mode: the operand bases as visibly wave-uniform pointers (the weights' may
    // come from a pointer array; each stage's weight loads went through per-load
    // loops over distinct resource values).  The wgrad's bases are arguments plus
    // offsets, already uniform.
    sa.init(MODE == MODE_ROWS ? uniform_ptr(t.a_base) : t.a_base, p.lda, t.a_rv, wave, lane);
    sb.init(MODE == MODE_ROWS ? uniform_ptr(t.b_base) : t.b_base, p.ldb, t.b_rv, wave, lane);
    // scale rows from their 16-byte aligned start; stage s's dword is d0 + s of the
    // row (the group's scale columns start at 4 per padded 128-element tile)
    const int d0 = MODE == MODE_ROWS ? 0 : cpre[t.g];
    ScaleStream ss;
    if (MODE == MODE_ROWS) {
      if (wave < 4) {
        ss.template init<MODE == MODE_ROWS>(p.a_scale + (t.g_off + (int64_t)t.it * kBM) * p.scale_ld, p.scale_ld, t.a_rv, wave * 64 + lane);
      } else {
        const uint8_t *bs = p.b_scale ? p.b_scale + (int64_t)t.g * p.cols_j * p.scale_ld : p.b_scale_ptrs[t.g];
        ss.template init<MODE == MODE_ROWS>(bs + (int64_t)t.jt * kBN * p.scale_ld, p.scale_ld, t.b_rv, (wave - 4) * 64 + lane);
      }
    } else {
      if (wave < 4)
        ss.template init<MODE == MODE_ROWS>(p.a_scale + (int64_t)t.it * kBM * p.scale_ld, p.scale_ld, t.a_rv, wave * 64 + lane);
      else
        ss.template init<MODE == MODE_ROWS>(p.b_scale + (int64_t)t.jt * kBN * p.scale_ld, p.scale_ld, t.b_rv, (wave - 4) * 64 + lane);
    }
    auto stage_ptr = [&](int s) { return lds + (s % kS) * kStageBytes; };
    // operands of stage s, and its scales: with 16-byte chunks, the chunk holding
    // stage s when s starts a chunk or the tile (chunk c goes to buffer c % 2, whose
    // previous chunk ended at least four stages back)
    auto issue = [&](int s) {
      char *st = stage_ptr(s);
      sa.issue_full(s, st, wave);
      sb.issue_full(s, st + kOpBytes, wave);
      const int d = d0 + s;
      if (S16) {
        if (s == kbeg || (d & 3) == 0) ss.issue16(d >> 2, &sc16[(d >> 2) & 1][wave >> 2][(wave & 3) * 64][0]);
      } else {
        ss.issue4(d, &sc4[s % kS][wave >> 2][(wave & 3) * 64]);
      }
    };

    Acc16 acc;
    L::zero(acc);
    const int sh = 8 * (lane >> 4);  // the block this lane supplies the scale of
    auto stage = [&](int s) {
      // scale dwords of this lane's A and B rows, their byte for this lane lowest
      uint32_t sca[kNI16], scb[kNJ16];
      const int d = d0 + s;
#pragma unroll
      for (int ii = 0; ii < kNI16; ++ii) {
        const int r = wm * kWTM + ii * 16 + (lane & 15);
        sca[ii] = (S16 ? sc16[(d >> 2) & 1][0][r][d & 3] : sc4[s % kS][0][r]) >> sh;
      }
#pragma unroll
      for (int jj = 0; jj < kNJ16; ++jj) {
        const int r = wn * kWTN + jj * 16 + (lane & 15);
        scb[jj] = (S16 ? sc16[(d >> 2) & 1][1][r][d & 3] : sc4[s % kS][1][r]) >> sh;
      }
      const char *ta = stage_ptr(s), *tb = ta + kOpBytes;
      i32x8_t bfr[kNJ16];
#pragma unroll
      for (int jj = 0; jj < kNJ16; ++jj) bfr[jj] = frag16_mx(tb, wn * kWTN + jj * 16, lane);
      // the B fragments first, then the A fragments one at a time (32-byte fragments
      // leave no room for a second fragment set)
#pragma unroll
      for (int ii = 0; ii < kNI16; ++ii) {
        const i32x8_t af = frag16_mx(ta, wm * kWTM + ii * 16, lane);
#pragma unroll
        for (int jj = 0; jj < kNJ16; ++jj)
          acc[ii][jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[jj], af, acc[ii][jj], 0, 0, 0,
                                                                         (int)scb[jj], 0, (int)sca[ii]);
      }
    };

    if (kend > kbeg) {
      issue(kbeg);
      wait_vm0();
      __builtin_amdgcn_s_barrier();
    }
    for (int kt = kbeg; kt < kend; ++kt) {
      // the stage kt + 1 loads go into the slot stage kt - 1 used, freed by the
      // barrier that ended stage kt - 1
      if (kt + 1 < kend) issue(kt + 1);
      fence();
      stage(kt);
      fence();
      wait_vm0();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
    }
    // 16-bit outputs go out through LDS as whole lines (the ring is idle after the
    // loop; the scale area lies beyond it): the wgrad's short contractions make its
    // 1 GiB output the larger cost, and the forward and dgrad gain 1-2% too.  A
    // row-mode launch with a bias keeps the direct stores, which add it.
    if (!p.out_f32 && !p.accumulate && (MODE != MODE_ROWS || (!p.bias && !p.bias_ptrs)))
      store_tile_lds<MODE, false>(p, t, acc, wm, wn, lane, lds);
    else
      store_tile<MODE, false, MODE == MODE_ROWS>(p, t, acc, wm, wn, lane);
  }
}

// Both launched variants, instantiated explicitly: with only the launch sites to go
// by, the host pass has left a variant's launch stub undefined.
template __global__ void gemm_mxfp8_kernel<MODE_ROWS, false>(Params);
template __global__ void gemm_mxfp8_kernel<MODE_KCONTR, false>(Params);
template __global__ void gemm_mxfp8_kernel<MODE_KCONTR, true>(Params);

}  // namespace gemm

namespace {
bool aligned16_ptr(const void *q) { return ((uintptr_t)q & 15u) == 0; }
}  // namespace

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
  hipLaunchKernelGGL((gemm_mxfp8_kernel<MODE_ROWS, false>), dim3(persistent_grid(max_items)), dim3(kThreads), 0, s,
                     p);
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
  // both scale tensors 16-byte aligned with rows a multiple of 16 bytes long
  const bool s16 = (ld / 32) % 16 == 0 && aligned16_ptr(dyt_s) && aligned16_ptr(xt_s);
  const int64_t max_items = (int64_t)G * p.tiles_i * p.tiles_j;
  if (s16)
    hipLaunchKernelGGL((gemm_mxfp8_kernel<MODE_KCONTR, true>), dim3(persistent_grid(max_items)), dim3(kThreads), 0, s,
                       p);
  else
    hipLaunchKernelGGL((gemm_mxfp8_kernel<MODE_KCONTR, false>), dim3(persistent_grid(max_items)), dim3(kThreads), 0,
                       s, p);
  return hipGetLastError();
}

}  // namespace gl
