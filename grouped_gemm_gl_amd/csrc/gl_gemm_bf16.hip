// Persistent grouped GEMM for bf16 on gfx950 MFMA: forward, dgrad and wgrad.
//
// All three passes of the grouped linear layer (page
// "transformer_engine/pytorch/ops/basic/grouped_linear.py", fuser_forward "Perform
// GEMMs" and fuser_backward "Perform dgrad GEMMs" / "Perform wgrad GEMMs") are one
// contraction C[i][j] = sum_p A[i][p] * B[j][p] per group, differing only in which
// index is grouped and how the operands sit in memory:
//
//   forward  i = token row of group g, j = n, p = k:  A = x  (p contiguous), B = W_g (p contiguous)
//   dgrad    i = token row of group g, j = k, p = n:  A = dy (p contiguous), B = W_g (j contiguous)
//   wgrad    i = n, j = k, p = token row of group g:  A = dy (i contiguous), B = x   (j contiguous)
//
// Tiles: 256x256 outputs per workgroup, 8 waves (two per SIMD, which keeps the MFMA
// pipe fuller than one wave can) in a 2x4 grid, each wave a 128x64 block of
// 32x32x16 bf16 MFMAs with fp32 accumulators.
//
// Operand staging: the contraction advances kBK at a time through a ring of kS LDS
// stages filled by direct buffer->LDS loads (16 bytes per lane, no register
// staging).  An operand whose contraction index is contiguous ("K-major") is staged
// as 256 rows of 2*kBK bytes and read with 16-byte LDS loads; one whose tile index
// is contiguous ("MN-major") is staged as kBK rows of 512 bytes and read with the
// gfx950 LDS transpose load (ds_read_b64_tr_b16), which hands each lane 4
// consecutive contraction values of one column -- the MFMA operand layout -- so no
// operand is transposed in registers.  Both layouts XOR-swizzle 16-byte slots so
// fragment reads are free of bank conflicts on gfx950's 64-bank LDS.
//
// Loads: per lane the address of a piece is a fixed 32-bit offset from a
// wave-uniform tile base held in a buffer resource (scalar registers), so issuing a
// stage costs no vector arithmetic; the base advances by one stage per tile.
//
// Pipeline, per stage kt: the loads of stage kt + kS - 1 go out first, into the
// slot stage kt - 1 used; MFMA steps run while the fragments of the following step
// are read; before the last step every wave waits for its own loads of stage kt + 1
// and the workgroup meets at one barrier, after which the last step's MFMAs run
// while the first fragments of stage kt + 1 are read.
//
// Masking: rows past the valid extent of a K-major tile are clamped onto a valid
// row (their products land in output rows that are never stored); columns past an
// MN-major tile's extent are clamped likewise; contraction indices past the end
// (the last stage of a group in wgrad, or a contraction length not a multiple of
// kBK) are not loaded -- those lanes write zeros into their LDS slot instead.
//
// Scheduling: persistent grid, one workgroup per CU; workgroup b walks items b,
// b + grid, ...; items are remapped so each XCD (blockIdx % 8) works on a run of
// neighbouring tiles (8 x 4 blocks of output tiles) that share operand panels in
// its L2.  In row mode the item -> (group, row tile, column tile) map comes from
// the row-tile prefix table the offsets kernel left in the workspace.
#include "gl_gemm_tile.hpp"

namespace gl {

namespace gemm {

// F16: the operands are fp16 (v_mfma_f32_32x32x16_f16) instead of bf16; staging and
// fragments are the same 16-byte moves of 2-byte elements.
// BGRAD (wgrad only): the tiles of the first column also produce the bias gradient.
template <bool A_KMAJ, bool B_KMAJ, int MODE, bool F16, bool BGRAD = false>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(Params p) {
  // the stage ring; wgrad adds the bias-grad partial sums after it (one LDS object:
  // a second __shared__ array makes the compiler wait for the direct loads before
  // every LDS read)
  __shared__ __attribute__((aligned(1024))) char lds[kS * kStageBytes + (BGRAD ? kDbLdsBytes : 0)];

  const WsView ws = ws_view(p.ws, p.G);
  if (!ws_usable(ws.hdr, p.G, p.T)) return;
  const int64_t *__restrict__ off = ws.off;
  const int32_t *__restrict__ pre = ws.pre[tile_rows_index(kBM)];

  const int total = MODE == MODE_ROWS ? pre[p.G] * p.tiles_j : p.G * p.tiles_i * p.tiles_j;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int grid = gridDim.x, b = blockIdx.x;
  const int first = (grid & 7) == 0 ? (b & 7) * (grid >> 3) + (b >> 3) : b;
  const int nk_rows = (int)((p.P + kBK - 1) / kBK);  // row mode: the same for every tile

  // One work item: the whole contraction of a tile, or (SPLIT) part `part` of S of
  // the u-th split tile.  A wgrad tile of the first column, when a bias gradient is
  // asked for, also sums its dy stages into the bias gradient of its n range (a
  // uniform run-time switch: a second copy of the loop would cost registers).
  auto item = [&](int tile, int part, int S, int u, auto split_tag) __attribute__((always_inline)) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    const Tile t = decode_tile<A_KMAJ, B_KMAJ, MODE>(p, off, pre, tile);
    const bool bgrad = BGRAD && t.jt == 0;
    float *dbl = (float *)(lds + kS * kStageBytes);  // bias grad partials [kDbGroups][256 columns]
    if (MODE == MODE_CONTR && p.accumulate && t.g_rows == 0) {  // main_grad untouched
      if (bgrad) store_bgrad_zero(p, t);
      return;
    }
    if (bgrad) db_zero(dbl);
    const int64_t pmax = t.pmax;
    const int nk = (int)((pmax + kBK - 1) / kBK);
    const int nfull = (int)(pmax / kBK);  // stages [0, nfull) are complete; nk - nfull <= 1
    // this item's stages [kbeg, kend)
    const int kbeg = SPLIT ? part * nk / S : 0;
    const int kend = SPLIT ? (part + 1) * nk / S : nk;
    const int kfull = SPLIT ? (nfull < kend ? nfull : kend) : nfull;

    Stream<A_KMAJ> sa;
    Stream<B_KMAJ> sb;
    sa.init(t.a_base, p.lda, t.a_rv, wave, lane);
    sb.init(t.b_base, p.ldb, t.b_rv, wave, lane);
    auto stage_ptr = [&](int s) { return lds + (s % kS) * kStageBytes; };
    auto issue = [&](int s) {
      char *st = stage_ptr(s);
      if (s < nfull) {
        sa.issue_full(s, st, wave);
        sb.issue_full(s, st + kOpBytes, wave);
      } else {
        sa.issue_masked(s, pmax, st, wave, lane);
        sb.issue_masked(s, pmax, st + kOpBytes, wave, lane);
      }
    };

    // -------------------------------------------------------------- main loop
    f32x16_t acc[kNI][kNJ];
#pragma unroll
    for (int ii = 0; ii < kNI; ++ii)
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[ii][jj][q] = 0.f;

    auto load_frags = [&](int s, int ks, bf16x8_t *af, bf16x8_t *bfr) {
      const char *ta = stage_ptr(s);
      const char *tb = ta + kOpBytes;
#pragma unroll
      for (int ii = 0; ii < kNI; ++ii)
        af[ii] = A_KMAJ ? frag_kmaj(ta, wm * kWTM + ii * 32, ks, lane) : frag_mnmaj(ta, wm * kWTM + ii * 32, ks, lane);
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj)
        bfr[jj] = B_KMAJ ? frag_kmaj(tb, wn * kWTN + jj * 32, ks, lane) : frag_mnmaj(tb, wn * kWTN + jj * 32, ks, lane);
    };
    auto mfmas = [&](const bf16x8_t *af, const bf16x8_t *bfr) {
      // operands swapped so each lane ends up with 4 consecutive output columns
#pragma unroll
      for (int ii = 0; ii < kNI; ++ii)
#pragma unroll
        for (int jj = 0; jj < kNJ; ++jj)
          acc[ii][jj] = F16 ? __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, bfr[jj]),
                                                                    __builtin_bit_cast(f16x8_t, af[ii]), acc[ii][jj],
                                                                    0, 0, 0)
                            : __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[jj], af[ii], acc[ii][jj], 0, 0, 0);
    };

    bf16x8_t fa[2][kNI], fb[2][kNJ];
    // prologue: stages kbeg .. kbeg+kS-2 in flight, stage kbeg visible, its step 0
    // fragments read
    for (int s = kbeg; s < kbeg + kS - 1 && s < kend; ++s) issue(s);
    if (kend > kbeg) {
      wait_vm0();
      __builtin_amdgcn_s_barrier();
      load_frags(kbeg, 0, fa[0], fb[0]);
    }
    // One stage per iteration; fragment set (ks & 1) feeds MFMA step ks while set
    // (ks + 1) & 1 is refilled.  The barrier before the last step makes stage kt + 1
    // visible and frees the slot stage kt used, which the next iteration refills.
    static_assert((kKS & 1) == 0, "step 0 of every stage must read fragment set 0");
    // Scheduling fences keep the order written here: the next step's fragment reads
    // go out before the current step's MFMAs, so each read has a whole block of
    // MFMAs to complete in.
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    auto body = [&](int kt, bool steady) {
      if (steady) {
        char *st = stage_ptr(kt + kS - 1);
        sa.issue_full(kt + kS - 1, st, wave);
        sb.issue_full(kt + kS - 1, st + kOpBytes, wave);
      } else if (kt + kS - 1 < kend) {
        issue(kt + kS - 1);
      }
      fence();
#pragma unroll
      for (int ks = 0; ks < kKS - 1; ++ks) {
        load_frags(kt, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
        fence();
        mfmas(fa[ks & 1], fb[ks & 1]);
        fence();
      }
      // stage kt stays in its slot until the barrier below
      if (BGRAD && bgrad) db_stage<F16>(stage_ptr(kt), dbl);
      // stage kt + 1 complete: at most the loads of stages kt + 2 .. kt + kS - 1
      // may still be in flight
      if (steady)
        wait_vm<(kS - 2) * kLoadsPerStage>();
      else
        wait_vm0();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      if (steady || kt + 1 < kend) load_frags(kt + 1, 0, fa[0], fb[0]);
      fence();
      mfmas(fa[(kKS - 1) & 1], fb[(kKS - 1) & 1]);
      fence();
    };

    int kt = kbeg;
    for (; kt + kS - 1 < kfull; ++kt) body(kt, true);  // every stage issued here is complete
    for (; kt < kend; ++kt) body(kt, false);
    __builtin_amdgcn_s_barrier();  // every wave is done with the ring before it is refilled

    if constexpr (SPLIT) {
      // the ring is idle after the loop's last barrier: its first word carries the flag
      if (!split_finish(ws, u, part, S, acc, (int *)lds)) return;
    }
    if (BGRAD && bgrad) store_bgrad<F16>(p, t, dbl);
    // wgrad tiles contract over one group's rows only, so their output stores weigh
    // more: there the tile goes out through LDS as whole lines (measured neutral to
    // slightly worse for forward and dgrad, which keep the direct stores)
    if (MODE != MODE_ROWS && !p.out_f32 && !p.accumulate)
      store_tile_lds<MODE, F16>(p, t, acc, wm, wn, lane, lds);
    else
      store_tile<MODE, F16>(p, t, acc, wm, wn, lane);
  };

  // whole tiles, round after round; in row mode the last round may be split
  const int full = MODE == MODE_ROWS ? split_plan(total, grid, nk_rows).full : total;
  for (int w = first; w < full; w += grid) item(w, 0, 1, 0, std::false_type{});
  if constexpr (MODE == MODE_ROWS) {
    const int tiles = pre[p.G] * p.tiles_j;
    const SplitPlan sp = split_plan(tiles, grid, nk_rows);
    // the parts of the last round: u = first, consecutive u are consecutive tiles
    if (first < sp.rem * sp.S)
      item(sp.full + first % sp.rem, first / sp.rem, sp.S, first % sp.rem, std::true_type{});
  }
}

}  // namespace gemm

// forward: y = x W^T (+ b); A = x [T,K], B = W [N,K]
hipError_t launch_forward_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *x, const uint16_t *w,
                               const uint16_t *const *w_ptrs, const void *bias, const void *const *bias_ptrs,
                               uint16_t *y, int f16, const void *ws, hipStream_t s) {
  using namespace gemm;
  Params p{};
  p.A = x; p.lda = K;
  p.B = w; p.B_ptrs = w_ptrs; p.b_gstride = N * K; p.ldb = K;
  p.C = y; p.ldc = N;
  p.bias = bias; p.bias_ptrs = bias_ptrs;
  p.ws = ws; p.G = G; p.T = T;
  p.cols_j = N; p.P = K;
  p.tiles_j = (int)((N + kBN - 1) / kBN);
  const int64_t max_items = ((T + kBM - 1) / kBM + G) * p.tiles_j;
  if (f16)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, MODE_ROWS, true>), dim3(persistent_grid(max_items)),
                       dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, MODE_ROWS, false>), dim3(persistent_grid(max_items)),
                       dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// dgrad: dx = dy W; A = dy [T,N] (n contiguous), B[j=k][p=n] = W[n][k] (k contiguous)
hipError_t launch_dgrad_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *dy, const uint16_t *w,
                             const uint16_t *const *w_ptrs, uint16_t *dx, int f16, const void *ws, hipStream_t s) {
  using namespace gemm;
  Params p{};
  p.A = dy; p.lda = N;
  p.B = w; p.B_ptrs = w_ptrs; p.b_gstride = N * K; p.ldb = K;
  p.C = dx; p.ldc = K;
  p.ws = ws; p.G = G; p.T = T;
  p.cols_j = K; p.P = N;
  p.tiles_j = (int)((K + kBN - 1) / kBN);
  const int64_t max_items = ((T + kBM - 1) / kBM + G) * p.tiles_j;
  if (f16)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, false, MODE_ROWS, true>), dim3(persistent_grid(max_items)),
                       dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<true, false, MODE_ROWS, false>), dim3(persistent_grid(max_items)),
                       dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// wgrad: dW_g[n][k] = sum_r dy[r][n] x[r][k]; A[i=n][p=r] (n contiguous), B[j=k][p=r] (k contiguous)
hipError_t launch_wgrad_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *x, const uint16_t *dy,
                             void *dw, void *const *dw_ptrs, int out_f32, int accumulate, int f16, void *db,
                             void *const *db_ptrs, int db_f32, const void *ws, hipStream_t s) {
  using namespace gemm;
  Params p{};
  p.A = dy; p.lda = N;
  p.B = x; p.ldb = K;
  p.C = dw; p.C_ptrs = dw_ptrs; p.c_gstride = N * K; p.ldc = K;
  p.ws = ws; p.G = G; p.T = T;
  p.rows_i = N; p.cols_j = K;
  p.tiles_i = (int)((N + kBM - 1) / kBM);
  p.tiles_j = (int)((K + kBN - 1) / kBN);
  p.accumulate = accumulate;
  p.out_f32 = out_f32;
  p.db = db; p.db_ptrs = db_ptrs; p.db_f32 = db_f32;
  const int64_t max_items = (int64_t)G * p.tiles_i * p.tiles_j;
  const dim3 grid(persistent_grid(max_items)), block(kThreads);
  const bool bg = db || db_ptrs;
  if (f16 && bg)
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, MODE_CONTR, true, true>), grid, block, 0, s, p);
  else if (f16)
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, MODE_CONTR, true>), grid, block, 0, s, p);
  else if (bg)
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, MODE_CONTR, false, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, MODE_CONTR, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace gl
