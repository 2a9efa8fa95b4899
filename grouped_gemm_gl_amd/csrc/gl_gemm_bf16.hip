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
// Tiles: 256x256 outputs per workgroup, 8 waves (two per SIMD) in a 2x4 grid, each
// wave a 128x64 block with fp32 accumulators.
//
// Operand staging: the contraction advances kBK = 64 at a time through a ring of two
// LDS stages.  An operand whose contraction index is contiguous ("K-major") is staged
// as 256 rows of 128 bytes and read with 16-byte LDS loads; one whose tile index is
// contiguous ("MN-major") is staged as 64 rows of 512 bytes and read with the gfx950
// LDS transpose load (ds_read_b64_tr_b16), which hands each lane consecutive
// contraction values of one column -- the MFMA operand layout -- so no operand is
// transposed in registers.  Both layouts XOR-swizzle 16-byte slots so fragment reads
// are free of bank conflicts on gfx950's 64-bank LDS.
//
// Ping-pong: the two waves of a SIMD (wm = 0 and 1) run the same phase sequence --
// read a 32-deep step of fragments from LDS, barrier, that step's MFMAs, barrier --
// but the wm = 1 waves start one barrier later.  So while one wave of each SIMD
// issues MFMAs, the other reads LDS, and the MFMA pipe of each SIMD is fed by one
// wave at a time.  Four phases per stage, one workgroup barrier after each.
//
// Two schedules of the same loop:
//   DIRECT (forward): direct buffer->LDS loads (16 bytes per lane, no VGPRs) of stage
//     kt + 1 issued at the start of stage kt; 16x16x32 MFMAs.  These GEMMs run at
//     the chip's power limit, and the 16x16x32 MFMA does the same work as the
//     32x32x16 one for less energy (at the same throughput per clock), which lets the
//     engine clock stay higher.  DIRECT_DEEP, for groups of at most 256 rows on
//     average: the weights' loads run two stages ahead, from a third weight slot
//     (the ring then fills the 160 KiB LDS), since there every weight byte comes
//     from HBM once and latency, not L2 traffic, bounds the loop.
//   STAGED (dgrad, wgrad): loads go global -> VGPR and are written to the ring by the
//     waves themselves, in the middle of a compute phase, a stage later; the loads of
//     stage kt + 2 go out in the read phase after stage kt + 1 is written, and the
//     direct-load return path no longer competes with the transpose reads for LDS.
//     32x32x16 MFMAs (two 16-deep steps per phase).  The wgrad tiles of one column
//     per group (column g mod the column count) also add their dy stages into the
//     bias gradient from the staging registers, before each stage is written to the
//     ring.
//
// Loads: per lane the address of a piece is a fixed 32-bit offset from a
// wave-uniform tile base held in a buffer resource (scalar registers), so issuing a
// stage costs no vector arithmetic; the base advances by one stage per tile.
//
// Masking: rows past the valid extent of a K-major tile are clamped onto a valid
// row (their products land in output rows that are never stored); columns past an
// MN-major tile's extent are clamped likewise; contraction indices past the end
// (the last stage of a group in wgrad, or a contraction length not a multiple of
// kBK) are not loaded -- those lanes put zeros into their LDS slot instead.
//
// Scheduling: persistent grid, one workgroup per CU; workgroup b walks items b,
// b + grid, ...; items are remapped so each XCD (blockIdx % 8) works on a run of
// neighbouring tiles (8 x 4 blocks of output tiles) that share operand panels in
// its L2.  In row mode the item -> (group, row tile, column tile) map comes from
// the row-tile prefix table the offsets kernel left in the workspace.
#include "gl_gemm_tile.hpp"

namespace gl {

namespace gemm {

// SCHED_DIRECT_DEEP: the direct-load schedule with the weights two stages ahead
// (three weight slots in the ring), for small groups whose weights stream from HBM.
enum { SCHED_DIRECT = 0, SCHED_STAGED = 1, SCHED_DIRECT_DEEP = 2 };

// F16: the operands are fp16 instead of bf16; staging and fragments are the same
// 16-byte moves of 2-byte elements.
// BGRAD (wgrad, STAGED only): the tiles of one column per group also produce the
// bias gradient.
template <bool A_KMAJ, bool B_KMAJ, int MODE, bool F16, int SCHED, bool BGRAD = false>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(Params p) {
  static_assert(!BGRAD || SCHED == SCHED_STAGED, "the bias-grad fusion runs on the staged schedule");
  constexpr bool DIRECT = SCHED != SCHED_STAGED;
  constexpr int kLeadB = SCHED == SCHED_DIRECT_DEEP ? 2 : 1;  // stages the weight loads run ahead
  using ACC = typename std::conditional<DIRECT, Acc16, Acc32>::type;
  using L = AccLayout<ACC>;
  // the stage ring; wgrad adds the bias-grad partial sums after it (one LDS object:
  // a second __shared__ array makes the compiler wait for the direct loads before
  // every LDS read)
  // The forward on the two-slot weight ring keeps each tile's 256 bias values in LDS
  // beside the ring (two 512-byte buffers, alternating by tile), loaded with the
  // tile's first stage: read from global memory in the epilogue, each tile waited
  // for them there.
  constexpr bool kBiasLds = DIRECT && kLeadB == 1;
  constexpr int kBiasBytes = kBN * 2;
  __shared__ __attribute__((aligned(1024)))
  char lds[DIRECT ? (2 + kLeadB + 1) * kOpBytes + (kBiasLds ? 2 * kBiasBytes : 0)
                  : kS * kStageBytes + (BGRAD ? kDbLdsBytes : 0)];
  int ntile = 0;  // items begun by this workgroup (the bias buffer's parity)

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
  const int slots = min(max(ws.hdr->split_slots, 0), kSplitSlots);
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  auto barrier = [&] {
    __builtin_amdgcn_s_barrier();
    fence();
  };

  // One work item: the whole contraction of tile t, or (SPLIT) part `part` of S of
  // the u-th split tile, whose partials go to slots slot0 .. slot0 + S - 1.  The
  // bias-grad tag marks a tile of a group's bias-grad column in a BGRAD launch: its loop is a
  // copy of its own, so the other tiles run the plain loop (its registers and code).
  auto item = [&](const Tile &t, int part, int S, int u, int slot0, auto split_tag,
                  auto bgrad_tag) __attribute__((always_inline)) {
    constexpr bool SPLIT = decltype(split_tag)::value;
    if (!device_check(t.ok && (!SPLIT || (part >= 0 && part < S && slot0 >= 0 && slot0 + S <= slots)), p.ws))
      return;
    constexpr bool bgrad = BGRAD && decltype(bgrad_tag)::value;
    if (MODE == MODE_CONTR && p.accumulate && t.g_rows == 0) {  // main_grad untouched
      if (bgrad) store_bgrad_zero(p, t);
      return;
    }
    const int64_t pmax = t.pmax;
    const int nk = (int)((pmax + kBK - 1) / kBK);
    const int nfull = (int)(pmax / kBK);  // stages [0, nfull) are complete; nk - nfull <= 1
    // this item's stages [kbeg, kend)
    const int kbeg = SPLIT ? part * nk / S : 0;
    const int kend = SPLIT ? (part + 1) * nk / S : nk;
    const int kfull = SPLIT ? (nfull < kend ? nfull : kend) : nfull;

    Stream<A_KMAJ> sa;
    Stream<B_KMAJ> sb;
    const char *bias_l = nullptr;  // this tile's bias in LDS (kBiasLds, when the launch has a bias)
    // the deep ring's operand bases as visibly wave-uniform pointers (its stage loads
    // otherwise went through per-load loops over distinct resource values)
    constexpr bool kUniformBases = SCHED == SCHED_DIRECT_DEEP;
    sa.init(kUniformBases ? uniform_ptr(t.a_base) : t.a_base, p.lda, t.a_rv, wave, lane);
    sb.init(kUniformBases ? uniform_ptr(t.b_base) : t.b_base, p.ldb, t.b_rv, wave, lane);
    auto stage_ptr = [&](int s) { return lds + (s % kS) * kStageBytes; };

    ACC acc;
    L::zero(acc);
    const int h = wm;  // ping-pong group
    // this lane's bias-grad column sums (STAGED), in LDS beside the ring
    float *dbs = db_slot((float *)(lds + kS * kStageBytes), wave, lane);
    if (BGRAD && bgrad) db_zero(dbs);

    if constexpr (DIRECT) {
      // A (the activations) in two slots, B (the weights) in kLeadB + 1: while stage
      // kt is computed, A stage kt + 1 and B stage kt + kLeadB are in flight (with
      // kLeadB = 2, each weight stage has two stages' time to arrive from HBM).
      auto a_ptr = [&](int s) { return lds + (s & 1) * kOpBytes; };
      auto b_ptr = [&](int s) { return lds + (2 + s % (kLeadB + 1)) * kOpBytes; };
      auto issue_a = [&](int s) {
        if (s < nfull) sa.issue_full(s, a_ptr(s), wave);
        else sa.issue_masked(s, pmax, a_ptr(s), wave, lane);
      };
      auto issue_b = [&](int s) {
        if (s < nfull) sb.issue_full(s, b_ptr(s), wave);
        else sb.issue_masked(s, pmax, b_ptr(s), wave, lane);
      };
      // 16-row blocks of this wave that hold valid rows (a group's last row tile is
      // often part padding): the others skip their fragment reads and MFMAs, which
      // saves power as well as LDS bandwidth.  Wave-uniform.
      const int vb = MODE == MODE_ROWS ? min(max((t.a_rv - wm * kWTM + 15) / 16, 0), kNI16) : kNI16;
      bf16x8_t fa[kNI16], fb[kNJ16];
      auto read_step = [&](int s, int ks) {
        if (vb == 0) return;
        const char *ta = a_ptr(s);
        const char *tb = b_ptr(s);
#pragma unroll
        for (int ii = 0; ii < kNI16; ++ii)
          if (ii < vb)
            fa[ii] = A_KMAJ ? frag16_kmaj(ta, wm * kWTM + ii * 16, ks, lane)
                            : frag16_mnmaj(ta, wm * kWTM + ii * 16, ks, lane);
#pragma unroll
        for (int jj = 0; jj < kNJ16; ++jj)
          fb[jj] = B_KMAJ ? frag16_kmaj(tb, wn * kWTN + jj * 16, ks, lane)
                          : frag16_mnmaj(tb, wn * kWTN + jj * 16, ks, lane);
      };
      auto compute_step = [&]() {
#pragma unroll
        for (int ii = 0; ii < kNI16; ++ii)
          if (ii < vb) {
#pragma unroll
            for (int jj = 0; jj < kNJ16; ++jj)
              acc[ii][jj] = F16 ? __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, fb[jj]),
                                                                        __builtin_bit_cast(f16x8_t, fa[ii]),
                                                                        acc[ii][jj], 0, 0, 0)
                                : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[jj], fa[ii], acc[ii][jj], 0, 0, 0);
          }
      };
      static_assert(kBK == 64, "two 32-deep steps per stage");
      // Waits: a full stage is kQ loads per wave and the loads complete in order, so
      // with kLeadB = 2, vmcnt(kQ) after A kt + 1 and B kt + 2 were sent leaves just
      // B kt + 2 in flight.  A masked stage may send fewer: then everything is waited
      // for.
      if (kend > kbeg) {
        if (kBiasLds) {
          // wave 0: the tile's bias columns (past the last column: zeros), 16 bytes per
          // lane of its first half; waited for with the first stage
          char *const buf = lds + (2 + kLeadB + 1) * kOpBytes + (ntile++ & 1) * kBiasBytes;
          const char *brow = p.bias ? (const char *)p.bias + (int64_t)t.g * p.cols_j * 2
                                    : p.bias_ptrs ? (const char *)p.bias_ptrs[t.g] : nullptr;
          bias_l = brow ? buf : nullptr;  // null: no bias
          if (brow && wave == 0 && lane < kBiasBytes / 16) {
            const int64_t c0 = (int64_t)t.jt * kBN;
            const __amdgpu_buffer_rsrc_t r =
                __builtin_amdgcn_make_buffer_rsrc((void *)(brow + c0 * 2), (short)0, t.b_rv * 2, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (GL_LDS void *)buf, 16, lane * 16, 0, 0, 0);
          }
        }
        issue_a(kbeg);
        issue_b(kbeg);
        if (kLeadB == 2 && kbeg + 1 < kend) issue_b(kbeg + 1);
        if (kLeadB == 2 && kbeg + 1 < kfull) wait_vm<kQ>();
        else wait_vm0();
        barrier();
      }
      if (h == 1) barrier();
      auto body = [&](int kt, bool steady) {
        if (steady) {
          sa.issue_full(kt + 1, a_ptr(kt + 1), wave);
          sb.issue_full(kt + kLeadB, b_ptr(kt + kLeadB), wave);
        } else {
          if (kt + 1 < kend) issue_a(kt + 1);
          if (kt + kLeadB < kend) issue_b(kt + kLeadB);
        }
        fence();
        read_step(kt, 0);
        wait_lgkm0();
        fence();
        barrier();
        compute_step();
        fence();
        barrier();
        read_step(kt, 1);
        wait_lgkm0();
        fence();
        // stage kt + 1 complete before the barrier after which group 0 reads it
        if (kLeadB == 2 && steady) wait_vm<kQ>();
        else wait_vm0();
        barrier();
        compute_step();
        fence();
        barrier();
      };
      int kt = kbeg;
      for (; kt + kLeadB < kfull; ++kt) body(kt, true);  // the stages issued here are complete
      for (; kt < kend; ++kt) body(kt, false);
    } else {
      uint4 ra[kQ], rb[kQ];
      auto load_stage = [&](int st_, bool full) {
        if (full) {
          sa.load_regs(st_, ra);
          sb.load_regs(st_, rb);
        } else {
          sa.load_regs_masked(st_, pmax, ra, wave, lane);
          sb.load_regs_masked(st_, pmax, rb, wave, lane);
        }
      };
      auto write_stage = [&](int st_) {
        char *st = stage_ptr(st_);
        sa.write_regs(st, ra, wave, lane);
        sb.write_regs(st + kOpBytes, rb, wave, lane);
      };
      constexpr int kH = kKS / 2;  // 16-deep steps per phase
      bf16x8_t fa[kH][kNI], fb[kH][kNJ];
      auto read_half = [&](int s, int half) {
        const char *ta = stage_ptr(s);
        const char *tb = ta + kOpBytes;
#pragma unroll
        for (int ks = 0; ks < kH; ++ks) {
#pragma unroll
          for (int ii = 0; ii < kNI; ++ii)
            fa[ks][ii] = A_KMAJ ? frag_kmaj(ta, wm * kWTM + ii * 32, half * kH + ks, lane)
                                : frag_mnmaj(ta, wm * kWTM + ii * 32, half * kH + ks, lane);
#pragma unroll
          for (int jj = 0; jj < kNJ; ++jj)
            fb[ks][jj] = B_KMAJ ? frag_kmaj(tb, wn * kWTN + jj * 32, half * kH + ks, lane)
                                : frag_mnmaj(tb, wn * kWTN + jj * 32, half * kH + ks, lane);
        }
      };
      auto compute = [&](int ks) {
#pragma unroll
        for (int ii = 0; ii < kNI; ++ii)
#pragma unroll
          for (int jj = 0; jj < kNJ; ++jj)
            acc[ii][jj] = F16 ? __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, fb[ks][jj]),
                                                                      __builtin_bit_cast(f16x8_t, fa[ks][ii]),
                                                                      acc[ii][jj], 0, 0, 0)
                              : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][jj], fa[ks][ii], acc[ii][jj], 0,
                                                                        0, 0);
      };
      static_assert(kH == 2, "two 16-deep steps per phase");
      if (kend > kbeg) {
        load_stage(kbeg, kbeg < nfull);
        wait_vm0();
        if (BGRAD && bgrad) db_add<F16>(dbs, ra);
        write_stage(kbeg);
        if (kbeg + 1 < kend) load_stage(kbeg + 1, kbeg + 1 < nfull);
        wait_lgkm0();
        barrier();
      }
      if (h == 1) barrier();
      // Per stage kt, four phases per wave: read the first half stage (and add the
      // stage's rows into the bias gradient); its MFMAs, with the ring writes of
      // stage kt + 1 between the two steps; read the second half and send the loads
      // of stage kt + 2; its MFMAs.
      auto body = [&](int kt, bool steady) {
        read_half(kt, 0);
        wait_lgkm0();
        fence();
        barrier();
        compute(0);
        fence();
        if (steady || kt + 1 < kend) {
          wait_vm0();
          if (BGRAD && bgrad) db_add<F16>(dbs, ra);  // dy rows of stage kt + 1
          write_stage(kt + 1);
        }
        fence();
        compute(1);
        fence();
        wait_lgkm0();
        barrier();
        read_half(kt, 1);
        fence();
        if (steady)
          load_stage(kt + 2, true);
        else if (kt + 2 < kend)
          load_stage(kt + 2, kt + 2 < nfull);
        fence();
        wait_lgkm0();
        barrier();
        compute(0);
        compute(1);
        fence();
        barrier();
      };
      int kt = kbeg;
      for (; kt + 2 < kfull; ++kt) body(kt, true);  // stages kt + 1 and kt + 2 are complete
      for (; kt < kend; ++kt) body(kt, false);
    }
    if (h == 0) barrier();
    __builtin_amdgcn_s_barrier();  // every wave is done with the ring before it is refilled

    // the tile's bias-grad column sums (thread t < 256: column t)
    float dbv = 0.f;
    if (BGRAD && bgrad) dbv = db_reduce((const float *)(lds + kS * kStageBytes));
    if constexpr (SPLIT) {
      // a part of a bias-grad tile leaves its column sums beside its partial tile
      GL_GLOBAL float *dbp = (GL_GLOBAL float *)ws.db_part;
      if (BGRAD && bgrad && threadIdx.x < 256) dbp[(slot0 + part) * 256 + threadIdx.x] = dbv;
      // the ring is idle after the loop's last barrier: its first word carries the flag
      if (!split_finish(ws, u, slot0, part, S, acc, (int *)lds)) return;
      if (BGRAD && bgrad && threadIdx.x < 256) {
        dbv = 0.f;
        for (int s_ = 0; s_ < S; ++s_) dbv += dbp[(slot0 + s_) * 256 + threadIdx.x];
      }
    }
    if (BGRAD && bgrad) store_bgrad<F16>(p, t, dbv);
    // Tiles of the register-staged schedule (dgrad, wgrad) with a 16-bit output go out
    // through LDS as whole lines (64-group dgrad -2.4%, 8-group dgrad neutral, wgrads
    // faster); the forward keeps its direct stores, which add its bias.
    if ((!DIRECT || kBiasLds) && !p.out_f32 && !p.accumulate)
      store_tile_lds<MODE, F16>(p, t, acc, wm, wn, lane, lds, bias_l);
    else
      store_tile<MODE, F16, A_KMAJ && B_KMAJ>(p, t, acc, wm, wn, lane, bias_l);  // the forward takes a bias
  };

  if constexpr (MODE == MODE_ROWS) {
    // whole tiles, round after round; the last round may be split
    const SplitPlan sp = split_plan(total, grid, nk_rows, slots);
    for (int w = first; w < sp.full; w += grid)
      item(decode_tile<A_KMAJ, B_KMAJ, MODE>(p, off, pre, w), 0, 1, 0, 0, std::false_type{}, std::false_type{});
    // the parts of the last round: u = first, consecutive u are consecutive tiles
    if (first < sp.rem * sp.S) {
      const int u = first % sp.rem;
      item(decode_tile<A_KMAJ, B_KMAJ, MODE>(p, off, pre, sp.full + u), first / sp.rem, sp.S, u, u * sp.S,
           std::true_type{}, std::false_type{});
    }
  } else {
    // the contraction schedule of the plan kernel: work items in order of decreasing
    // contraction length, the tiles of the longest groups cut into parts of at most
    // `cap` stages (parts first, part-major, so the tiles of one part run side by
    // side and share their rows in L2); the grid walks the list in snake order
    // (round r in reverse when r is odd), which evens out what each CU gets
    const int ntiles = p.tiles_i * p.tiles_j;
    const int cap = ws.plan[0];
    const int nitems = ws.items[p.G];
    const int32_t *__restrict__ stg = ws.pre[tile_rows_index(kBK)];
    for (int base = 0; base < nitems; base += grid) {
      const int w = base + (((base / grid) & 1) ? grid - 1 - first : first);
      if (w >= nitems) continue;
      const int pos = find_group(ws.items, p.G, w);
      if (!device_check(pos >= 0 && pos < p.G, p.ws)) continue;
      const int g = ws.order[pos];
      if (!device_check(g >= 0 && g < p.G, p.ws)) continue;
      const int sg = stg[g + 1] - stg[g];
      const int pg = sg > cap ? (sg + cap - 1) / cap : 1;
      const int local = w - ws.items[pos];
      const int part = local / ntiles, tl = local - part * ntiles;
      if (!device_check(local >= 0 && part < pg, p.ws)) continue;
      const Tile t = decode_tile<A_KMAJ, B_KMAJ, MODE>(p, off, pre, g * ntiles + tl);
      auto run = [&](auto bgrad_tag) __attribute__((always_inline)) {
        if (pg > 1)
          item(t, part, pg, pos * ntiles + tl, ws.items[pos] + tl * pg, std::true_type{}, bgrad_tag);
        else
          item(t, 0, 1, 0, 0, std::false_type{}, bgrad_tag);
      };
      if constexpr (BGRAD) {
        // Any tile of a row block streams the same dy columns, so the bias grad may come
        // from any column: group g takes column g mod tiles_j, which spreads these
        // slower tiles over the grid (8-group workload: at most 2 per CU instead of 4;
        // the sums and their order are the same in every column).
        if (t.jt == t.g % p.tiles_j) run(std::true_type{});
        else run(std::false_type{});
      } else {
        run(std::false_type{});
      }
    }
  }
}

// Every launched variant, instantiated explicitly: with only the launch sites to go
// by, the host pass has left a variant's launch stub undefined.
template __global__ void gemm_bf16_kernel<true, true, MODE_ROWS, false, SCHED_DIRECT>(Params);
template __global__ void gemm_bf16_kernel<true, true, MODE_ROWS, true, SCHED_DIRECT>(Params);
template __global__ void gemm_bf16_kernel<true, true, MODE_ROWS, false, SCHED_DIRECT_DEEP>(Params);
template __global__ void gemm_bf16_kernel<true, true, MODE_ROWS, true, SCHED_DIRECT_DEEP>(Params);
template __global__ void gemm_bf16_kernel<true, false, MODE_ROWS, false, SCHED_STAGED>(Params);
template __global__ void gemm_bf16_kernel<true, false, MODE_ROWS, true, SCHED_STAGED>(Params);
template __global__ void gemm_bf16_kernel<false, false, MODE_CONTR, false, SCHED_STAGED>(Params);
template __global__ void gemm_bf16_kernel<false, false, MODE_CONTR, true, SCHED_STAGED>(Params);
template __global__ void gemm_bf16_kernel<false, false, MODE_CONTR, false, SCHED_STAGED, true>(Params);
template __global__ void gemm_bf16_kernel<false, false, MODE_CONTR, true, SCHED_STAGED, true>(Params);

// The contraction schedule of a wgrad launch (one workgroup, before the GEMM): the
// groups in order of decreasing stage count s_g = ceil(m_g / kBK) (ties by index),
// and a cap on the stages of one work item -- two thirds of the average stage count
// per CU, raised until the split parts fit the partial slots -- above which a
// group's tiles are cut into ceil(s_g / cap) parts; items[] is the prefix of work
// items (tiles x parts) over that order.  Splitting is off (cap = INT_MAX) when
// `split` is 0 or there are more than kPlanThreads groups (then the order is the
// group order).
constexpr int kPlanThreads = 1024;
__global__ __launch_bounds__(kPlanThreads) void contr_plan_kernel(void *ws_, int G, int64_t T, int ntiles, int grid,
                                                                  int split) {
  const WsView ws = ws_view(ws_, G);
  if (!ws_usable(ws.hdr, G, T)) return;
  const int32_t *__restrict__ stg = ws.pre[tile_rows_index(kBK)];
  const int tid = threadIdx.x;
  if (G > kPlanThreads) {
    for (int g = tid; g <= G; g += kPlanThreads) {
      if (g < G) ws.order[g] = g;
      ws.items[g] = g * ntiles;
    }
    if (tid == 0) {
      ws.plan[0] = INT32_MAX;
      ws.plan[1] = 0;
    }
    return;
  }
  __shared__ int32_t sz[kPlanThreads], cnt[kPlanThreads];
  __shared__ int32_t s_cap;
  const int sg = tid < G ? stg[tid + 1] - stg[tid] : -1;
  sz[tid] = sg;
  __syncthreads();
  if (tid == 0) {
    const int slots = min(max(ws.hdr->split_slots, 0), kSplitSlots);
    const int64_t avg = ((int64_t)stg[G] * ntiles + grid - 1) / grid;
    int cap = INT32_MAX;
    if (split) {
      cap = (int)max((int64_t)kMinSplitStages, (2 * avg + 2) / 3);
      for (;;) {  // parts of the split tiles must fit the partial slots
        int64_t need = 0;
        for (int g = 0; g < G; ++g)
          if (sz[g] > cap) need += (int64_t)ntiles * ((sz[g] + cap - 1) / cap);
        if (need <= slots || cap >= (1 << 28)) break;
        cap += cap / 4 + 1;
      }
      if (cap >= (1 << 28)) cap = INT32_MAX;
    }
    s_cap = cap;
  }
  __syncthreads();
  const int cap = s_cap;
  if (tid < G) {
    int r = 0;
    for (int h = 0; h < G; ++h) r += (sz[h] > sg) || (sz[h] == sg && h < tid);
    ws.order[r] = tid;
    cnt[r] = ntiles * (sg > cap ? (sg + cap - 1) / cap : 1);
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0, nsplit = 0;
    for (int r = 0; r < G; ++r) {
      ws.items[r] = acc;
      if (sz[ws.order[r]] > cap) nsplit = acc + cnt[r];
      acc += cnt[r];
    }
    ws.items[G] = acc;
    ws.plan[0] = cap;
    ws.plan[1] = nsplit;
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
  const dim3 grid(persistent_grid(max_items)), block(kThreads);
  // Groups of at most 256 rows on average: each weight panel serves about one row
  // tile, so the weights stream from HBM and the deeper weight ring pays (measured:
  // 256 groups of 128 rows 6-10% faster; 8 groups of 2048 rows 3.5% slower).
  const bool deep = T <= (int64_t)kBM * G;
  if (f16 && deep)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, MODE_ROWS, true, SCHED_DIRECT_DEEP>), grid, block, 0, s, p);
  else if (f16)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, MODE_ROWS, true, SCHED_DIRECT>), grid, block, 0, s, p);
  else if (deep)
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, MODE_ROWS, false, SCHED_DIRECT_DEEP>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<true, true, MODE_ROWS, false, SCHED_DIRECT>), grid, block, 0, s, p);
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
    hipLaunchKernelGGL((gemm_bf16_kernel<true, false, MODE_ROWS, true, SCHED_STAGED>), dim3(persistent_grid(max_items)),
                       dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<true, false, MODE_ROWS, false, SCHED_STAGED>), dim3(persistent_grid(max_items)),
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
  // the same plan with or without a bias grad, so gl_wgrad and gl_wgrad_bgrad give
  // the same dW bit for bit
  hipLaunchKernelGGL(contr_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, const_cast<void *>(ws), G, T,
                     p.tiles_i * p.tiles_j, (int)grid.x, 1);
  if (f16 && bg)
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, MODE_CONTR, true, SCHED_STAGED, true>), grid, block, 0, s, p);
  else if (f16)
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, MODE_CONTR, true, SCHED_STAGED>), grid, block, 0, s, p);
  else if (bg)
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, MODE_CONTR, false, SCHED_STAGED, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((gemm_bf16_kernel<false, false, MODE_CONTR, false, SCHED_STAGED>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace gl
