// Persistent grouped GEMM for the MXFP8 forward on gfx950 (scaled fp8 MFMA).
//
// The kernel template below still carries the bf16 paths it grew out of; only the
// MXFP8 forward (MX = true) is instantiated here.  The bf16 passes have their own
// kernel in gl_gemm_bf16.hip.
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
// wave a 128x64 block of 32x32x16 bf16 MFMAs with fp32 accumulators.
//
// Operand staging: the contraction advances 64 at a time through two LDS stages
// (32 KiB per operand per stage) filled by direct global->LDS loads
// (global_load_lds, 16 bytes per lane).  An operand whose contraction index is
// contiguous ("K-major") is staged as 256 rows of 128 bytes -- whole cache lines --
// and read with 16-byte LDS loads; one whose tile index is contiguous ("MN-major")
// is staged as 64 rows of 512 bytes and read with the gfx950 LDS transpose load
// (ds_read_b64_tr_b16), which hands each lane 4 consecutive contraction values of
// one column -- exactly the MFMA operand layout -- so no operand is transposed in
// registers.  Both layouts XOR-swizzle 16-byte slots so fragment reads are free of
// bank conflicts on gfx950's 64-bank LDS.
//
// Pipeline, per 64-deep tile kt (4 MFMA steps of 16): the loads of tile kt + 1 go
// out first, into the stage tile kt - 1 used; MFMA steps 0-2 run while the
// fragments of the following step are read; then every wave waits for its own
// loads of tile kt + 1 and the workgroup meets at one barrier, after which step 3
// runs while the first fragments of tile kt + 1 are read.  The steady-state body
// (every tile but the last two) is straight-line code: unconditional loads, no
// per-lane predicates.
//
// Masking: rows past the valid extent of a K-major tile are clamped onto a valid
// row (their products land in output rows that are never stored); columns past an
// MN-major tile's extent are clamped likewise; contraction indices past the end
// (the last tile of a group in wgrad, or a contraction length not a multiple of
// 64) are not loaded -- those lanes write zeros into their LDS slot instead.
//
// Scheduling: persistent grid, one workgroup per CU; workgroup b walks items b,
// b + grid, ...; items are remapped so each XCD (blockIdx % 8) works on a run of
// neighbouring tiles (8 x 4 blocks of output tiles) that share operand panels in
// its L2.  In row mode the item -> (group, row tile, column tile) map comes from
// the row-tile prefix table the offsets kernel left in the workspace.
#include "gl_common.hpp"

namespace gl {

namespace mfma_mx {

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kWM = 2, kWN = kWaves / kWM;          // wave grid
constexpr int kWTM = kBM / kWM, kWTN = kBN / kWN;   // wave tile 128 x 64
constexpr int kNI = kWTM / 32, kNJ = kWTN / 32;     // 32x32 MFMA blocks per wave
constexpr int kKS = kBK / 16;                       // MFMA steps per tile
constexpr int kOpElems = 256 * kBK;                 // bf16 elements per operand per stage
constexpr int kOpBytes = kOpElems * 2;
constexpr int kPieces = kOpBytes / 1024;            // 1 KiB direct-load pieces per operand per stage
constexpr int kQ = kPieces / kWaves;                // pieces per wave per operand per tile
constexpr int kOrdM = 8, kOrdN = 4;                 // blocked work-item order

enum { MODE_ROWS = 0, MODE_CONTR = 1 };

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
#define GL_LDS __attribute__((address_space(3)))

struct Params {
  const uint16_t *A;
  int64_t lda;
  const uint16_t *B;
  const uint16_t *const *B_ptrs;
  int64_t b_gstride;
  int64_t ldb;
  void *C;
  void *const *C_ptrs;
  int64_t c_gstride;
  int64_t ldc;
  const void *bias;
  const void *const *bias_ptrs;
  const void *ws;
  int G;
  int64_t T;
  int64_t rows_i, cols_j, P;
  int tiles_i, tiles_j;
  int accumulate;
  int out_f32;
  // MXFP8 forward only: E8M0 scales, one byte per 32 codes of a row
  const uint8_t *a_scale;              // [T, K/32]
  const uint8_t *b_scale;              // [G, N, K/32] stacked, or
  const uint8_t *const *b_scale_ptrs;  // per-group [N, K/32]
  int64_t scale_ld;                    // K / 32
};

// 16-byte slot swizzles for gfx950's LDS (64 banks of 4 bytes; a 16-byte read
// serves 16 lanes per cycle, an 8-byte read 32 lanes).
// K-major rows are 128 bytes (8 slots): chunk c of row r sits in slot c ^ swz_k(r).
// A fragment read takes one chunk of 16 consecutive rows per cycle; rows r and
// r + 2 share a 256-byte bank window, so the slot must differ across r >> 1.
// MN-major rows are 512 bytes (32 slots): chunk c of contraction row p sits in slot
// c ^ swz_m(p).  A transpose read serves 4 rows x 64 bytes per 32 lanes; the rows
// are 512 bytes apart (same banks), so the XOR moves each row's 64 bytes to its own
// quarter of the 256-byte window.
__device__ __forceinline__ int swz_k(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz_m(int p) { return (p & 3) << 2; }

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0f70); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Direct global->LDS loads of one operand, one 256 x 64 tile per contraction step.
// A wave owns the 1 KiB pieces wave, wave + kWaves, ... of each 32 KiB operand
// stage; lane l of a piece fills bytes [16 l, 16 l + 16) of it.  Per lane the
// global address of a piece is a fixed 32-bit offset from a wave-uniform tile base
// that advances by `step` bytes per tile, so issuing a full tile is straight-line
// code: no per-lane predicate, no 64-bit address arithmetic.
template <bool KMAJ>
struct Stream {
  const char *base;  // operand tile base for contraction tile 0
  int64_t step;      // bytes per contraction tile
  uint32_t off[kQ];  // lane byte offsets of its pieces

  // K-major: element (r, p) at b[r * ld + p]; rows >= rv clamp to rv - 1; a piece
  // is 8 rows x 128 bytes.  MN-major: element (r, p) at b[p * ld + r]; a piece is
  // 2 contraction rows x 512 bytes; columns >= rv clamp to the last valid 8-column
  // chunk (rv is a multiple of 8).
  __device__ __forceinline__ void init(const uint16_t *b, int64_t ld, int rv, int wave, int lane) {
    base = (const char *)b;
    step = KMAJ ? kBK * 2 : (int64_t)kBK * ld * 2;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int u = wave + kWaves * q;
      if (KMAJ) {
        const int R = 8 * u + (lane >> 3);
        const int c = (lane & 7) ^ swz_k(R);
        const int r = R < rv ? R : rv - 1;
        off[q] = (uint32_t)(((int64_t)r * ld + c * 8) * 2);
      } else {
        const int prow = 2 * u + (lane >> 5);
        int col = ((lane & 31) ^ swz_m(prow)) * 8;
        col = col < rv - 8 ? col : rv - 8;
        off[q] = (uint32_t)(((int64_t)prow * ld + col) * 2);
      }
    }
  }

  // All contraction indices of tile t are valid.
  __device__ __forceinline__ void issue_full(int t, char *st, int wave) const {
    const char *tb = base + (int64_t)t * step;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      __builtin_amdgcn_global_load_lds(tb + off[q], (GL_LDS void *)(st + (wave + kWaves * q) * 1024), 16, 0, 0);
  }

  // The last tile of a contraction: lanes whose piece lies past pmax write zeros
  // into their LDS slot instead of loading.
  __device__ __forceinline__ void issue_masked(int t, int64_t pmax, char *st, int wave, int lane) const {
    const char *tb = base + (int64_t)t * step;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int u = wave + kWaves * q;
      char *dst = st + u * 1024;
      // first contraction index (within the tile) this lane's piece holds
      const int pfirst = KMAJ ? ((lane & 7) ^ swz_k(8 * u + (lane >> 3))) * 8 : 2 * u + (lane >> 5);
      if ((int64_t)t * kBK + pfirst < pmax)
        __builtin_amdgcn_global_load_lds(tb + off[q], (GL_LDS void *)dst, 16, 0, 0);
      else
        *(uint4 *)(dst + lane * 16) = make_uint4(0, 0, 0, 0);
    }
  }
};

// MFMA operand fragment (32 rows/columns x 16 contraction values; lane l holds row
// l % 32, contraction values 8 (l / 32) + 0..7) for MFMA step ks of a stage.
__device__ __forceinline__ bf16x8_t frag_kmaj(const uint16_t *st, int row0, int ks, int lane) {
  const int r = row0 + (lane & 31);
  const int c = 2 * ks + (lane >> 5);
  return *(const bf16x8_t *)(st + r * kBK + ((c ^ swz_k(r)) << 3));
}

__device__ __forceinline__ bf16x8_t frag_mnmaj(const uint16_t *st, int col0, int ks, int lane) {
  // 16-lane groups: lanes 0-15 / 16-31 take columns 0-15 / 16-31, lane halves take
  // contraction rows 0-7 / 8-15 of the step; lane s of a group names row s / 4 and
  // columns 4 (s % 4) .. + 3, and the transpose hands lane s column s of those rows.
  const int s = lane & 15, grp = lane >> 4;
  const int col = col0 + ((grp & 1) << 4) + ((s & 3) << 2);
  const int chunk = col >> 3, within = col & 7;
  v4i16 h[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int prow = ks * 16 + (grp >> 1) * 8 + t * 4 + (s >> 2);
    const uint16_t *a = st + prow * 256 + ((chunk ^ swz_m(prow)) << 3) + within;
    h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GL_LDS v4i16 *)a);
  }
  const v8i16 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// MXFP8 operand fragment for the scaled 32x32x64 MFMA, step s (64 codes) of a
// 128-code K-major row: lane l holds row l % 32 and, for each of the step's two
// 32-code scale blocks, 16 codes -- those at byte 16 (l / 32) of the block.
__device__ __forceinline__ i32x8_t frag_mx(const uint16_t *st, int row0, int s, int lane) {
  const int r = row0 + (lane & 31), h = lane >> 5;
  const i32x4_t lo = *(const i32x4_t *)(st + r * kBK + (((4 * s + h) ^ swz_k(r)) << 3));
  const i32x4_t hi = *(const i32x4_t *)(st + r * kBK + (((4 * s + 2 + h) ^ swz_k(r)) << 3));
  return (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// MX == true: the MXFP8 forward.  Operands are E4M3 codes handled as two-byte
// units (a 128-byte tile row is 128 codes = 4 scale blocks); each tile also brings
// the 4 scale bytes of every A and B row into a small LDS area.
template <bool A_KMAJ, bool B_KMAJ, int MODE, bool MX>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2][2][kOpElems];
  __shared__ __attribute__((aligned(1024))) uint32_t lds_sc[2][2][256];  // MXFP8 scale dwords per row

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

  for (int w = first; w < total; w += grid) {
    // ------------------------------------------------------------ decode item
    int g, local, MT;
    const int NT = p.tiles_j;
    if (MODE == MODE_ROWS) {
      g = find_group(pre, p.G, w / NT);
      local = w - pre[g] * NT;
      MT = pre[g + 1] - pre[g];
    } else {
      const int per = p.tiles_i * NT;
      g = w / per;
      local = w - g * per;
      MT = p.tiles_i;
    }
    // bands of kOrdN tile columns; inside a band, blocks of kOrdM tile rows; inside
    // a block, row tiles fastest
    const int cb = local / (MT * kOrdN);
    const int bw = min(kOrdN, NT - cb * kOrdN);
    const int l2 = local - cb * MT * kOrdN;
    const int rb = l2 / (kOrdM * bw);
    const int bh = min(kOrdM, MT - rb * kOrdM);
    const int l3 = l2 - rb * kOrdM * bw;
    const int it = rb * kOrdM + l3 % bh;
    const int jt = cb * kOrdN + l3 / bh;

    const int64_t g_off = off[g];
    const int64_t g_rows = off[g + 1] - g_off;
    if (MODE == MODE_CONTR && p.accumulate && g_rows == 0) continue;  // main_grad untouched

    const uint16_t *a_base, *b_base;
    int a_rv, b_rv;
    int64_t pmax;
    if (MODE == MODE_ROWS) {
      a_base = p.A + (g_off + (int64_t)it * kBM) * p.lda;
      a_rv = (int)min64(kBM, g_rows - (int64_t)it * kBM);
      const uint16_t *bg = p.B ? p.B + (int64_t)g * p.b_gstride : p.B_ptrs[g];
      b_base = B_KMAJ ? bg + (int64_t)jt * kBN * p.ldb : bg + (int64_t)jt * kBN;
      b_rv = (int)min64(kBN, p.cols_j - (int64_t)jt * kBN);
      pmax = p.P;
    } else {
      a_base = p.A + g_off * p.lda + (int64_t)it * kBM;
      a_rv = (int)min64(kBM, p.rows_i - (int64_t)it * kBM);
      b_base = p.B + g_off * p.ldb + (int64_t)jt * kBN;
      b_rv = (int)min64(kBN, p.cols_j - (int64_t)jt * kBN);
      pmax = g_rows;
    }
    const int nk = (int)((pmax + kBK - 1) / kBK);
    const int nfull = (int)(pmax / kBK);  // tiles [0, nfull) are complete; nk - nfull <= 1

    Stream<A_KMAJ> sa;
    Stream<B_KMAJ> sb;
    sa.init(a_base, p.lda, a_rv, wave, lane);
    sb.init(b_base, p.ldb, b_rv, wave, lane);
    char *const ring = (char *)&lds[0][0][0];
    // MXFP8: wave w loads the scale dwords (4 blocks = one tile) of 64 rows per
    // tile -- waves 0-3 the A rows, waves 4-7 the B rows
    const char *sc_base = nullptr;
    uint32_t sc_off = 0;
    if (MX) {
      const int r = (wave & 3) * 64 + lane;
      if (wave < 4) {
        sc_base = (const char *)p.a_scale + (g_off + (int64_t)it * kBM) * p.scale_ld;
        sc_off = (uint32_t)((r < a_rv ? r : a_rv - 1) * p.scale_ld);
      } else {
        const uint8_t *bs = p.b_scale ? p.b_scale + (int64_t)g * p.cols_j * p.scale_ld : p.b_scale_ptrs[g];
        sc_base = (const char *)bs + (int64_t)jt * kBN * p.scale_ld;
        sc_off = (uint32_t)((r < b_rv ? r : b_rv - 1) * p.scale_ld);
      }
    }
    auto issue_scales = [&](int t) {
      if (MX)
        __builtin_amdgcn_global_load_lds(sc_base + sc_off + 4 * t,
                                         (GL_LDS void *)&lds_sc[t & 1][wave >> 2][(wave & 3) * 64], 4, 0, 0);
    };
    auto issue = [&](int t) {
      char *st = ring + (t & 1) * 2 * kOpBytes;
      if (t < nfull) {
        sa.issue_full(t, st, wave);
        sb.issue_full(t, st + kOpBytes, wave);
      } else {
        sa.issue_masked(t, pmax, st, wave, lane);
        sb.issue_masked(t, pmax, st + kOpBytes, wave, lane);
      }
      issue_scales(t);
    };

    // -------------------------------------------------------------- main loop
    f32x16_t acc[kNI][kNJ];
#pragma unroll
    for (int ii = 0; ii < kNI; ++ii)
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[ii][jj][q] = 0.f;

    auto load_frags = [&](int t, int ks, bf16x8_t *af, bf16x8_t *bfr) {
      const uint16_t *ta = lds[t & 1][0];
      const uint16_t *tb = lds[t & 1][1];
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
          acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[jj], af[ii], acc[ii][jj], 0, 0, 0);
    };

    if constexpr (MX) {
      // two scaled 32x32x64 steps per tile; per step the two B fragments are read
      // first and the A fragments streamed one at a time (32-byte fragments leave
      // no room for a second fragment set)
      auto step_mx = [&](int t, int st_, const uint32_t *scl) {
        const int sh = 8 * (2 * st_ + (lane >> 5));  // this lane's scale block in the step
        i32x8_t bfr[kNJ];
#pragma unroll
        for (int jj = 0; jj < kNJ; ++jj) bfr[jj] = frag_mx(lds[t & 1][1], wn * kWTN + jj * 32, st_, lane);
#pragma unroll
        for (int ii = 0; ii < kNI; ++ii) {
          const i32x8_t af = frag_mx(lds[t & 1][0], wm * kWTM + ii * 32, st_, lane);
#pragma unroll
          for (int jj = 0; jj < kNJ; ++jj)
            acc[ii][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bfr[jj], af, acc[ii][jj], 0, 0, 0, (int)(scl[kNI + jj] >> sh), 0, (int)(scl[ii] >> sh));
        }
      };
      if (nk > 0) {
        issue(0);
        wait_vm0();
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
      }
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) issue(kt + 1);
        uint32_t sc[kNI + kNJ];  // scale dwords of this lane's A and B rows for tile kt
#pragma unroll
        for (int ii = 0; ii < kNI; ++ii) sc[ii] = lds_sc[kt & 1][0][wm * kWTM + ii * 32 + (lane & 31)];
#pragma unroll
        for (int jj = 0; jj < kNJ; ++jj) sc[kNI + jj] = lds_sc[kt & 1][1][wn * kWTN + jj * 32 + (lane & 31)];
        step_mx(kt, 0, sc);
        step_mx(kt, 1, sc);
        wait_vm0();
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
      }
    } else {
    bf16x8_t fa[2][kNI], fb[2][kNJ];
    if (nk > 0) {
      issue(0);
      wait_vm0();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      load_frags(0, 0, fa[0], fb[0]);
    }
    // One tile per iteration; fragment set (ks & 1) feeds MFMA step ks while set
    // (ks + 1) & 1 is refilled.  The barrier before the last step makes tile kt + 1
    // visible and frees the stage tile kt - 1 used for the loads of tile kt + 2.
    static_assert((kKS & 1) == 0, "step 0 of every tile must read fragment set 0");
    auto body = [&](int kt, bool steady) {
      if (steady) {
        char *st = ring + ((kt + 1) & 1) * 2 * kOpBytes;
        sa.issue_full(kt + 1, st, wave);
        sb.issue_full(kt + 1, st + kOpBytes, wave);
      } else if (kt + 1 < nk) {
        issue(kt + 1);
      }
#pragma unroll
      for (int ks = 0; ks < kKS - 1; ++ks) {
        load_frags(kt, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
        mfmas(fa[ks & 1], fb[ks & 1]);
      }
      wait_vm0();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      if (steady || kt + 1 < nk) load_frags(kt + 1, 0, fa[0], fb[0]);
      mfmas(fa[(kKS - 1) & 1], fb[(kKS - 1) & 1]);
    };

    int kt = 0;
    for (; kt + 1 < nfull; ++kt) body(kt, true);  // tile kt + 1 complete: straight-line body
    for (; kt < nk; ++kt) body(kt, false);
    }
    __builtin_amdgcn_s_barrier();  // every wave is done with the stages before they are refilled

    // --------------------------------------------------------------- epilogue
    // lane holds C[i][j..j+3] with i = ii*32 + lane%32, j = jj*32 + q4*8 + (lane/32)*4
    char *cbase;
    int64_t row0;
    if (MODE == MODE_ROWS) {
      cbase = (char *)p.C;
      row0 = g_off + (int64_t)it * kBM;
    } else {
      cbase = p.C ? (char *)p.C + (int64_t)g * p.c_gstride * (p.out_f32 ? 4 : 2) : (char *)p.C_ptrs[g];
      row0 = (int64_t)it * kBM;
    }
    const char *bias_g = nullptr;
    if (p.bias) bias_g = (const char *)p.bias + (int64_t)g * p.cols_j * (p.out_f32 ? 4 : 2);
    else if (p.bias_ptrs) bias_g = (const char *)p.bias_ptrs[g];
#pragma unroll
    for (int ii = 0; ii < kNI; ++ii) {
      const int il = wm * kWTM + ii * 32 + (lane & 31);
      if (il >= a_rv) continue;
      const int64_t row = row0 + il;
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int jl = wn * kWTN + jj * 32 + q4 * 8 + (lane >> 5) * 4;
          if (jl >= b_rv) continue;
          const int64_t col = (int64_t)jt * kBN + jl;
          float v0 = acc[ii][jj][q4 * 4 + 0], v1 = acc[ii][jj][q4 * 4 + 1];
          float v2 = acc[ii][jj][q4 * 4 + 2], v3 = acc[ii][jj][q4 * 4 + 3];
          if (bias_g) {
            if (p.out_f32) {
              const float4 bv = *(const float4 *)(bias_g + col * 4);
              v0 += bv.x; v1 += bv.y; v2 += bv.z; v3 += bv.w;
            } else {
              const uint2 bv = *(const uint2 *)(bias_g + col * 2);
              v0 += bf16_to_f32(bv.x & 0xffff); v1 += bf16_to_f32(bv.x >> 16);
              v2 += bf16_to_f32(bv.y & 0xffff); v3 += bf16_to_f32(bv.y >> 16);
            }
          }
          if (p.out_f32) {
            float4 *dst = (float4 *)(cbase + (row * p.ldc + col) * 4);
            if (p.accumulate) {
              const float4 o = *dst;
              v0 += o.x; v1 += o.y; v2 += o.z; v3 += o.w;
            }
            *dst = make_float4(v0, v1, v2, v3);
          } else {
            uint2 *dst = (uint2 *)(cbase + (row * p.ldc + col) * 2);
            if (p.accumulate) {
              const uint2 o = *dst;
              v0 += bf16_to_f32(o.x & 0xffff); v1 += bf16_to_f32(o.x >> 16);
              v2 += bf16_to_f32(o.y & 0xffff); v3 += bf16_to_f32(o.y >> 16);
            }
            *dst = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
          }
        }
      }
    }
  }
}

// Compute units of the current device (one persistent workgroup per CU).
static int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || n <= 0)
    n = 256;
  return n;
}

static int persistent_grid(int64_t max_items) {
  const int cus = num_cus();
  int64_t g = max_items < cus ? max_items : cus;
  if (g >= 8) g &= ~7;  // keeps the XCD-aware remap a bijection
  return (int)(g > 0 ? g : 1);
}

}  // namespace mfma_mx

// MXFP8 forward: y = deq(xq) deq(wq)^T (+ b).  Codes travel as two-byte units, so
// the loads see K/2 units per row; K % 128 == 0 keeps every tile whole and the
// per-tile scale dwords aligned.
hipError_t launch_forward_mxfp8(int G, int64_t K, int64_t N, int64_t T, const uint8_t *xq, const uint8_t *xs,
                                const uint8_t *wq, const uint8_t *const *wq_ptrs, const uint8_t *ws_scale,
                                const uint8_t *const *ws_scale_ptrs, const void *bias,
                                const void *const *bias_ptrs, void *y, int out_f32, const void *ws,
                                hipStream_t s) {
  using namespace mfma_mx;
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
  hipLaunchKernelGGL((gemm_bf16_kernel<true, true, MODE_ROWS, true>), dim3(persistent_grid(max_items)),
                     dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace gl
