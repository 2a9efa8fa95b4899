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
#include "gl_common.hpp"

// Stage depth and ring length (tuning parameters; 64 x 2 measured best on MI355X)
#ifndef GL_BK
#define GL_BK 64
#endif
#ifndef GL_STAGES
#define GL_STAGES 2
#endif

namespace gl {

namespace gemm_bf16 {

constexpr int kBM = 256, kBN = 256;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kWN = kWaves / 2;                     // wave grid 2 x 4
constexpr int kWTM = kBM / 2, kWTN = kBN / kWN;     // wave tile
constexpr int kNI = kWTM / 32, kNJ = kWTN / 32;     // 32x32 MFMA blocks per wave
constexpr int kBK = GL_BK;                          // contraction depth of a stage
constexpr int kS = GL_STAGES;                       // stages in the LDS ring
constexpr int kKS = kBK / 16;                       // MFMA steps per stage
constexpr int kRowB = 2 * kBK;                      // bytes of a K-major stage row
constexpr int kChunks = kRowB / 16;                 // 16-byte chunks per K-major row
constexpr int kRowsPerPiece = 1024 / kRowB;         // K-major rows per 1 KiB piece
constexpr int kOpBytes = 256 * kRowB;               // bytes per operand per stage
constexpr int kStageBytes = 2 * kOpBytes;
constexpr int kQ = kOpBytes / 1024 / kWaves;        // pieces per wave per operand per stage
constexpr int kLoadsPerStage = 2 * kQ;              // direct loads per wave per stage
constexpr int kOrdM = 8, kOrdN = 4;                 // blocked work-item order
static_assert(kBK == 32 || kBK == 64, "stage depth");
static_assert(kS >= 2 && kS * kStageBytes <= 160 * 1024, "LDS ring");
static_assert((kS - 2) * kLoadsPerStage <= 63, "vmcnt range");

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
};

// 16-byte slot swizzles for gfx950's LDS (64 banks of 4 bytes; a 16-byte read
// serves 16 lanes per cycle, an 8-byte read 32 lanes).
// K-major rows hold kChunks slots: chunk c of row r sits in slot c ^ swz_k(r).  A
// fragment read takes one chunk of 16 consecutive rows per cycle; 16 / kChunks
// consecutive rows share a 256-byte bank window, so the slot must differ across
// r / (16 / kChunks).
// MN-major rows are 512 bytes (32 slots): chunk c of contraction row p sits in slot
// c ^ swz_m(p).  A transpose read serves 4 rows x 64 bytes per 32 lanes; the rows
// are 512 bytes apart (same banks), so the XOR moves each row's 64 bytes to its own
// quarter of the 256-byte window.
__device__ __forceinline__ int swz_k(int r) { return (r / (16 / kChunks)) & (kChunks - 1); }
__device__ __forceinline__ int swz_m(int p) { return (p & 3) << 2; }

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0f70); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }
// s_waitcnt vmcnt(n) (lgkmcnt and expcnt left at their maxima), gfx9 encoding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// Buffer resource over [base, base + 2 GiB): raw (unswizzled, stride 0) addressing,
// gfx9 data format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_at(const char *base) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, 0x7fffffff, 0x00020000);
}

// Direct buffer->LDS loads of one operand, one 256 x kBK tile per stage.  A wave
// owns the 1 KiB pieces wave, wave + kWaves, ... of each operand stage; lane l of a
// piece fills bytes [16 l, 16 l + 16) of it.
template <bool KMAJ>
struct Stream {
  const char *base;  // operand tile base for contraction stage 0
  int64_t step;      // bytes per contraction stage
  uint32_t off[kQ];  // lane byte offsets of its pieces from the stage's base

  // K-major: element (r, p) at b[r * ld + p]; rows >= rv clamp to rv - 1; a piece
  // is kRowsPerPiece rows x kRowB bytes.  MN-major: element (r, p) at b[p * ld + r];
  // a piece is 2 contraction rows x 512 bytes; columns >= rv clamp to the last
  // valid 8-column chunk (rv is a multiple of 8).
  __device__ __forceinline__ void init(const uint16_t *b, int64_t ld, int rv, int wave, int lane) {
    base = (const char *)b;
    step = KMAJ ? kRowB : (int64_t)kBK * ld * 2;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int u = wave + kWaves * q;
      if (KMAJ) {
        const int R = kRowsPerPiece * u + lane / kChunks;
        const int c = (lane % kChunks) ^ swz_k(R);
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

  // Every contraction index of stage t is valid.
  __device__ __forceinline__ void issue_full(int t, char *st, int wave) const {
    const __amdgpu_buffer_rsrc_t r = rsrc_at(base + (int64_t)t * step);
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (GL_LDS void *)(st + (wave + kWaves * q) * 1024), 16, off[q], 0, 0,
                                               0);
  }

  // The last stage of a contraction: lanes whose piece lies past pmax write zeros
  // into their LDS slot instead of loading.
  __device__ __forceinline__ void issue_masked(int t, int64_t pmax, char *st, int wave, int lane) const {
    const __amdgpu_buffer_rsrc_t r = rsrc_at(base + (int64_t)t * step);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int u = wave + kWaves * q;
      char *dst = st + u * 1024;
      // first contraction index (within the stage) this lane's piece holds
      const int pfirst =
          KMAJ ? ((lane % kChunks) ^ swz_k(kRowsPerPiece * u + lane / kChunks)) * 8 : 2 * u + (lane >> 5);
      if ((int64_t)t * kBK + pfirst < pmax)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (GL_LDS void *)dst, 16, off[q], 0, 0, 0);
      else
        *(uint4 *)(dst + lane * 16) = make_uint4(0, 0, 0, 0);
    }
  }
};

// MFMA operand fragment (32 rows/columns x 16 contraction values; lane l holds row
// l % 32, contraction values 8 (l / 32) + 0..7) for MFMA step ks of a stage.
__device__ __forceinline__ bf16x8_t frag_kmaj(const char *st, int row0, int ks, int lane) {
  const int r = row0 + (lane & 31);
  const int c = 2 * ks + (lane >> 5);
  return *(const bf16x8_t *)(st + r * kRowB + ((c ^ swz_k(r)) << 4));
}

__device__ __forceinline__ bf16x8_t frag_mnmaj(const char *st, int col0, int ks, int lane) {
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
    const char *a = st + prow * 512 + ((chunk ^ swz_m(prow)) << 4) + within * 2;
    h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GL_LDS v4i16 *)a);
  }
  const v8i16 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Stores 4 consecutive output columns of one row: optional bias (per output
// column), optional accumulate into the existing bf16 or fp32 values.
__device__ __forceinline__ void store4(char *cbase, int64_t row, int64_t ldc, int64_t col, const char *bias_g,
                                      int out_f32, int accumulate, float v0, float v1, float v2, float v3) {
  if (bias_g) {
    if (out_f32) {
      const float4 bv = *(const float4 *)(bias_g + col * 4);
      v0 += bv.x; v1 += bv.y; v2 += bv.z; v3 += bv.w;
    } else {
      const uint2 bv = *(const uint2 *)(bias_g + col * 2);
      v0 += bf16_to_f32(bv.x & 0xffff); v1 += bf16_to_f32(bv.x >> 16);
      v2 += bf16_to_f32(bv.y & 0xffff); v3 += bf16_to_f32(bv.y >> 16);
    }
  }
  if (out_f32) {
    float4 *dst = (float4 *)(cbase + (row * ldc + col) * 4);
    if (accumulate) {
      const float4 o = *dst;
      v0 += o.x; v1 += o.y; v2 += o.z; v3 += o.w;
    }
    *dst = make_float4(v0, v1, v2, v3);
  } else {
    uint2 *dst = (uint2 *)(cbase + (row * ldc + col) * 2);
    if (accumulate) {
      const uint2 o = *dst;
      v0 += bf16_to_f32(o.x & 0xffff); v1 += bf16_to_f32(o.x >> 16);
      v2 += bf16_to_f32(o.y & 0xffff); v3 += bf16_to_f32(o.y >> 16);
    }
    *dst = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
  }
}

template <bool A_KMAJ, bool B_KMAJ, int MODE>
__global__ __launch_bounds__(kThreads) void gemm_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) char lds[kS * kStageBytes];

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
    const int nfull = (int)(pmax / kBK);  // stages [0, nfull) are complete; nk - nfull <= 1

    Stream<A_KMAJ> sa;
    Stream<B_KMAJ> sb;
    sa.init(a_base, p.lda, a_rv, wave, lane);
    sb.init(b_base, p.ldb, b_rv, wave, lane);
    auto stage_ptr = [&](int t) { return lds + (t % kS) * kStageBytes; };
    auto issue = [&](int t) {
      char *st = stage_ptr(t);
      if (t < nfull) {
        sa.issue_full(t, st, wave);
        sb.issue_full(t, st + kOpBytes, wave);
      } else {
        sa.issue_masked(t, pmax, st, wave, lane);
        sb.issue_masked(t, pmax, st + kOpBytes, wave, lane);
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

    auto load_frags = [&](int t, int ks, bf16x8_t *af, bf16x8_t *bfr) {
      const char *ta = stage_ptr(t);
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
          acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[jj], af[ii], acc[ii][jj], 0, 0, 0);
    };

    bf16x8_t fa[2][kNI], fb[2][kNJ];
    // prologue: stages 0 .. kS-2 in flight, stage 0 visible, step 0 fragments read
    for (int t = 0; t < kS - 1 && t < nk; ++t) issue(t);
    if (nk > 0) {
      wait_vm0();
      __builtin_amdgcn_s_barrier();
      load_frags(0, 0, fa[0], fb[0]);
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
      } else if (kt + kS - 1 < nk) {
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
      // stage kt + 1 complete: at most the loads of stages kt + 2 .. kt + kS - 1
      // may still be in flight
      if (steady)
        wait_vm<(kS - 2) * kLoadsPerStage>();
      else
        wait_vm0();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      if (steady || kt + 1 < nk) load_frags(kt + 1, 0, fa[0], fb[0]);
      fence();
      mfmas(fa[(kKS - 1) & 1], fb[(kKS - 1) & 1]);
      fence();
    };

    int kt = 0;
    for (; kt + kS - 1 < nfull; ++kt) body(kt, true);  // every stage issued here is complete
    for (; kt < nk; ++kt) body(kt, false);
    __builtin_amdgcn_s_barrier();  // every wave is done with the ring before it is refilled

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
          store4(cbase, row, p.ldc, (int64_t)jt * kBN + jl, bias_g, p.out_f32, p.accumulate,
                 acc[ii][jj][q4 * 4 + 0], acc[ii][jj][q4 * 4 + 1], acc[ii][jj][q4 * 4 + 2], acc[ii][jj][q4 * 4 + 3]);
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

}  // namespace gemm_bf16

// forward: y = x W^T (+ b); A = x [T,K], B = W [N,K]
hipError_t launch_forward_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *x, const uint16_t *w,
                               const uint16_t *const *w_ptrs, const void *bias, const void *const *bias_ptrs,
                               uint16_t *y, const void *ws, hipStream_t s) {
  using namespace gemm_bf16;
  Params p{};
  p.A = x; p.lda = K;
  p.B = w; p.B_ptrs = w_ptrs; p.b_gstride = N * K; p.ldb = K;
  p.C = y; p.ldc = N;
  p.bias = bias; p.bias_ptrs = bias_ptrs;
  p.ws = ws; p.G = G; p.T = T;
  p.cols_j = N; p.P = K;
  p.tiles_j = (int)((N + kBN - 1) / kBN);
  const int64_t max_items = ((T + kBM - 1) / kBM + G) * p.tiles_j;
  hipLaunchKernelGGL((gemm_kernel<true, true, MODE_ROWS>), dim3(persistent_grid(max_items)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// dgrad: dx = dy W; A = dy [T,N] (n contiguous), B[j=k][p=n] = W[n][k] (k contiguous)
hipError_t launch_dgrad_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *dy, const uint16_t *w,
                             const uint16_t *const *w_ptrs, uint16_t *dx, const void *ws, hipStream_t s) {
  using namespace gemm_bf16;
  Params p{};
  p.A = dy; p.lda = N;
  p.B = w; p.B_ptrs = w_ptrs; p.b_gstride = N * K; p.ldb = K;
  p.C = dx; p.ldc = K;
  p.ws = ws; p.G = G; p.T = T;
  p.cols_j = K; p.P = N;
  p.tiles_j = (int)((K + kBN - 1) / kBN);
  const int64_t max_items = ((T + kBM - 1) / kBM + G) * p.tiles_j;
  hipLaunchKernelGGL((gemm_kernel<true, false, MODE_ROWS>), dim3(persistent_grid(max_items)), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// wgrad: dW_g[n][k] = sum_r dy[r][n] x[r][k]; A[i=n][p=r] (n contiguous), B[j=k][p=r] (k contiguous)
hipError_t launch_wgrad_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *x, const uint16_t *dy,
                             void *dw, void *const *dw_ptrs, int out_f32, int accumulate, const void *ws,
                             hipStream_t s) {
  using namespace gemm_bf16;
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
  const int64_t max_items = (int64_t)G * p.tiles_i * p.tiles_j;
  hipLaunchKernelGGL((gemm_kernel<false, false, MODE_CONTR>), dim3(persistent_grid(max_items)), dim3(kThreads), 0, s,
                     p);
  return hipGetLastError();
}

}  // namespace gl
