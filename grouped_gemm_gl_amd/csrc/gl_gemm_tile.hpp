// Tile machinery shared by the gfx950 MFMA grouped GEMMs (bf16 and MXFP8): tile
// shape, direct buffer->LDS operand streams, LDS layouts and their fragment
// readers, work-item decode and the output store.  See gl_gemm_bf16.hip for how
// the pieces fit together.
#pragma once

#include <type_traits>

#include "gl_common.hpp"

namespace gl {
namespace gemm {

constexpr int kBM = 256, kBN = 256;
constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int kWN = kWaves / 2;                     // wave grid 2 x 4
constexpr int kWTM = kBM / 2, kWTN = kBN / kWN;     // wave tile 128 x 64
constexpr int kNI = kWTM / 32, kNJ = kWTN / 32;     // 32x32 MFMA blocks per wave
constexpr int kBK = 64;                             // contraction depth of a stage (2-byte units)
constexpr int kS = 2;                               // stages in the LDS ring
constexpr int kKS = kBK / 16;                       // bf16 MFMA steps per stage
constexpr int kRowB = 2 * kBK;                      // bytes of a K-major stage row
constexpr int kChunks = kRowB / 16;                 // 16-byte chunks per K-major row
constexpr int kRowsPerPiece = 1024 / kRowB;         // K-major rows per 1 KiB piece
constexpr int kOpBytes = 256 * kRowB;               // bytes per operand per stage
constexpr int kStageBytes = 2 * kOpBytes;
constexpr int kQ = kOpBytes / 1024 / kWaves;        // pieces per wave per operand per stage
constexpr int kLoadsPerStage = 2 * kQ;              // direct loads per wave per stage
constexpr int kOrdM = 8, kOrdN = 4;                 // blocked work-item order
static_assert(kS >= 2 && kS * kStageBytes <= 160 * 1024, "LDS ring");
static_assert((kS - 2) * kLoadsPerStage <= 63, "vmcnt range");

// MODE_ROWS: the grouped index is the tile row (forward, dgrad).  MODE_CONTR: the
// grouped index is the contraction, MN-major operands (bf16 wgrad).  MODE_KCONTR:
// the grouped index is the contraction, K-major operands whose groups start at
// 128-aligned contraction offsets and are zero-padded to whole 128-element tiles
// (MXFP8 wgrad on columnwise codes stored transposed).
enum { MODE_ROWS = 0, MODE_CONTR = 1, MODE_KCONTR = 2 };
constexpr int kKcontrUnits = 64;  // one padded 128-code contraction tile, in 2-byte units

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
#define GL_LDS __attribute__((address_space(3)))
// Global memory, spelled out: a pointer the compiler cannot trace to a kernel
// argument (one taken from a per-group pointer array) would otherwise be accessed
// with flat instructions, which also count in lgkmcnt -- and the next tile's first
// wait for its LDS reads would then wait for the previous tile's output stores.
#if defined(__HIP_DEVICE_COMPILE__)
#define GL_GLOBAL __attribute__((address_space(1)))
#else
#define GL_GLOBAL  // the host pass only checks these device bodies
#endif

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
  // bf16 / fp16 wgrad only: bias gradient of the same dy, stacked [G, N] or per group
  void *db;
  void *const *db_ptrs;
  int db_f32;                          // db is fp32 (else the input's 16-bit type)
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
// column, of the output's type), optional accumulate into the existing values.
// 16-bit outputs are bf16, or fp16 when F16.
// Addresses arrive as integers: a cast of a generic pointer to the global address
// space can be folded back to a flat access when the pointer is a select of a
// kernel argument and a loaded one; an integer cannot.
template <bool F16>
__device__ __forceinline__ void store4(uintptr_t cbase, int64_t row, int64_t ldc, int64_t col, uintptr_t bias_g,
                                      int out_f32, int accumulate, float v0, float v1, float v2, float v3) {
  if (bias_g) {
    if (out_f32) {
      const float4 bv = *(const GL_GLOBAL float4 *)(bias_g + col * 4);
      v0 += bv.x; v1 += bv.y; v2 += bv.z; v3 += bv.w;
    } else {
      const uint2 bv = *(const GL_GLOBAL uint2 *)(bias_g + col * 2);
      v0 += h16_to_f32<F16>(bv.x & 0xffff); v1 += h16_to_f32<F16>(bv.x >> 16);
      v2 += h16_to_f32<F16>(bv.y & 0xffff); v3 += h16_to_f32<F16>(bv.y >> 16);
    }
  }
  if (out_f32) {
    GL_GLOBAL float4 *dst = (GL_GLOBAL float4 *)(cbase + (row * ldc + col) * 4);
    if (accumulate) {
      const float4 o = *dst;
      v0 += o.x; v1 += o.y; v2 += o.z; v3 += o.w;
    }
    *dst = make_float4(v0, v1, v2, v3);
  } else {
    GL_GLOBAL uint2 *dst = (GL_GLOBAL uint2 *)(cbase + (row * ldc + col) * 2);
    if (accumulate) {
      const uint2 o = *dst;
      v0 += h16_to_f32<F16>(o.x & 0xffff); v1 += h16_to_f32<F16>(o.x >> 16);
      v2 += h16_to_f32<F16>(o.y & 0xffff); v3 += h16_to_f32<F16>(o.y >> 16);
    }
    *dst = make_uint2((uint32_t)f32_to_h16<F16>(v0) | ((uint32_t)f32_to_h16<F16>(v1) << 16),
                      (uint32_t)f32_to_h16<F16>(v2) | ((uint32_t)f32_to_h16<F16>(v3) << 16));
  }
}

// MXFP8 operand fragment for the scaled 32x32x64 MFMA, step s (64 codes) of a
// 128-code K-major stage row: lane l holds row l % 32 and, for each of the step's
// two 32-code scale blocks, 16 codes -- those at byte 16 (l / 32) of the block.
__device__ __forceinline__ i32x8_t frag_mx(const char *st, int row0, int s, int lane) {
  const int r = row0 + (lane & 31), h = lane >> 5;
  const i32x4_t lo = *(const i32x4_t *)(st + r * kRowB + (((4 * s + h) ^ swz_k(r)) << 4));
  const i32x4_t hi = *(const i32x4_t *)(st + r * kRowB + (((4 * s + 2 + h) ^ swz_k(r)) << 4));
  return (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// One output tile of one group: what a work item decodes to.
struct Tile {
  int g, it, jt;
  int64_t g_off, g_rows;
  const uint16_t *a_base, *b_base;  // operand tile bases at contraction 0
  int a_rv, b_rv;                   // valid rows of the A and B tiles
  int64_t pmax;                     // contraction length
};

// Work item w -> tile.  Row mode (forward, dgrad): the grouped index is the tile
// row, mapped through the row-tile prefix table; contraction mode (wgrad): the
// grouped index is the contraction.  Inside a group: bands of kOrdN tile columns,
// inside a band blocks of kOrdM tile rows, inside a block row tiles fastest.
template <bool A_KMAJ, bool B_KMAJ, int MODE>
__device__ __forceinline__ Tile decode_tile(const Params &p, const int64_t *__restrict__ off,
                                            const int32_t *__restrict__ pre, int w,
                                            const int32_t *__restrict__ cpre = nullptr) {
  Tile t;
  int local, MT;
  const int NT = p.tiles_j;
  if (MODE == MODE_ROWS) {
    t.g = find_group(pre, p.G, w / NT);
    local = w - pre[t.g] * NT;
    MT = pre[t.g + 1] - pre[t.g];
  } else {
    const int per = p.tiles_i * NT;
    t.g = w / per;
    local = w - t.g * per;
    MT = p.tiles_i;
  }
  const int cb = local / (MT * kOrdN);
  const int bw = min(kOrdN, NT - cb * kOrdN);
  const int l2 = local - cb * MT * kOrdN;
  const int rb = l2 / (kOrdM * bw);
  const int bh = min(kOrdM, MT - rb * kOrdM);
  const int l3 = l2 - rb * kOrdM * bw;
  t.it = rb * kOrdM + l3 % bh;
  t.jt = cb * kOrdN + l3 / bh;
  t.g_off = off[t.g];
  t.g_rows = off[t.g + 1] - t.g_off;
  if (MODE == MODE_ROWS) {
    t.a_base = p.A + (t.g_off + (int64_t)t.it * kBM) * p.lda;
    t.a_rv = (int)min64(kBM, t.g_rows - (int64_t)t.it * kBM);
    const uint16_t *bg = p.B ? p.B + (int64_t)t.g * p.b_gstride : p.B_ptrs[t.g];
    t.b_base = B_KMAJ ? bg + (int64_t)t.jt * kBN * p.ldb : bg + (int64_t)t.jt * kBN;
    t.b_rv = (int)min64(kBN, p.cols_j - (int64_t)t.jt * kBN);
    t.pmax = p.P;
  } else if (MODE == MODE_CONTR) {
    t.a_base = p.A + t.g_off * p.lda + (int64_t)t.it * kBM;
    t.a_rv = (int)min64(kBM, p.rows_i - (int64_t)t.it * kBM);
    t.b_base = p.B + t.g_off * p.ldb + (int64_t)t.jt * kBN;
    t.b_rv = (int)min64(kBN, p.cols_j - (int64_t)t.jt * kBN);
    t.pmax = t.g_rows;
  } else {  // MODE_KCONTR: cpre = prefix of the groups' padded 128-element tiles
    const int64_t c0 = (int64_t)cpre[t.g] * kKcontrUnits;
    t.a_base = p.A + (int64_t)t.it * kBM * p.lda + c0;
    t.a_rv = (int)min64(kBM, p.rows_i - (int64_t)t.it * kBM);
    t.b_base = p.B + (int64_t)t.jt * kBN * p.ldb + c0;
    t.b_rv = (int)min64(kBN, p.cols_j - (int64_t)t.jt * kBN);
    t.pmax = (int64_t)(cpre[t.g + 1] - cpre[t.g]) * kKcontrUnits;
  }
  return t;
}

// ------------------------------------------------------- bias grad in wgrad --
// A wgrad tile (n tile it, k tile jt) streams the group's dy[:, n tile] through the
// ring as its A operand, MN-major: stage row p (a token row) holds the tile's 256
// n values, 16-byte chunk c in slot c ^ swz_m(p).  The tiles of the first k column
// also sum those rows: thread (row group rg = tid / 64, 4-column group c = tid % 64)
// adds rows rg, rg + 8, ..., rg + 56 of every stage into its own 4 fp32 slots of an
// LDS area [8][256]; at the end the 8 partials of each column are added and stored.
// db_g = sum over the group's rows of dy, read once for both outputs.  Rows past
// the group's end are zero in the ring, so they add nothing.  (Four columns per
// thread keep the extra registers few: the loop runs at the register limit.)
constexpr int kDbGroups = kThreads / 64;
constexpr int kDbLdsBytes = kDbGroups * 256 * 4;
static_assert(kThreads == 512 && kBK == 64, "bias-grad thread mapping");

__device__ __forceinline__ void db_zero(float *dbl) {
  *(float4 *)(dbl + (threadIdx.x >> 6) * 256 + (threadIdx.x & 63) * 4) = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <bool F16>
__device__ __forceinline__ void db_stage(const char *st, float *dbl) {
  const int c = threadIdx.x & 63, rg = threadIdx.x >> 6;
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int q = 0; q < kBK / kDbGroups; ++q) {
    const int r = rg + kDbGroups * q;
    const uint2 v = *(const uint2 *)(st + r * 512 + (((c >> 1) ^ swz_m(r)) << 4) + (c & 1) * 8);
    s0 += h16_to_f32<F16>((uint16_t)(v.x & 0xffffu));
    s1 += h16_to_f32<F16>((uint16_t)(v.x >> 16));
    s2 += h16_to_f32<F16>((uint16_t)(v.y & 0xffffu));
    s3 += h16_to_f32<F16>((uint16_t)(v.y >> 16));
  }
  float4 *slot = (float4 *)(dbl + rg * 256 + c * 4);
  float4 a = *slot;
  a.x += s0; a.y += s1; a.z += s2; a.w += s3;
  *slot = a;
}

__device__ __forceinline__ uintptr_t db_row(const Params &p, int g) {
  return p.db ? (uintptr_t)p.db + (uintptr_t)((int64_t)g * p.rows_i * (p.db_f32 ? 4 : 2)) : (uintptr_t)p.db_ptrs[g];
}

// Adds the kDbGroups partials of each column and stores db[g][n tile]; whole workgroup.
template <bool F16>
__device__ __forceinline__ void store_bgrad(const Params &p, const Tile &t, const float *dbl) {
  __syncthreads();  // every thread's last stage is in the partials
  const int col = threadIdx.x;
  if (col < t.a_rv) {
    float v = 0.f;
#pragma unroll
    for (int rg = 0; rg < kDbGroups; ++rg) v += dbl[rg * 256 + col];
    const uintptr_t row = db_row(p, t.g);
    const int64_t n = (int64_t)t.it * kBM + col;
    if (p.db_f32)
      ((GL_GLOBAL float *)row)[n] = v;
    else
      ((GL_GLOBAL uint16_t *)row)[n] = f32_to_h16<F16>(v);
  }
  __syncthreads();  // the partials area is free for the next tile
}

// An empty group whose wgrad is skipped (accumulate mode) still has db = 0.
__device__ __forceinline__ void store_bgrad_zero(const Params &p, const Tile &t) {
  const int col = threadIdx.x;
  if (col < t.a_rv) {
    const uintptr_t row = db_row(p, t.g);
    const int64_t n = (int64_t)t.it * kBM + col;
    if (p.db_f32)
      ((GL_GLOBAL float *)row)[n] = 0.f;
    else
      ((GL_GLOBAL uint16_t *)row)[n] = 0;
  }
}

// ------------------------------------------------------------- split tail --
// A launch's tiles go round the persistent grid.  When the last round would leave
// at least half the CUs idle (rem = tiles % grid <= grid / 2), each of those rem
// tiles is cut into S = grid / rem contraction ranges instead (at most kSplitSlots
// parts in all, each at least kMinSplitStages stages long), and the parts fill the
// last round.  Every part writes its fp32 accumulators to a partial slot of the
// workspace and counts itself in; the part that arrives last adds the S partials
// in part order -- a fixed order, so the result does not depend on which part
// finishes last -- and stores the tile.  No workgroup ever waits for another.
constexpr int kMinSplitStages = 4;

struct SplitPlan {
  int full;   // items [0, full) are whole tiles
  int rem;    // tiles [full, full + rem) are split
  int S;      // parts per split tile (1: nothing is split)
  int items;  // full + rem * S
};

// nk: contraction stages of every tile (the same for all tiles of a row-mode launch)
__device__ __forceinline__ SplitPlan split_plan(int tiles, int grid, int nk) {
  SplitPlan sp{tiles, 0, 1, tiles};
  const int rem = tiles % grid;
  if (rem == 0) return sp;
  int S = grid / rem;
  if (S * rem > kSplitSlots) S = kSplitSlots / rem;
  if (S > nk / kMinSplitStages) S = nk / kMinSplitStages;
  if (S < 2) return sp;
  sp.full = tiles - rem;
  sp.rem = rem;
  sp.S = S;
  sp.items = sp.full + rem * S;
  return sp;
}

// Part `part` of S of the u-th split tile is done: publish its partial; true when
// this workgroup arrived last and acc now holds the sum of all parts.  Called by
// the whole workgroup, as its last work item; `flag` is a workgroup-shared int.
// (The flag lives inside the kernel's one LDS array: a second __shared__ object
// makes the compiler wait for every direct-to-LDS load before each LDS read.)  The parts of the last
// round are items u + rem * part, so a part's CUs on one XCD run neighbouring tiles.
__device__ __forceinline__ bool split_finish(const WsView &ws, int u, int part, int S, f32x16_t (&acc)[kNI][kNJ],
                                             int *flag) {
  const int tid = threadIdx.x;
  constexpr size_t kSlotF4 = kPartialBytes / 16;
  GL_GLOBAL float4 *slots = (GL_GLOBAL float4 *)ws.split_part + (size_t)u * S * kSlotF4;
  GL_GLOBAL float4 *mine = slots + (size_t)part * kSlotF4;
#pragma unroll
  for (int ii = 0; ii < kNI; ++ii)
#pragma unroll
    for (int jj = 0; jj < kNJ; ++jj)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        mine[((ii * kNJ + jj) * 4 + c) * kThreads + tid] =
            make_float4(acc[ii][jj][4 * c], acc[ii][jj][4 * c + 1], acc[ii][jj][4 * c + 2], acc[ii][jj][4 * c + 3]);
  __threadfence();  // release: the partial is visible device-wide before the count
  __syncthreads();
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(ws.split_cnt + u, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const int last = old == S - 1;
    if (last) __hip_atomic_store(ws.split_cnt + u, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  // the same value in every lane; read as wave-uniform so control flow stays uniform
  if (!__builtin_amdgcn_readfirstlane(*flag)) return false;
  __threadfence();  // acquire: every part's partial
  for (int s = 0; s < S; ++s) {
    const GL_GLOBAL float4 *src = slots + (size_t)s * kSlotF4;
#pragma unroll
    for (int ii = 0; ii < kNI; ++ii)
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float4 o = src[((ii * kNJ + jj) * 4 + c) * kThreads + tid];
          if (s == 0) {
            acc[ii][jj][4 * c] = o.x; acc[ii][jj][4 * c + 1] = o.y;
            acc[ii][jj][4 * c + 2] = o.z; acc[ii][jj][4 * c + 3] = o.w;
          } else {
            acc[ii][jj][4 * c] += o.x; acc[ii][jj][4 * c + 1] += o.y;
            acc[ii][jj][4 * c + 2] += o.z; acc[ii][jj][4 * c + 3] += o.w;
          }
        }
  }
  return true;
}

// Stores a wave's 128 x 64 block of a tile: lane holds C[i][j..j+3] with
// i = ii*32 + lane%32, j = jj*32 + q4*8 + (lane/32)*4 (operands were swapped in
// the MFMAs for that); only rows < a_rv and columns < b_rv are written.
template <int MODE, bool F16 = false>
__device__ __forceinline__ void store_tile(const Params &p, const Tile &t, const f32x16_t (&acc)[kNI][kNJ], int wm,
                                           int wn, int lane) {
  char *cbase;
  int64_t row0;
  if (MODE == MODE_ROWS) {
    cbase = (char *)p.C;
    row0 = t.g_off + (int64_t)t.it * kBM;
  } else {
    cbase = p.C ? (char *)p.C + (int64_t)t.g * p.c_gstride * (p.out_f32 ? 4 : 2) : (char *)p.C_ptrs[t.g];
    row0 = (int64_t)t.it * kBM;
  }
  const char *bias_g = nullptr;
  if (p.bias) bias_g = (const char *)p.bias + (int64_t)t.g * p.cols_j * (p.out_f32 ? 4 : 2);
  else if (p.bias_ptrs) bias_g = (const char *)p.bias_ptrs[t.g];
#pragma unroll
  for (int ii = 0; ii < kNI; ++ii) {
    const int il = wm * kWTM + ii * 32 + (lane & 31);
    if (il >= t.a_rv) continue;
    const int64_t row = row0 + il;
#pragma unroll
    for (int jj = 0; jj < kNJ; ++jj) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int jl = wn * kWTN + jj * 32 + q4 * 8 + (lane >> 5) * 4;
        if (jl >= t.b_rv) continue;
        store4<F16>((uintptr_t)cbase, row, p.ldc, (int64_t)t.jt * kBN + jl, (uintptr_t)bias_g, p.out_f32, p.accumulate,
                    acc[ii][jj][q4 * 4 + 0],
               acc[ii][jj][q4 * 4 + 1], acc[ii][jj][q4 * 4 + 2], acc[ii][jj][q4 * 4 + 3]);
      }
    }
  }
}

// 16-bit output without accumulate, staged through the idle stage ring so that
// every store instruction writes whole cache lines.  Written directly, each store
// instruction would touch 32 rows with 16 bytes each, and every 128-byte line of the
// output would be assembled in L2 from 8 partial writes; on the MXFP8 wgrad (short
// contractions, a 1 GiB output) that epilogue took half the kernel's time.
// The tile goes to LDS as [256 rows][512 B] (16-byte slot s of row r at slot
// s ^ (r % 32), so the 32 rows one write instruction touches spread over the
// banks), then each wave stores 2 rows x 512 B per instruction.  Whole workgroup;
// needs 128 KiB of `lds`, which no wave may still be reading on entry.
template <int MODE, bool F16>
__device__ __forceinline__ void store_tile_lds(const Params &p, const Tile &t, const f32x16_t (&acc)[kNI][kNJ],
                                               int wm, int wn, int lane, char *lds) {
  uintptr_t cbase;
  int64_t row0;
  if (MODE == MODE_ROWS) {
    cbase = (uintptr_t)p.C;
    row0 = t.g_off + (int64_t)t.it * kBM;
  } else {
    cbase = p.C ? (uintptr_t)p.C + (uintptr_t)((int64_t)t.g * p.c_gstride * 2) : (uintptr_t)p.C_ptrs[t.g];
    row0 = (int64_t)t.it * kBM;
  }
  uintptr_t bias_g = 0;
  if (p.bias) bias_g = (uintptr_t)p.bias + (uintptr_t)((int64_t)t.g * p.cols_j * 2);
  else if (p.bias_ptrs) bias_g = (uintptr_t)p.bias_ptrs[t.g];
  __syncthreads();  // a split tile's arrival flag sits in the ring's first word
#pragma unroll
  for (int ii = 0; ii < kNI; ++ii) {
    const int il = wm * kWTM + ii * 32 + (lane & 31);
#pragma unroll
    for (int jj = 0; jj < kNJ; ++jj) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int jl = wn * kWTN + jj * 32 + q4 * 8 + (lane >> 5) * 4;
        float v0 = acc[ii][jj][q4 * 4 + 0], v1 = acc[ii][jj][q4 * 4 + 1];
        float v2 = acc[ii][jj][q4 * 4 + 2], v3 = acc[ii][jj][q4 * 4 + 3];
        if (bias_g && jl < t.b_rv) {
          const uint2 bv = *(const GL_GLOBAL uint2 *)(bias_g + ((int64_t)t.jt * kBN + jl) * 2);
          v0 += h16_to_f32<F16>(bv.x & 0xffff); v1 += h16_to_f32<F16>(bv.x >> 16);
          v2 += h16_to_f32<F16>(bv.y & 0xffff); v3 += h16_to_f32<F16>(bv.y >> 16);
        }
        const int slot = jl >> 3, half = (jl >> 2) & 1;
        *(uint2 *)(lds + il * 512 + ((slot ^ (il & 31)) << 4) + half * 8) =
            make_uint2((uint32_t)f32_to_h16<F16>(v0) | ((uint32_t)f32_to_h16<F16>(v1) << 16),
                       (uint32_t)f32_to_h16<F16>(v2) | ((uint32_t)f32_to_h16<F16>(v3) << 16));
      }
    }
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, s = lane & 31;
#pragma unroll 4
  for (int it = 0; it < kBM / kWaves / 2; ++it) {
    const int r = wave * (kBM / kWaves) + it * 2 + (lane >> 5);
    if (r < t.a_rv && s * 8 < t.b_rv) {
      const uint4 v = *(const uint4 *)(lds + r * 512 + ((s ^ (r & 31)) << 4));
      *(GL_GLOBAL uint4 *)(cbase + ((row0 + r) * p.ldc + (int64_t)t.jt * kBN + s * 8) * 2) = v;
    }
  }
  __syncthreads();  // the ring is refilled by the next tile
}
static_assert(kS * kStageBytes >= kBM * kBN * 2, "the staged epilogue needs the whole tile in the ring");

// Compute units of the current device (one persistent workgroup per CU).
inline int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || n <= 0)
    n = 256;
  return n;
}

inline int persistent_grid(int64_t max_items) {
  const int cus = num_cus();
  int64_t g = max_items < cus ? max_items : cus;
  if (g >= 8) g &= ~7;  // keeps the XCD-aware remap a bijection
  return (int)(g > 0 ? g : 1);
}

}  // namespace gemm
}  // namespace gl
