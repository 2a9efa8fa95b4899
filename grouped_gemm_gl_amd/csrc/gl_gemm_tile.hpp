// Tile machinery shared by the gfx950 MFMA grouped GEMMs (bf16 and MXFP8): tile
// shape, direct buffer->LDS operand streams, LDS layouts and their fragment
// readers, work-item decode and the output store.  See gl_gemm_bf16.hip for how
// the pieces fit together.
#pragma once

#include <atomic>
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
static_assert(5 * kOpBytes <= 160 * 1024, "direct-load ring with three weight slots");
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
// c ^ swz_m(p).  The rows are 512 bytes apart (same banks).  A 32x32x16 transpose
// read serves rows p .. p + 3 x 64 bytes per 32 lanes: bits 2-3 of the slot move
// each row's 64 bytes to its own quarter of the 256-byte window.  A 16x16x32
// transpose read serves rows p .. p + 3 and p + 8 .. p + 11 x 32 bytes: bit 1 of
// the slot then separates p from p + 8.
__device__ __forceinline__ int swz_k(int r) { return (r / (16 / kChunks)) & (kChunks - 1); }
__device__ __forceinline__ int swz_m(int p) { return ((p & 3) << 2) | (((p >> 3) & 1) << 1); }

__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0f70); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }
// s_waitcnt vmcnt(n) (lgkmcnt and expcnt left at their maxima), gfx9 encoding
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// A pointer the whole wave holds, made visibly wave-uniform (scalar registers).  A
// per-group pointer loaded from a pointer array is otherwise taken as varying per
// lane, and every buffer load through a resource built from it may become a loop
// over the distinct values (readfirstlane, compare, exec mask) -- five of them per
// stage in the MXFP8 forward.  Each half is read as unsigned, so the high word is
// not sign-extended.  (Applied where the compiler made such loops: in the bf16
// forward on the two-slot ring, whose steady loop had none, it measured 2.6%
// slower.)
template <class T>
__device__ __forceinline__ T *uniform_ptr(T *q) {
  const uint64_t v = (uint64_t)(uintptr_t)q;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (T *)(uintptr_t)(((uint64_t)hi << 32) | lo);
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

  // Register staging: this lane's pieces of stage t into r (global -> VGPRs), written
  // to the ring later by write_regs at the same LDS places the direct loads fill.
  __device__ __forceinline__ void load_regs(int t, uint4 (&r)[kQ]) const {
    const __amdgpu_buffer_rsrc_t rs = rsrc_at(base + (int64_t)t * step);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off[q], 0, 0);
      r[q] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
  // The last stage of a contraction: pieces past pmax are zeros.  (The count of
  // valid contraction indices left is wave-uniform and at most kBK, so the per-lane
  // test is a 32-bit compare.)
  __device__ __forceinline__ void load_regs_masked(int t, int64_t pmax, uint4 (&r)[kQ], int wave, int lane) const {
    const __amdgpu_buffer_rsrc_t rs = rsrc_at(base + (int64_t)t * step);
    const int left = (int)min64(pmax - (int64_t)t * kBK, kBK);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int u = wave + kWaves * q;
      const int pfirst =
          KMAJ ? ((lane % kChunks) ^ swz_k(kRowsPerPiece * u + lane / kChunks)) * 8 : 2 * u + (lane >> 5);
      if (pfirst < left) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, off[q], 0, 0);
        r[q] = make_uint4(v[0], v[1], v[2], v[3]);
      } else {
        r[q] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void write_regs(char *st, const uint4 (&r)[kQ], int wave, int lane) const {
#pragma unroll
    for (int q = 0; q < kQ; ++q) *(uint4 *)(st + (wave + kWaves * q) * 1024 + lane * 16) = r[q];
  }

  // The last stage of a contraction: lanes whose piece lies past pmax write zeros
  // into their LDS slot instead of loading.
  __device__ __forceinline__ void issue_masked(int t, int64_t pmax, char *st, int wave, int lane) const {
    const __amdgpu_buffer_rsrc_t r = rsrc_at(base + (int64_t)t * step);
    const int left = (int)min64(pmax - (int64_t)t * kBK, kBK);
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int u = wave + kWaves * q;
      char *dst = st + u * 1024;
      // first contraction index (within the stage) this lane's piece holds
      const int pfirst =
          KMAJ ? ((lane % kChunks) ^ swz_k(kRowsPerPiece * u + lane / kChunks)) * 8 : 2 * u + (lane >> 5);
      if (pfirst < left)
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

// 16x16x32 operand fragment (16 rows/columns x 32 contraction values; lane l holds
// row l % 16, contraction values 8 (l / 16) + 0..7) for the 32-deep step s of a stage.
constexpr int kNI16 = kWTM / 16, kNJ16 = kWTN / 16;  // 16x16 MFMA blocks per wave
__device__ __forceinline__ bf16x8_t frag16_kmaj(const char *st, int row0, int s, int lane) {
  const int r = row0 + (lane & 15);
  const int c = 4 * s + (lane >> 4);
  return *(const bf16x8_t *)(st + r * kRowB + ((c ^ swz_k(r)) << 4));
}

__device__ __forceinline__ bf16x8_t frag16_mnmaj(const char *st, int col0, int s, int lane) {
  // lane q of a 16-lane group names contraction row q / 4 and columns 4 (q % 4) .. + 3
  // of the group's 4 rows; the transpose hands lane q column q of those rows.  Group
  // g (lanes 16 g ..) takes contraction rows 8 g .. 8 g + 7 of the step.
  const int q = lane & 15, grp = lane >> 4;
  const int col = col0 + ((q & 3) << 2);
  const int chunk = col >> 3, within = col & 7;
  v4i16 h[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int prow = s * 32 + grp * 8 + t * 4 + (q >> 2);
    const char *a = st + prow * 512 + ((chunk ^ swz_m(prow)) << 4) + within * 2;
    h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GL_LDS v4i16 *)a);
  }
  const v8i16 v = {h[0][0], h[0][1], h[0][2], h[0][3], h[1][0], h[1][1], h[1][2], h[1][3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// ------------------------------------------------------ accumulator layouts --
// A wave's 128 x 64 block of fp32 accumulators in the two MFMA shapes, seen as 32
// "quads" per lane: 4 consecutive output columns (il, jl .. jl + 3) of one row
// (operands are swapped in the MFMAs so a lane's 4 values run along a row).
//   32x32x16: 4 x 2 blocks of f32x16; quad q = (ii, jj, q4) holds row ii*32 + l%32,
//             columns jj*32 + q4*8 + (l/32)*4 ..
//   16x16x32: 8 x 4 blocks of f32x4; quad q = (ii, jj) holds row ii*16 + l%16,
//             columns jj*16 + (l/16)*4 ..
typedef f32x16_t Acc32[kNI][kNJ];
typedef f32x4_t Acc16[kNI16][kNJ16];
constexpr int kQuads = 32;

template <class ACC>
struct AccLayout;
template <>
struct AccLayout<Acc32> {
  // a lane's column in quad q depends only on q % kColGroups
  static constexpr int kColGroups = 8;
  __device__ static __forceinline__ void pos(int q, int lane, int &il, int &jl) {
    il = (q >> 3) * 32 + (lane & 31);
    jl = ((q >> 2) & 1) * 32 + (q & 3) * 8 + (lane >> 5) * 4;
  }
  __device__ static __forceinline__ float4 get(const Acc32 &a, int q) {
    const f32x16_t &v = a[q >> 3][(q >> 2) & 1];
    const int b = (q & 3) * 4;
    return make_float4(v[b], v[b + 1], v[b + 2], v[b + 3]);
  }
  __device__ static __forceinline__ void set(Acc32 &a, int q, float4 o) {
    f32x16_t &v = a[q >> 3][(q >> 2) & 1];
    const int b = (q & 3) * 4;
    v[b] = o.x; v[b + 1] = o.y; v[b + 2] = o.z; v[b + 3] = o.w;
  }
  __device__ static __forceinline__ void zero(Acc32 &a) {
#pragma unroll
    for (int ii = 0; ii < kNI; ++ii)
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj)
#pragma unroll
        for (int e = 0; e < 16; ++e) a[ii][jj][e] = 0.f;
  }
};
template <>
struct AccLayout<Acc16> {
  static constexpr int kColGroups = 4;
  __device__ static __forceinline__ void pos(int q, int lane, int &il, int &jl) {
    il = (q >> 2) * 16 + (lane & 15);
    jl = (q & 3) * 16 + (lane >> 4) * 4;
  }
  __device__ static __forceinline__ float4 get(const Acc16 &a, int q) {
    const f32x4_t &v = a[q >> 2][q & 3];
    return make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ static __forceinline__ void set(Acc16 &a, int q, float4 o) {
    a[q >> 2][q & 3] = (f32x4_t){o.x, o.y, o.z, o.w};
  }
  __device__ static __forceinline__ void zero(Acc16 &a) {
#pragma unroll
    for (int ii = 0; ii < kNI16; ++ii)
#pragma unroll
      for (int jj = 0; jj < kNJ16; ++jj) a[ii][jj] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  }
};

// Stores 4 consecutive output columns of one row, optionally adding the existing
// values (accumulate).  16-bit outputs are bf16, or fp16 when F16.
// Addresses arrive as integers: a cast of a generic pointer to the global address
// space can be folded back to a flat access when the pointer is a select of a
// kernel argument and a loaded one; an integer cannot.
template <bool F16>
__device__ __forceinline__ void store4(uintptr_t cbase, int64_t row, int64_t ldc, int64_t col, int out_f32,
                                      int accumulate, float v0, float v1, float v2, float v3) {
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
    // (value by value: measured faster here than the pair conversion in the forward)
    *dst = make_uint2((uint32_t)f32_to_h16<F16>(v0) | ((uint32_t)f32_to_h16<F16>(v1) << 16),
                      (uint32_t)f32_to_h16<F16>(v2) | ((uint32_t)f32_to_h16<F16>(v3) << 16));
  }
}

// One output tile of one group: what a work item decodes to.
struct Tile {
  int g, it, jt;
  int64_t g_off, g_rows;
  const uint16_t *a_base, *b_base;  // operand tile bases at contraction 0
  int a_rv, b_rv;                   // valid rows of the A and B tiles
  bool ok;                          // device-check build: the item lies inside the launch
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
    t.ok = t.g >= 0 && t.g < p.G;
    if (GL_DEVICE_CHECKS && !t.ok) return t;
    local = w - pre[t.g] * NT;
    MT = pre[t.g + 1] - pre[t.g];
  } else {
    const int per = p.tiles_i * NT;
    t.g = w / per;
    t.ok = w >= 0 && t.g < p.G;
    if (GL_DEVICE_CHECKS && !t.ok) return t;
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
  if (GL_DEVICE_CHECKS) {
    t.ok = MT > 0 && local >= 0 && local < MT * NT && t.it < MT && t.jt < NT && t.g_off >= 0 && t.g_rows >= 0 &&
           t.g_off + t.g_rows <= p.T;
    if (MODE == MODE_ROWS) t.ok = t.ok && (int64_t)t.it * kBM < t.g_rows;
    if (MODE == MODE_KCONTR) t.ok = t.ok && cpre[t.g] >= 0 && cpre[t.g + 1] >= cpre[t.g];
    if (!t.ok) return t;
  }
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
// A wgrad tile (n tile it, k tile jt) streams the group's dy[:, n tile] as its A
// operand, MN-major, through the staging registers: piece q of a lane holds the 8
// columns c*8 .. c*8 + 7 of contraction row p = 2 (wave + 8 q) + lane / 32, with
// c = (lane % 32) ^ swz_m(p).  The swizzle of p does not depend on q, so a lane's
// pieces of every stage cover the same 8 columns: the tiles of one k column per
// group add each stage's pieces, as they come in, into 8 fp32 column sums per lane (rows
// past the group's end are zero pieces and add nothing).  The sums live in the
// lane's own 32-byte slot of an LDS area beside the stage ring, not in registers:
// 8 registers held across the contraction loop made the compiler spill inside it.
// At the end the 16 partial sums of each column (8 waves x 2 lane halves) are added
// in a fixed order.  db_g = sum over the group's rows of dy, read once for both
// outputs.
constexpr int kDbParts = 2 * kWaves;
constexpr int kDbLdsBytes = kDbParts * 256 * 4;
static_assert(kThreads == 512 && kBK == 64 && kQ == 4, "bias-grad lane mapping");

// first tile column this lane's bias-grad sums cover
__device__ __forceinline__ int db_col(int wave, int lane) {
  return ((lane & 31) ^ swz_m(2 * wave + (lane >> 5))) * 8;
}

// This lane's slot of the bias-grad area `dbl` (kDbLdsBytes): part 2 wave + lane / 32,
// columns db_col .. + 7.
__device__ __forceinline__ float *db_slot(float *dbl, int wave, int lane) {
  return dbl + (2 * wave + (lane >> 5)) * 256 + db_col(wave, lane);
}

__device__ __forceinline__ void db_zero(float *slot) {
  *(float4 *)slot = make_float4(0.f, 0.f, 0.f, 0.f);
  *(float4 *)(slot + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
}

// Adds the rows of this lane's staged pieces into its 8 column sums.  bf16: pieces
// q and q + 1 hold the same columns of two rows, so one byte permute pairs a column's
// two values and one v_dot2_f32_bf16 against (1, 1) adds both into the column's sum
// (two VALU instructions per column and pair of rows instead of four: this add sits
// between the two MFMA steps of a stage).  fp16: one conversion and one add per value.
template <bool F16>
__device__ __forceinline__ void db_add(float *slot, const uint4 (&r)[kQ]) {
  const float4 lo = *(const float4 *)slot, hi = *(const float4 *)(slot + 4);
  float dbr[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  if constexpr (!F16) {
    static_assert(kQ % 2 == 0, "pieces pair up");
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
    const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
#pragma unroll
    for (int q = 0; q < kQ; q += 2) {
      const uint32_t a[4] = {r[q].x, r[q].y, r[q].z, r[q].w};
      const uint32_t b[4] = {r[q + 1].x, r[q + 1].y, r[q + 1].z, r[q + 1].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // byte pool {b, a}, a in bytes 0-3: pl = low halves (a in its low half), ph = high halves
        const uint32_t pl = __builtin_amdgcn_perm(b[e], a[e], 0x05040100u);
        const uint32_t ph = __builtin_amdgcn_perm(b[e], a[e], 0x07060302u);
        dbr[2 * e] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pl), one, dbr[2 * e], false);
        dbr[2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ph), one, dbr[2 * e + 1], false);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const uint32_t d[4] = {r[q].x, r[q].y, r[q].z, r[q].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dbr[2 * e] += h16_to_f32<F16>((uint16_t)(d[e] & 0xffffu));
        dbr[2 * e + 1] += h16_to_f32<F16>((uint16_t)(d[e] >> 16));
      }
    }
  }
  *(float4 *)slot = make_float4(dbr[0], dbr[1], dbr[2], dbr[3]);
  *(float4 *)(slot + 4) = make_float4(dbr[4], dbr[5], dbr[6], dbr[7]);
}

__device__ __forceinline__ uintptr_t db_row(const Params &p, int g) {
  return p.db ? (uintptr_t)p.db + (uintptr_t)((int64_t)g * p.rows_i * (p.db_f32 ? 4 : 2)) : (uintptr_t)p.db_ptrs[g];
}

// The bias-grad column sums of the whole workgroup: thread t < 256 returns column
// t's total over the kDbParts partials in `dbl`, added in a fixed order.  Whole
// workgroup.
__device__ __forceinline__ float db_reduce(const float *dbl) {
  __syncthreads();
  float v = 0.f;
  if (threadIdx.x < 256) {
#pragma unroll
    for (int k = 0; k < kDbParts; ++k) v += dbl[k * 256 + threadIdx.x];
  }
  __syncthreads();  // the partials area is free for the next tile
  return v;
}

// Stores column t = threadIdx.x of db[g][n tile] (v from db_reduce).
template <bool F16>
__device__ __forceinline__ void store_bgrad(const Params &p, const Tile &t, float v) {
  const int col = threadIdx.x;
  if (col < t.a_rv) {
    const uintptr_t row = db_row(p, t.g);
    const int64_t n = (int64_t)t.it * kBM + col;
    if (p.db_f32)
      ((GL_GLOBAL float *)row)[n] = v;
    else
      ((GL_GLOBAL uint16_t *)row)[n] = f32_to_h16<F16>(v);
  }
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

// nk: contraction stages of every tile (the same for all tiles of a row-mode launch);
// slots: partial-tile slots of the workspace
__device__ __forceinline__ SplitPlan split_plan(int tiles, int grid, int nk, int slots) {
  SplitPlan sp{tiles, 0, 1, tiles};
  const int rem = tiles % grid;
  if (rem == 0) return sp;
  int S = grid / rem;
  if (S * rem > slots) S = slots / rem;
  if (S > nk / kMinSplitStages) S = nk / kMinSplitStages;
  if (S < 2) return sp;
  sp.full = tiles - rem;
  sp.rem = rem;
  sp.S = S;
  sp.items = sp.full + rem * S;
  return sp;
}

// Part `part` of S of the u-th split tile is done: publish its partial (into slot
// slot0 + part); true when this workgroup arrived last and acc now holds the sum
// of all parts.  Called by the whole workgroup; `flag` is a workgroup-shared int.
// (The flag lives inside the kernel's one LDS array: a second __shared__ object
// makes the compiler wait for every direct-to-LDS load before each LDS read.)  The parts of the last
// round are items u + rem * part, so a part's CUs on one XCD run neighbouring tiles.
template <class ACC>
__device__ __forceinline__ bool split_finish(const WsView &ws, int u, int slot0, int part, int S, ACC &acc,
                                             int *flag) {
  using L = AccLayout<ACC>;
  const int tid = threadIdx.x;
  constexpr size_t kSlotF4 = kPartialBytes / 16;
  GL_GLOBAL float4 *slots = (GL_GLOBAL float4 *)ws.split_part + (size_t)slot0 * kSlotF4;
  GL_GLOBAL float4 *mine = slots + (size_t)part * kSlotF4;
#pragma unroll
  for (int q = 0; q < kQuads; ++q) mine[q * kThreads + tid] = L::get(acc, q);
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
    for (int q = 0; q < kQuads; ++q) {
      const float4 o = src[q * kThreads + tid];
      if (s == 0) {
        L::set(acc, q, o);
      } else {
        const float4 c = L::get(acc, q);
        L::set(acc, q, make_float4(c.x + o.x, c.y + o.y, c.z + o.z, c.w + o.w));
      }
    }
  }
  return true;
}

// Stores a wave's 128 x 64 block of a tile, quad by quad (see AccLayout); only rows
// < a_rv and columns < b_rv are written.  The optional bias (per output column, of
// the output's type) is added to the fp32 sum first; a lane's column depends only
// on q % kColGroups, so its bias values are loaded once per distinct column, ahead
// of the stores (loaded beside each store, every quad waited for its load: the
// compiler cannot move a load above a store that may alias it), or read from
// `bias_lds` when the caller staged the tile's 16-bit bias there.  BIAS: the kernel
// takes a bias at all (the forward); the others carry no bias code or registers.
template <int MODE, bool F16, bool BIAS, class ACC>
__device__ __forceinline__ void store_tile(const Params &p, const Tile &t, const ACC &acc, int wm, int wn, int lane,
                                           const char *bias_lds = nullptr) {
  using L = AccLayout<ACC>;
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
  if (BIAS && p.bias) bias_g = (const char *)p.bias + (int64_t)t.g * p.cols_j * (p.out_f32 ? 4 : 2);
  else if (BIAS && p.bias_ptrs) bias_g = (const char *)p.bias_ptrs[t.g];
  float4 bv[L::kColGroups];
#pragma unroll
  for (int c = 0; c < L::kColGroups; ++c) {
    int il, jl;
    L::pos(c, lane, il, jl);
    const int64_t col = (int64_t)t.jt * kBN + jl + wn * kWTN;
    bv[c] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (BIAS && bias_g && bias_lds) {  // the tile's 16-bit bias, staged in LDS
      const uint2 u = *(const uint2 *)(bias_lds + (jl + wn * kWTN) * 2);
      bv[c] = make_float4(h16_to_f32<F16>(u.x & 0xffff), h16_to_f32<F16>(u.x >> 16),
                          h16_to_f32<F16>(u.y & 0xffff), h16_to_f32<F16>(u.y >> 16));
    } else if (BIAS && bias_g && jl + wn * kWTN < t.b_rv) {
      if (p.out_f32) {
        bv[c] = *(const GL_GLOBAL float4 *)((uintptr_t)bias_g + col * 4);
      } else {
        const uint2 u = *(const GL_GLOBAL uint2 *)((uintptr_t)bias_g + col * 2);
        bv[c] = make_float4(h16_to_f32<F16>(u.x & 0xffff), h16_to_f32<F16>(u.x >> 16),
                            h16_to_f32<F16>(u.y & 0xffff), h16_to_f32<F16>(u.y >> 16));
      }
    }
  }
  // the lane index, opaque to the compiler here, so that the per-quad addresses are
  // computed per tile instead of being hoisted out of the tile loop and spilled
  // (measured: dgrad and wgrad faster; the forward, with its bias, slower)
  int lane_t = lane;
  if (!BIAS) asm volatile("" : "+v"(lane_t));
#pragma unroll
  for (int q = 0; q < kQuads; ++q) {
    int il, jl;
    L::pos(q, lane_t, il, jl);
    il += wm * kWTM;
    jl += wn * kWTN;
    if (il >= t.a_rv || jl >= t.b_rv) continue;
    float4 v = L::get(acc, q);
    if (BIAS && bias_g) {
      const float4 c = bv[q % L::kColGroups];
      v.x += c.x; v.y += c.y; v.z += c.z; v.w += c.w;
    }
    store4<F16>((uintptr_t)cbase, row0 + il, p.ldc, (int64_t)t.jt * kBN + jl, p.out_f32, p.accumulate, v.x, v.y,
                v.z, v.w);
  }
}

// 16-bit output without accumulate, staged through the idle stage ring so that
// every store instruction writes whole cache lines.  Written directly, each store
// instruction would touch 32 (or 16) rows with 16 (or 32) bytes each, and every
// 128-byte line of the output would be assembled in L2 from partial writes; on the
// MXFP8 wgrad (short contractions, a 1 GiB output) that epilogue took half the
// kernel's time.  The tile goes to LDS as [256 rows][512 B] (16-byte slot s of row r
// at slot s ^ (r % 32), so the rows one write instruction touches spread over the
// banks), then each wave stores 2 rows x 512 B per instruction.  Whole workgroup;
// needs 128 KiB of `lds`, which no wave may still be reading on entry.
template <int MODE, bool F16, class ACC>
__device__ __forceinline__ void store_tile_lds(const Params &p, const Tile &t, const ACC &acc, int wm, int wn,
                                               int lane, char *lds, const char *bias_lds = nullptr) {
  // bias_lds: the tile's 16-bit bias, staged in LDS outside the first 128 KiB (the
  // forward); null for the others.
  using L = AccLayout<ACC>;
  uintptr_t cbase;
  int64_t row0;
  if (MODE == MODE_ROWS) {
    cbase = (uintptr_t)p.C;
    row0 = t.g_off + (int64_t)t.it * kBM;
  } else {
    cbase = p.C ? (uintptr_t)p.C + (uintptr_t)((int64_t)t.g * p.c_gstride * 2) : (uintptr_t)p.C_ptrs[t.g];
    row0 = (int64_t)t.it * kBM;
  }
  __syncthreads();  // a split tile's arrival flag sits in the ring's first word
  // the lane index opaque, as in store_tile, so that the per-row offsets are not
  // hoisted out of the tile loop and spilled (measured: faster in the bf16 wgrad and
  // dgrad, not in the MXFP8 wgrad)
  int lane_t = lane;
  if (MODE != MODE_KCONTR) asm volatile("" : "+v"(lane_t));
#pragma unroll
  for (int q = 0; q < kQuads; ++q) {
    int il, jl;
    L::pos(q, lane_t, il, jl);
    il += wm * kWTM;
    jl += wn * kWTN;
    float4 v = L::get(acc, q);
    if (bias_lds) {
      const uint2 u = *(const uint2 *)(bias_lds + jl * 2);
      v.x += h16_to_f32<F16>(u.x & 0xffff); v.y += h16_to_f32<F16>(u.x >> 16);
      v.z += h16_to_f32<F16>(u.y & 0xffff); v.w += h16_to_f32<F16>(u.y >> 16);
    }
    const int slot = jl >> 3, half = (jl >> 2) & 1;
    *(uint2 *)(lds + il * 512 + ((slot ^ (il & 31)) << 4) + half * 8) =
        make_uint2(pack_h16x2<F16>(v.x, v.y), pack_h16x2<F16>(v.z, v.w));
  }
  __syncthreads();
  // The stores go through a buffer resource over the tile's output block, from its
  // first element: a lane outside the block stores at an offset past the resource's
  // end, which the hardware drops.  So every store is issued unconditionally, and
  // each group of four rows has its LDS reads in flight together (guarded stores
  // each waited for their own read).  Offsets: r < 256 rows of at most 2^22
  // columns, under 2^31 bytes.
  const int wave = threadIdx.x >> 6, s = lane_t & 31;
  const __amdgpu_buffer_rsrc_t rs =
      rsrc_at(uniform_ptr((const char *)(cbase + (uintptr_t)(row0 * p.ldc + (int64_t)t.jt * kBN) * 2)));
  const bool col_ok = s * 8 < t.b_rv;
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  constexpr int kRowsPerWave = kBM / kWaves, kIters = kRowsPerWave / 2, kBatch = 4;
#pragma unroll
  for (int it0 = 0; it0 < kIters; it0 += kBatch) {
    u32x4_t v[kBatch];
    uint32_t o[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int r = wave * kRowsPerWave + (it0 + k) * 2 + (lane_t >> 5);
      v[k] = *(const u32x4_t *)(lds + r * 512 + ((s ^ (r & 31)) << 4));
      o[k] = r < t.a_rv && col_ok ? (uint32_t)(((int64_t)r * p.ldc + s * 8) * 2) : 0x80000000u;
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) __builtin_amdgcn_raw_buffer_store_b128(v[k], rs, o[k], 0, 0);
  }
  __syncthreads();  // the ring is refilled by the next tile
}
static_assert(kS * kStageBytes >= kBM * kBN * 2, "the staged epilogue needs the whole tile in the ring");

// Compute units of the current device (one persistent workgroup per CU), queried
// once per device and cached.
constexpr int kMaxDevices = 64;
inline int num_cus() {
  static std::atomic<int> cached[kMaxDevices];  // 0: not queried yet
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < kMaxDevices && (n = cached[dev].load(std::memory_order_relaxed)) > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev >= 0 && dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
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
