// Internal definitions shared by the gfx950 kernels and the host entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gl {

// ----------------------------------------------------------------- workspace --
// Layout of the caller-provided workspace written by the offsets kernel:
//   [0]   WsHeader (32 bytes)
//   [32]  int64 offsets[G+1]
//   then  int32 row-tile prefix tables, one per row-tile height in kTileRows:
//         pre[g] = sum_{h<g} ceil(m_h / rows), pre[G] = total row tiles.
//   then  (1 KiB aligned) the split-contraction area of the GEMMs: int32 arrival
//         counters[kSplitSlots] (zeroed by the offsets kernel, left zero by every
//         GEMM launch), then kSplitSlots fp32 partial tiles of kPartialBytes each.
struct WsHeader {
  int32_t status;      // GL_STATUS_* bits, 0 = valid splits
  int32_t num_groups;
  int64_t total_rows;
  int32_t magic;
  int32_t pad[3];
};
static_assert(sizeof(WsHeader) == 32, "workspace header is 32 bytes");

constexpr int32_t kWsMagic = 0x474c5753;  // "GLWS"
constexpr int kNumTileRows = 4;
constexpr int kTileRows[kNumTileRows] = {32, 64, 128, 256};

__host__ __device__ inline int tile_rows_index(int rows) {
  return rows == 32 ? 0 : rows == 64 ? 1 : rows == 128 ? 2 : 3;
}
__host__ __device__ inline size_t ws_offsets_byte(int) { return 32; }
__host__ __device__ inline size_t ws_prefix_byte(int G, int idx) {
  size_t base = 32 + 8 * (size_t)(G + 1);
  return base + (size_t)idx * 4 * (size_t)(G + 1);
}
// A GEMM launch splits at most kSplitSlots tile parts over the contraction; each
// part leaves one 256 x 256 fp32 partial tile.
constexpr int kSplitSlots = 256;
constexpr size_t kPartialBytes = 256 * 256 * 4;
__host__ __device__ inline size_t ws_split_byte(int G) {
  return (ws_prefix_byte(G, kNumTileRows) + 1023) & ~(size_t)1023;
}
__host__ __device__ inline size_t ws_bytes(int G) {
  return ws_split_byte(G) + 4 * kSplitSlots + (size_t)kSplitSlots * kPartialBytes;
}

struct WsView {
  WsHeader *hdr;
  const int64_t *off;
  const int32_t *pre[kNumTileRows];
  int32_t *split_cnt;   // [kSplitSlots]
  float *split_part;    // [kSplitSlots][kPartialBytes / 4]
};
__host__ __device__ inline WsView ws_view(const void *ws, int G) {
  WsView v;
  char *b = (char *)ws;
  v.hdr = (WsHeader *)b;
  v.off = (const int64_t *)(b + ws_offsets_byte(G));
  for (int i = 0; i < kNumTileRows; ++i) v.pre[i] = (const int32_t *)(b + ws_prefix_byte(G, i));
  v.split_cnt = (int32_t *)(b + ws_split_byte(G));
  v.split_part = (float *)(b + ws_split_byte(G) + 4 * kSplitSlots);
  return v;
}

// Kernels that consume a workspace first check that the offsets kernel produced it
// for the same (G, T) and found the splits valid; otherwise they write nothing.
__device__ inline bool ws_usable(const WsHeader *h, int G, int64_t T) {
  int32_t st = h->status;
  if (h->magic != kWsMagic || h->num_groups != G || h->total_rows != T) {
    if (threadIdx.x == 0) atomicOr((int *)&h->status, 4);
    return false;
  }
  return st == 0;
}

__host__ __device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// Index of the group owning row tile q: the last g with pre[g] <= q (pre is the
// non-decreasing exclusive prefix of per-group tile counts, pre[G] = total).
// The whole wave searches: each lane tests a slice of pre[] and the ballots count.
__device__ __forceinline__ int find_group(const int32_t *__restrict__ pre, int G, int q) {
  const int lane = threadIdx.x & 63;
  int count = 0;
  for (int base = 0; base <= G; base += 64) {
    const int idx = base + lane;
    const bool le = idx <= G && pre[idx] <= q;
    count += __popcll(__ballot(le));
  }
  return count - 1;
}

// ---------------------------------------------------------------- bf16 helpers --
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round-to-nearest-even float -> bfloat16 bits; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// fp16 <-> fp32 (the float -> half conversion rounds to nearest even; overflow gives inf)
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }
// 16-bit storage type of a kernel's inputs / 16-bit outputs: bf16 or fp16
template <bool F16>
__device__ __forceinline__ float h16_to_f32(uint16_t h) { return F16 ? f16_to_f32(h) : bf16_to_f32(h); }
template <bool F16>
__device__ __forceinline__ uint16_t f32_to_h16(float f) { return F16 ? f32_to_f16(f) : f32_to_bf16(f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

}  // namespace gl
