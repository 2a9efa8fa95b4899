// Split-offset scan + row-tile tables (one workgroup, wave-shuffle scan), as a
// device routine shared by the offsets kernel and the fused offsets + activation
// quantize kernel.
//
// Computes the exclusive prefix sum with a leading zero of the split sizes (page
// "Single parameter for GroupedLinear module": the offsets of a grouped tensor are
// a cumsum with a leading zero, done there by a single-block Kogge-Stone kernel).
// Here the same pass also builds, for each row-tile height the GEMMs use, the
// exclusive prefix of per-group tile counts ceil(m_g / rows) -- the table the
// persistent GEMM scheduler maps work items from -- and validates the splits
// (review comment on that page: fuse the tile-offset computation with the cumsum).
#pragma once

#include "gl_common.hpp"

namespace gl {

constexpr int kScanThreads = 1024;  // the standalone offsets kernel's workgroup

template <typename T>
__device__ __forceinline__ T wave_inclusive_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    T o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// The whole scan, run by one workgroup of THREADS threads (groups are taken
// THREADS at a time with a running carry); also zeroes the workspace's
// split-contraction arrival counters and records how many partial-tile slots its
// split area holds.
template <int THREADS>
__device__ __forceinline__ void offsets_block(const int64_t *__restrict__ m_splits, int G, int64_t total_rows,
                                              void *ws, int split_slots) {
  WsView v = ws_view(ws, G);
  int64_t *off = const_cast<int64_t *>(v.off);
  int32_t *pre[kNumTileRows];
  for (int i = 0; i < kNumTileRows; ++i) pre[i] = const_cast<int32_t *>(v.pre[i]);

  constexpr int kScanWaves = THREADS / 64;
  __shared__ int64_t s_off[kScanWaves];
  __shared__ int32_t s_t[kNumTileRows][kScanWaves];
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) s_bad = 0;
  for (int i = tid; i < kSplitSlots; i += THREADS) v.split_cnt[i] = 0;
  __syncthreads();

  int64_t carry = 0;
  int32_t tcarry[kNumTileRows] = {0, 0, 0, 0};
  for (int base = 0; base < G; base += THREADS) {
    const int g = base + tid;
    int64_t m = g < G ? m_splits[g] : 0;
    if (m < 0) {
      atomicOr(&s_bad, 1);
      m = 0;
    }
    int32_t t[kNumTileRows];
#pragma unroll
    for (int i = 0; i < kNumTileRows; ++i) t[i] = (int32_t)((m + kTileRows[i] - 1) / kTileRows[i]);

    int64_t inc = wave_inclusive_scan(m);
    int32_t tinc[kNumTileRows];
#pragma unroll
    for (int i = 0; i < kNumTileRows; ++i) tinc[i] = wave_inclusive_scan(t[i]);
    if (lane == 63) {
      s_off[wave] = inc;
#pragma unroll
      for (int i = 0; i < kNumTileRows; ++i) s_t[i][wave] = tinc[i];
    }
    __syncthreads();
    // every thread adds the totals of the waves before its own (16 values, no second scan)
    int64_t wbase = carry;
    int32_t tbase[kNumTileRows];
#pragma unroll
    for (int i = 0; i < kNumTileRows; ++i) tbase[i] = tcarry[i];
    int64_t chunk = 0;
    int32_t tchunk[kNumTileRows] = {0, 0, 0, 0};
    for (int w = 0; w < kScanWaves; ++w) {
      const int64_t so = s_off[w];
      if (w < wave) wbase += so;
      chunk += so;
#pragma unroll
      for (int i = 0; i < kNumTileRows; ++i) {
        const int32_t st = s_t[i][w];
        if (w < wave) tbase[i] += st;
        tchunk[i] += st;
      }
    }
    if (g < G) {
      off[g] = wbase + inc - m;
#pragma unroll
      for (int i = 0; i < kNumTileRows; ++i) pre[i][g] = tbase[i] + tinc[i] - t[i];
    }
    carry += chunk;
#pragma unroll
    for (int i = 0; i < kNumTileRows; ++i) tcarry[i] += tchunk[i];
    __syncthreads();  // s_off / s_t are rewritten by the next chunk
  }
  if (tid == 0) {
    off[G] = carry;
#pragma unroll
    for (int i = 0; i < kNumTileRows; ++i) pre[i][G] = tcarry[i];
    WsHeader *h = v.hdr;
    h->num_groups = G;
    h->total_rows = total_rows;
    h->magic = kWsMagic;
    h->split_slots = split_slots;
    h->status = (s_bad ? 1 : 0) | (carry != total_rows ? 2 : 0);
  }
}

// The same scan by a single wave with no LDS (groups 64 at a time, the running
// totals broadcast from lane 63): for the fused offsets + quantize launch, whose
// other workgroups then need no LDS either.  Called by the 64 lanes of one wave.
__device__ __forceinline__ void offsets_wave(const int64_t *__restrict__ m_splits, int G, int64_t total_rows,
                                             void *ws) {
  WsView v = ws_view(ws, G);
  int64_t *off = const_cast<int64_t *>(v.off);
  int32_t *pre[kNumTileRows];
  for (int i = 0; i < kNumTileRows; ++i) pre[i] = const_cast<int32_t *>(v.pre[i]);
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < kSplitSlots; i += 64) v.split_cnt[i] = 0;

  int64_t carry = 0;
  int32_t tcarry[kNumTileRows] = {0, 0, 0, 0};
  bool bad = false;
  for (int base = 0; base < G; base += 64) {
    const int g = base + lane;
    int64_t m = g < G ? m_splits[g] : 0;
    if (m < 0) {
      bad = true;
      m = 0;
    }
    int32_t t[kNumTileRows], tinc[kNumTileRows];
#pragma unroll
    for (int i = 0; i < kNumTileRows; ++i) t[i] = (int32_t)((m + kTileRows[i] - 1) / kTileRows[i]);
    const int64_t inc = wave_inclusive_scan(m);
#pragma unroll
    for (int i = 0; i < kNumTileRows; ++i) tinc[i] = wave_inclusive_scan(t[i]);
    if (g < G) {
      off[g] = carry + inc - m;
#pragma unroll
      for (int i = 0; i < kNumTileRows; ++i) pre[i][g] = tcarry[i] + tinc[i] - t[i];
    }
    carry += __shfl(inc, 63, 64);
#pragma unroll
    for (int i = 0; i < kNumTileRows; ++i) tcarry[i] += __shfl(tinc[i], 63, 64);
  }
  const bool any_bad = __ballot(bad) != 0;
  if (lane == 0) {
    off[G] = carry;
#pragma unroll
    for (int i = 0; i < kNumTileRows; ++i) pre[i][G] = tcarry[i];
    WsHeader *h = v.hdr;
    h->num_groups = G;
    h->total_rows = total_rows;
    h->magic = kWsMagic;
    h->split_slots = kSplitSlots;
    h->status = (any_bad ? 1 : 0) | (carry != total_rows ? 2 : 0);
  }
}

}  // namespace gl
