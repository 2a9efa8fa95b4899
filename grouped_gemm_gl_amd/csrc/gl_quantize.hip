// MXFP8 quantization: bf16 -> E4M3 codes + one E8M0 scale per 32 elements, rowwise
// (blocks along a row) and columnwise (blocks down a column, per group, stored
// transposed; the quantized backward pass of grouped_linear.py takes columnwise
// usage for the operands whose contraction runs over rows).
//
// Format from page "transformer_engine/pytorch/ops/basic/grouped_linear.py"
// (_quantize_weights_mxfp8: E4M3 data, one scale per 32 elements of the inner
// dimension); scale rule from OCP MX v1.0: shared exponent floor(log2(amax)) - 8
// clamped to [-127, 127], elements rounded to nearest-even E4M3 and saturated at
// 448.  HBM-bound: each thread owns one 32-element block (64 bytes in, 32 + 1 out),
// so a wave streams 4 KiB of contiguous input.  The scale comes from the exponent
// bits and multiplies exactly (a power of two); the rounding to E4M3 is the
// hardware pack conversion, bit-identical to the rule over every value it can see.
#include "gl_offsets.hpp"

namespace gl {

constexpr int kQThreads = 256;

// E4M3 codes of four finite floats (already scaled into the block's range), packed
// one per byte: round to nearest even, magnitudes above 448 saturate to 448, the sign
// bit is kept (also for zero).  gfx950's pack conversion to OCP E4M3 rounds to
// nearest even and keeps the sign; the clamp first makes overflow saturate.  Over
// every value the quantizers can pass (8 significant bits, exponents -149 .. 9, both
// signs) it gives the same bytes as the rule spelled out (checked exhaustively on
// the device).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  const auto sat = [](float v) { return __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f); };
  uint32_t o = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(a), sat(b), 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat(c), sat(d), (int)o, true);
}

// One block of 32 bf16 values, given as 16 words of two packed values each (element
// 2i in the low half of w[i]): 32 E4M3 codes packed four per word, and the scale byte.
__device__ __forceinline__ void quantize_block(const uint32_t *w, uint32_t *out, uint8_t &sbyte) {
  uint32_t amax = 0;  // |bf16| bit patterns order like magnitudes (Inf 0x7f80, NaN above)
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = max(amax, w[i] & 0x7fffu);
    amax = max(amax, (w[i] >> 16) & 0x7fffu);
  }
  if (amax >= 0x7f80u) {  // Inf or NaN in the block
    sbyte = 0xff;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t o = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t h = (w[(i * 4 + k) >> 1] >> (((i * 4 + k) & 1) * 16)) & 0xffffu;
        o |= (0x7fu | ((h >> 8) & 0x80u)) << (8 * k);
      }
      out[i] = o;
    }
  } else {
    const int ef = (int)(amax >> 7);          // biased exponent of amax (0 for zero/subnormal)
    const int byte = ef > 8 ? ef - 8 : 0;     // e + 127 with e = floor(log2 amax) - 8, e >= -127
    sbyte = (uint8_t)byte;
    const float mul = __builtin_ldexpf(1.0f, 127 - byte);  // 2^-e, a normal float
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // elements 4i .. 4i + 3 are the halves of words 2i and 2i + 1
      const uint32_t w0 = w[2 * i], w1 = w[2 * i + 1];
      out[i] = e4m3_pack4(__uint_as_float(w0 << 16) * mul, __uint_as_float(w0 & 0xffff0000u) * mul,
                          __uint_as_float(w1 << 16) * mul, __uint_as_float(w1 & 0xffff0000u) * mul);
    }
  }
}

__device__ __forceinline__ void store_block(uint8_t *dst, const uint32_t *out) {
  uint4 *d = (uint4 *)dst;
  d[0] = make_uint4(out[0], out[1], out[2], out[3]);
  d[1] = make_uint4(out[4], out[5], out[6], out[7]);
}

// Rowwise block b (blocks are numbered row-major, so block b covers elements
// [32 b, 32 b + 32) of the matrix).
__device__ __forceinline__ void quantize_row_block(const uint16_t *__restrict__ src, int64_t b,
                                                   uint8_t *__restrict__ data, uint8_t *__restrict__ scale) {
  const uint4 *in = (const uint4 *)(src + b * 32);
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = in[i];
  uint32_t out[8];
  uint8_t sbyte;
  quantize_block((const uint32_t *)v, out, sbyte);
  store_block(data + b * 32, out);
  scale[b] = sbyte;
}

__global__ __launch_bounds__(kQThreads) void quantize_mxfp8_kernel(const uint16_t *__restrict__ src,
                                                                   int64_t nblocks, uint8_t *__restrict__ data,
                                                                   uint8_t *__restrict__ scale) {
  const int64_t b = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  if (b < nblocks) quantize_row_block(src, b, data, scale);
}

// Fused split-offset scan and rowwise activation quantization, one launch of
// kQThreads-thread workgroups: the first wave of workgroup 0 runs the scan (the
// quantization does not depend on the splits), every thread of the other
// workgroups quantizes one block.  The kernel uses no LDS (an LDS allocation per
// workgroup slows the dispatch of these short workgroups).
__global__ __launch_bounds__(kQThreads) void offsets_quantize_mxfp8_kernel(
    const int64_t *__restrict__ m_splits, int G, int64_t total_rows, void *ws, const uint16_t *__restrict__ src,
    int64_t nblocks, uint8_t *__restrict__ data, uint8_t *__restrict__ scale) {
  if (blockIdx.x == 0) {
    if (threadIdx.x < 64) offsets_wave(m_splits, G, total_rows, ws);
    return;
  }
  const int64_t b = (int64_t)(blockIdx.x - 1) * kQThreads + threadIdx.x;
  if (b < nblocks) quantize_row_block(src, b, data, scale);
}

// Columnwise MXFP8 (blocks of 32 consecutive rows of a column), stored transposed:
// thread t handles the 4 adjacent columns 4 (t % (cols / 4)) .. + 3 of padded block
// b = t / (cols / 4), reading 8 bytes per row, so a wave's row read covers 512
// contiguous bytes.
//   Group mode (ws != null): rows split by the workspace's offsets; group g's rows
//   are padded to whole 128-row tiles and its blocks are numbered from 4 pre128[g],
//   so padded block b lands at output column 32 b of row c of a [cols, ld] matrix.
//   Rows past a group's end read as zero (padding blocks come out all zero).
//   Uniform mode (ws == null): groups of urows rows (a multiple of 32) each, group g
//   stored as its own [cols, urows] matrix at data + g * cols * urows.
__device__ __forceinline__ void quantize_colwise_thread(int64_t t, const uint16_t *__restrict__ src, int64_t cols,
                                                        int64_t nblk, const void *ws, int G, int64_t total_rows,
                                                        int64_t urows, uint8_t *__restrict__ data,
                                                        uint8_t *__restrict__ scale, int64_t ld) {
  const int64_t quads = cols / 4;
  const int64_t c4 = (t % quads) * 4, b = t / quads;
  if (b >= nblk) return;
  int64_t r0, rend, out_base, out_ld, s_base, s_ld;
  if (ws) {
    const WsView v = ws_view(ws, G);
    if (!ws_usable(v.hdr, G, total_rows)) return;
    const int32_t *__restrict__ pre = v.pre[tile_rows_index(128)];
    if (b >= 4 * (int64_t)pre[G]) return;  // past the last group's padding: untouched
    int lo = 0, hi = G;  // last g with 4 pre[g] <= b
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (4 * (int64_t)pre[mid] <= b) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    r0 = v.off[g] + (b - 4 * (int64_t)pre[g]) * 32;
    rend = v.off[g + 1];
    out_base = b * 32;
    out_ld = ld;
    s_base = b;
    s_ld = ld / 32;
  } else {
    const int64_t per = urows / 32, g = b / per, lb = b - g * per;
    r0 = g * urows + lb * 32;
    rend = r0 + 32;
    out_base = g * cols * urows + lb * 32;
    out_ld = urows;
    s_base = g * cols * per + lb;
    s_ld = per;
  }
  uint32_t w[4][16];  // per column, 32 rows as 16 words of two packed bf16
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t r = r0 + 2 * i;
    const uint2 lo = r < rend ? *(const uint2 *)(src + r * cols + c4) : make_uint2(0, 0);
    const uint2 hi = r + 1 < rend ? *(const uint2 *)(src + (r + 1) * cols + c4) : make_uint2(0, 0);
    w[0][i] = (lo.x & 0xffffu) | (hi.x << 16);
    w[1][i] = (lo.x >> 16) | (hi.x & 0xffff0000u);
    w[2][i] = (lo.y & 0xffffu) | (hi.y << 16);
    w[3][i] = (lo.y >> 16) | (hi.y & 0xffff0000u);
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t out[8];
    uint8_t sbyte;
    quantize_block(w[k], out, sbyte);
    store_block(data + out_base + (c4 + k) * out_ld, out);
    scale[s_base + (c4 + k) * s_ld] = sbyte;
  }
}

__global__ __launch_bounds__(kQThreads) void quantize_mxfp8_colwise_kernel(
    const uint16_t *__restrict__ src, int64_t cols, int64_t nblk, const void *ws, int G, int64_t total_rows,
    int64_t urows, uint8_t *__restrict__ data, uint8_t *__restrict__ scale, int64_t ld) {
  quantize_colwise_thread((int64_t)blockIdx.x * kQThreads + threadIdx.x, src, cols, nblk, ws, G, total_rows, urows,
                          data, scale, ld);
}

// Group-mode columnwise MXFP8 by tiles of 128 rows x 64 columns, one workgroup
// each: the tile is read with 16-byte row loads into LDS, each thread quantizes one
// column's 32-row block from there, and the codes go back through LDS so that every
// store instruction writes whole 128-byte lines of the transposed output (8 rows of
// 128 codes per wave) and each output row gets its 4 scale bytes as one word.  A
// 128-row tile is one of a group's padded 128-row tiles (the workspace's 128-row
// prefix table), so it lies in one group; rows past the group's end read as zero.
// Needs cols % 8 == 0 and a 4-byte aligned scale matrix; the per-thread kernel
// above serves the other cases.  Tiles past the last group's padding are left
// untouched.  With row_data set (cols % 32 == 0) the same tile also gives the
// rowwise codes of its valid rows (blocks of 32 along a row, layout [T, cols]),
// so a tensor needed both ways is read once.  FROM_SPLITS (fewer than 64 groups):
// every workgroup derives the offsets and tile prefix from m_splits itself (one
// wave scan), so the launch needs no workspace written before it; its first wave
// of workgroup 0 also writes the workspace, as the offsets kernel does, for the
// kernels after it.  Invalid splits (a negative size, or a sum other than
// total_rows): the workspace gets its status word and no code is written.
// 128-column tiles (256-byte row reads, two columns per thread) measured slower:
// the larger LDS and register footprint costs more occupancy than they save.
constexpr int kCtRows = 128, kCtCols = 64;

// One 128-row x 64-column tile of the columnwise (and optionally rowwise) MXFP8
// quantization: rows [r0, rend) of src [*, cols] (rows past rend read as zero),
// columns c0 .. c0 + 63.  Output row c (input column c0 + c) gets its 128 codes at
// dt + c * dt_ld and its 4 scale bytes as one word at st + c * st_ld; with row_data
// set, the tile's valid rows also get their rowwise codes (layout [*, cols]).  The
// tile goes in through LDS with 16-byte row loads, one wave quantizes each 32-row
// block of every column, and the codes go back through LDS so that each store
// instruction writes whole 128-byte lines (8 output rows per wave).  Whole
// workgroup; lds holds kCtLdsBytes.
constexpr int kCtLdsBytes = kCtRows * kCtCols * 2 + kCtCols * kCtRows + kCtCols * 4;

__device__ __forceinline__ void ct_tile(const uint16_t *__restrict__ src, int64_t cols, int64_t r0, int64_t rend,
                                        int64_t c0, uint8_t *__restrict__ dt, int64_t dt_ld,
                                        uint8_t *__restrict__ st, int64_t st_ld, uint8_t *__restrict__ row_data,
                                        uint8_t *__restrict__ row_scale, char *lds) {
  char *in = lds, *outc = lds + kCtRows * kCtCols * 2, *sc = outc + kCtCols * kCtRows;
  const int tid = threadIdx.x;
  constexpr int kRowBytes = kCtCols * 2, kLanesPerRow = kRowBytes / 16, kRowsPerPass = kQThreads / kLanesPerRow;

  // load: 16 bytes (8 columns) per thread, kRowsPerPass rows per pass
  {
    const int cc = (tid % kLanesPerRow) * 8;
#pragma unroll
    for (int i = 0; i < kCtRows / kRowsPerPass; ++i) {
      const int r = tid / kLanesPerRow + kRowsPerPass * i;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (r0 + r < rend && c0 + cc < cols) val = *(const uint4 *)(src + (r0 + r) * cols + c0 + cc);
      *(uint4 *)(in + r * kRowBytes + cc * 2) = val;
    }
  }
  __syncthreads();
  // quantize: thread (column c = t % 64, block k = t / 64) -- one wave per block
  {
    const int c = tid & 63, k = tid >> 6;
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 32 * k + 2 * i;
      const uint32_t lo = *(const uint16_t *)(in + r * kRowBytes + c * 2);
      const uint32_t hi = *(const uint16_t *)(in + (r + 1) * kRowBytes + c * 2);
      w[i] = lo | (hi << 16);
    }
    uint32_t out[8];
    uint8_t sbyte;
    quantize_block(w, out, sbyte);
    char *row = outc + c * kCtRows;
    *(uint4 *)(row + (((2 * k) ^ (c & 7)) << 4)) = make_uint4(out[0], out[1], out[2], out[3]);
    *(uint4 *)(row + (((2 * k + 1) ^ (c & 7)) << 4)) = make_uint4(out[4], out[5], out[6], out[7]);
    sc[c * 4 + k] = sbyte;
  }
  // rowwise: thread (row t / 2, block t % 2) of the tile's valid rows
  if (row_data) {
    const int r = tid >> 1, hb = tid & 1;
    if (r0 + r < rend && c0 + hb * 32 < cols) {
      const uint4 *q = (const uint4 *)(in + r * kRowBytes + hb * 64);
      uint4 vv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) vv[i] = q[i];
      uint32_t out[8];
      uint8_t sbyte;
      quantize_block((const uint32_t *)vv, out, sbyte);
      store_block(row_data + (r0 + r) * cols + c0 + hb * 32, out);
      row_scale[(r0 + r) * (cols / 32) + c0 / 32 + hb] = sbyte;
    }
  }
  __syncthreads();
  // store: thread t writes 16 codes of output row t / 8 (+ 32 i), whole lines per wave
#pragma unroll
  for (int i = 0; i < kCtCols / 32; ++i) {
    const int c = (tid >> 3) + 32 * i, j = tid & 7;
    if (c0 + c < cols) {
      const uint4 val = *(const uint4 *)(outc + c * kCtRows + ((j ^ (c & 7)) << 4));
      *(uint4 *)(dt + c * dt_ld + j * 16) = val;
    }
  }
  for (int c = tid; c < kCtCols; c += kQThreads)
    if (c0 + c < cols)
      *(uint32_t *)(st + c * st_ld) = *(const uint32_t *)(sc + c * 4);
  __syncthreads();  // the LDS is free for the next tile
}

template <bool FROM_SPLITS>
__global__ __launch_bounds__(kQThreads) void quantize_mxfp8_colwise_tile_kernel(
    const uint16_t *__restrict__ src, int64_t cols, const void *ws, int G, int64_t total_rows,
    uint8_t *__restrict__ data, uint8_t *__restrict__ scale, int64_t ld, uint8_t *__restrict__ row_data,
    uint8_t *__restrict__ row_scale, const int64_t *__restrict__ m_splits) {
  // [128 rows][kCtCols bf16] input, then [kCtCols rows][128 codes] output (16-byte
  // slots XOR-swizzled by row), then [kCtCols][4] scale bytes: one array (see the GEMMs)
  __shared__ __attribute__((aligned(16))) char lds[kCtLdsBytes];
  const int ncol_tiles = (int)((cols + kCtCols - 1) / kCtCols);
  const int64_t b128 = blockIdx.x / ncol_tiles;
  const int64_t c0 = (int64_t)(blockIdx.x % ncol_tiles) * kCtCols;
  const WsView v = ws_view(ws, G);
  const int32_t *__restrict__ pre = v.pre[tile_rows_index(kCtRows)];
  const int tid = threadIdx.x;
  // The tile's group and rows.  Up to 63 groups the header, pre[] and off[] are read
  // in one round (lane i holds entry i; a ballot finds the group and shuffles hand
  // out its entries), so a workgroup waits for one load latency before its input
  // loads instead of three.
  int64_t r0, rend;
  if constexpr (FROM_SPLITS) {
    const int lane = tid & 63;
    if (blockIdx.x == 0 && tid < 64) offsets_wave(m_splits, G, total_rows, (void *)ws);
    const int64_t m = lane < G ? m_splits[lane] : 0;
    const bool bad = __ballot(m < 0) != 0;
    const int64_t mv = m > 0 ? m : 0;
    const int64_t incl = wave_inclusive_scan(mv);
    const int32_t t128 = (int32_t)((mv + kCtRows - 1) / kCtRows);
    const int32_t tincl = wave_inclusive_scan(t128);
    if (bad || __shfl(incl, 63, 64) != total_rows) return;  // the status word says why
    // lane l <= G: exclusive prefixes (lane G: the totals)
    const int32_t pv = lane <= G ? tincl - t128 : 0x7fffffff;
    if (b128 >= __shfl(pv, G, 64)) return;  // past the last group's padding: untouched
    const int g = __popcll(__ballot(pv <= (int)b128)) - 1;
    r0 = __shfl(incl - mv, g, 64) + (b128 - __shfl(pv, g, 64)) * kCtRows;
    rend = __shfl(incl, g, 64);
  } else if (G < 64) {
    const int lane = tid & 63;
    const WsHeader *h = v.hdr;
    const int32_t st = h->status, mg = h->magic, ng = h->num_groups;
    const int64_t tr = h->total_rows;
    const int32_t pv = lane <= G ? pre[lane] : 0x7fffffff;
    const int64_t ov = lane <= G ? v.off[lane] : 0;
    if (mg != kWsMagic || ng != G || tr != total_rows) {
      if (tid == 0) atomicOr((int *)&h->status, 4);
      return;
    }
    if (st != 0) return;
    if (b128 >= __shfl(pv, G, 64)) return;  // past the last group's padding: untouched
    const int g = __popcll(__ballot(pv <= (int)b128)) - 1;
    r0 = __shfl(ov, g, 64) + (b128 - __shfl(pv, g, 64)) * kCtRows;
    rend = __shfl(ov, g + 1, 64);
  } else {
    if (!ws_usable(v.hdr, G, total_rows)) return;
    if (b128 >= pre[G]) return;
    const int g = find_group(pre, G, (int)b128);
    r0 = v.off[g] + (b128 - pre[g]) * kCtRows;
    rend = v.off[g + 1];
  }
  // (device-check build) the tile's rows lie inside the input, its codes inside the output
  if (!device_check(r0 >= 0 && r0 < rend && rend <= total_rows && (b128 + 1) * kCtRows <= ld, ws)) return;
  ct_tile(src, cols, r0, rend, c0, data + c0 * ld + b128 * kCtRows, ld, scale + c0 * (ld / 32) + b128 * (kCtRows / 32),
          ld / 32, row_data, row_scale, lds);
}

// The weights' MXFP8 workspace by tiles (N % 128 == 0, columnwise codes wanted,
// 4-byte aligned columnwise scales): group g of w [G, N, K] is a uniform matrix of
// N rows, so 128-row tile bl of group g gives rowwise codes of rows g N + 128 bl ..
// and columnwise codes [K, N] of group g at columns 128 bl ..  Persistent over a
// bounded grid, so that a refresh skipped by its no-op flag stays one small launch.
__global__ __launch_bounds__(kQThreads) void quantize_mxfp8_weights_tile_kernel(
    const uint16_t *__restrict__ w, int G, int64_t N, int64_t K, uint8_t *__restrict__ data,
    uint8_t *__restrict__ scale, uint8_t *__restrict__ data_t, uint8_t *__restrict__ scale_t,
    const int32_t *__restrict__ noop) {
  __shared__ __attribute__((aligned(16))) char lds[kCtLdsBytes];
  if (noop && *noop) return;
  const int64_t tpg = N / kCtRows, nct = (K + kCtCols - 1) / kCtCols;
  const int64_t tiles = (int64_t)G * tpg * nct;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t ct = t % nct, rt = t / nct, g = rt / tpg, bl = rt % tpg;
    const int64_t c0 = ct * kCtCols, r0 = g * N + bl * kCtRows;
    ct_tile(w, K, r0, r0 + kCtRows, c0, data_t + g * K * N + c0 * N + bl * kCtRows, N,
            scale_t + g * K * (N / 32) + c0 * (N / 32) + bl * (kCtRows / 32), N / 32, data, scale, lds);
  }
}

// The weights' MXFP8 workspace in one launch: rowwise codes of w [G*N, K] (forward
// operand, row_threads threads of one block each) and, when data_t is set, the
// columnwise codes [G, K, N] (dgrad operand, col_threads threads), walked
// grid-stride over one index space.  A nonzero *noop (device flag, may be null)
// makes every workgroup return at once, leaving the workspace as it was; the grid
// is bounded so that a skipped refresh costs one small launch.
__global__ __launch_bounds__(kQThreads) void quantize_mxfp8_weights_kernel(
    const uint16_t *__restrict__ w, int G, int64_t N, int64_t K, int64_t row_threads, int64_t col_threads,
    uint8_t *__restrict__ data, uint8_t *__restrict__ scale, uint8_t *__restrict__ data_t,
    uint8_t *__restrict__ scale_t, const int32_t *__restrict__ noop) {
  if (noop && *noop) return;
  const int64_t stride = (int64_t)gridDim.x * kQThreads;
  for (int64_t i = (int64_t)blockIdx.x * kQThreads + threadIdx.x; i < row_threads + col_threads; i += stride) {
    if (i < row_threads)
      quantize_row_block(w, i, data, scale);
    else
      quantize_colwise_thread(i - row_threads, w, K, (int64_t)G * (N / 32), nullptr, G, 0, N, data_t, scale_t, N);
  }
}

hipError_t launch_quantize_mxfp8(const uint16_t *src, int64_t rows, int64_t cols, uint8_t *data, uint8_t *scale,
                                 hipStream_t s) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return hipSuccess;
  const int64_t grid = (nblocks + kQThreads - 1) / kQThreads;
  hipLaunchKernelGGL(quantize_mxfp8_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, s, src, nblocks, data, scale);
  return hipGetLastError();
}

// Workgroups of the grid-stride weight refresh: enough to fill the chip several
// times, few enough that a launch skipped by its no-op flag is cheap.
constexpr int64_t kQuantizeWgs = 8192;

hipError_t launch_offsets_quantize_mxfp8(const int64_t *m_splits, int G, int64_t total_rows, void *ws,
                                         const uint16_t *src, int64_t cols, uint8_t *data, uint8_t *scale,
                                         hipStream_t s) {
  const int64_t nblocks = total_rows * (cols / 32);
  const int64_t grid = 1 + (nblocks + kQThreads - 1) / kQThreads;
  hipLaunchKernelGGL(offsets_quantize_mxfp8_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, s, m_splits, G,
                     total_rows, ws, src, nblocks, data, scale);
  return hipGetLastError();
}

hipError_t launch_quantize_mxfp8_weights(const uint16_t *w, int G, int64_t N, int64_t K, uint8_t *data,
                                         uint8_t *scale, uint8_t *data_t, uint8_t *scale_t, const int32_t *noop,
                                         hipStream_t s) {
  if (data_t && N % kCtRows == 0 && ((uintptr_t)scale_t & 3u) == 0) {
    const int64_t tiles = (int64_t)G * (N / kCtRows) * ((K + kCtCols - 1) / kCtCols);
    const int64_t grid = tiles < kQuantizeWgs ? tiles : kQuantizeWgs;
    hipLaunchKernelGGL(quantize_mxfp8_weights_tile_kernel, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(kQThreads), 0,
                       s, w, G, N, K, data, scale, data_t, scale_t, noop);
    return hipGetLastError();
  }
  const int64_t row_threads = (int64_t)G * N * (K / 32);
  const int64_t col_threads = data_t ? (int64_t)G * (N / 32) * (K / 4) : 0;
  const int64_t wgs = (row_threads + col_threads + kQThreads - 1) / kQThreads;
  const int64_t grid = wgs < kQuantizeWgs ? wgs : kQuantizeWgs;
  hipLaunchKernelGGL(quantize_mxfp8_weights_kernel, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(kQThreads), 0, s,
                     w, G, N, K, row_threads, col_threads, data, scale, data_t, scale_t, noop);
  return hipGetLastError();
}

// Group mode: ld columns of output per input column (a multiple of 128, at least
// total_rows + 127 G, so every group's padded rows fit).
hipError_t launch_quantize_mxfp8_colwise(const uint16_t *src, int64_t cols, int G, int64_t total_rows,
                                         const void *ws, uint8_t *data, uint8_t *scale, int64_t ld, hipStream_t s) {
  const int64_t nblk = ld / 32;
  const int64_t threads = nblk * (cols / 4);
  if (threads == 0) return hipSuccess;
  if (cols % 8 == 0 && ((uintptr_t)scale & 3u) == 0) {
    const int64_t tiles = (ld / kCtRows) * ((cols + kCtCols - 1) / kCtCols);
    hipLaunchKernelGGL(quantize_mxfp8_colwise_tile_kernel<false>, dim3((unsigned)tiles), dim3(kQThreads), 0, s, src,
                       cols, ws, G, total_rows, data, scale, ld, (uint8_t *)nullptr, (uint8_t *)nullptr,
                       (const int64_t *)nullptr);
  } else {
    hipLaunchKernelGGL(quantize_mxfp8_colwise_kernel, dim3((unsigned)((threads + kQThreads - 1) / kQThreads)),
                       dim3(kQThreads), 0, s, src, cols, nblk, ws, G, total_rows, (int64_t)0, data, scale, ld);
  }
  return hipGetLastError();
}

// Rowwise codes [T, cols] / scales [T, cols / 32] and group-mode columnwise codes
// of the same bf16 tensor (cols % 32 == 0), reading it once when the tile kernel
// applies, else as the two separate launches.
hipError_t launch_quantize_mxfp8_rowwise_colwise(const uint16_t *src, int64_t cols, int G, int64_t total_rows,
                                                 const void *ws, uint8_t *row_data, uint8_t *row_scale,
                                                 uint8_t *data, uint8_t *scale, int64_t ld, hipStream_t s) {
  if (((uintptr_t)scale & 3u) == 0) {
    const int64_t tiles = (ld / kCtRows) * ((cols + kCtCols - 1) / kCtCols);
    if (tiles == 0) return hipSuccess;
    hipLaunchKernelGGL(quantize_mxfp8_colwise_tile_kernel<false>, dim3((unsigned)tiles), dim3(kQThreads), 0, s, src,
                       cols, ws, G, total_rows, data, scale, ld, row_data, row_scale, (const int64_t *)nullptr);
    return hipGetLastError();
  }
  hipError_t e = launch_quantize_mxfp8(src, total_rows, cols, row_data, row_scale, s);
  if (e != hipSuccess) return e;
  return launch_quantize_mxfp8_colwise(src, cols, G, total_rows, ws, data, scale, ld, s);
}

// The split-offset scan and both usages of the activations in one launch when the
// tile kernel can take the splits itself (fewer than 64 groups, a 4-byte aligned
// columnwise scale matrix), else the fused scan + rowwise launch and the columnwise
// launch after it.
hipError_t launch_offsets_quantize_mxfp8_rowwise_colwise(const int64_t *m_splits, int G, int64_t total_rows,
                                                         void *ws, const uint16_t *src, int64_t cols,
                                                         uint8_t *row_data, uint8_t *row_scale, uint8_t *data,
                                                         uint8_t *scale, int64_t ld, hipStream_t s) {
  if (G < 64 && ((uintptr_t)scale & 3u) == 0) {
    const int64_t tiles = (ld / kCtRows) * ((cols + kCtCols - 1) / kCtCols);
    hipLaunchKernelGGL(quantize_mxfp8_colwise_tile_kernel<true>, dim3((unsigned)(tiles > 0 ? tiles : 1)),
                       dim3(kQThreads), 0, s, src, cols, (const void *)ws, G, total_rows, data, scale, ld, row_data,
                       row_scale, m_splits);
    return hipGetLastError();
  }
  hipError_t e = launch_offsets_quantize_mxfp8(m_splits, G, total_rows, ws, src, cols, row_data, row_scale, s);
  if (e != hipSuccess) return e;
  return launch_quantize_mxfp8_colwise(src, cols, G, total_rows, ws, data, scale, ld, s);
}

// Uniform mode for stacked weights [G, N, K] (N % 32 == 0): codes [G, K, N], scales
// [G, K, N / 32].
hipError_t launch_quantize_mxfp8_colwise_weights(const uint16_t *w, int G, int64_t N, int64_t K, uint8_t *data,
                                                 uint8_t *scale, hipStream_t s) {
  const int64_t nblk = (int64_t)G * (N / 32);
  const int64_t threads = nblk * (K / 4);
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(quantize_mxfp8_colwise_kernel, dim3((unsigned)((threads + kQThreads - 1) / kQThreads)),
                     dim3(kQThreads), 0, s, w, K, nblk, (const void *)nullptr, G, (int64_t)0, N, data, scale, N);
  return hipGetLastError();
}

}  // namespace gl
