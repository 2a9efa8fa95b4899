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
// so a wave streams 4 KiB of contiguous input.  Everything is exact integer /
// power-of-two arithmetic, bit-identical to the rule.
#include "gl_offsets.hpp"

namespace gl {

constexpr int kQThreads = 256;

// E4M3 code of a finite float s (already scaled into the block's range), RNE,
// magnitudes >= 448 saturate to 448; the sign bit is kept (also for zero).
__device__ __forceinline__ uint32_t e4m3_code(float s) {
  const uint32_t sign = (__float_as_uint(s) >> 24) & 0x80u;
  const float a = fabsf(s);
  uint32_t mag;
  if (a >= 448.0f) {
    mag = 0x7e;
  } else if (a < 0.015625f) {                    // below 2^-6: subnormal spacing 2^-9
    mag = (uint32_t)__builtin_rintf(a * 512.0f);  // 0..8; 8 is the smallest normal's code
  } else {
    const int E = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;  // -6 .. 8
    const float m = __builtin_rintf(__builtin_ldexpf(a, 3 - E));   // 8 .. 16 (16 carries)
    mag = (uint32_t)((E + 6) * 8) + (uint32_t)m;
  }
  return sign | mag;
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
      uint32_t o = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int el = i * 4 + k;
        const uint32_t h = (w[el >> 1] >> ((el & 1) * 16)) & 0xffffu;
        o |= e4m3_code(__uint_as_float(h << 16) * mul) << (8 * k);
      }
      out[i] = o;
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
  hipLaunchKernelGGL(quantize_mxfp8_colwise_kernel, dim3((unsigned)((threads + kQThreads - 1) / kQThreads)),
                     dim3(kQThreads), 0, s, src, cols, nblk, ws, G, total_rows, (int64_t)0, data, scale, ld);
  return hipGetLastError();
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
