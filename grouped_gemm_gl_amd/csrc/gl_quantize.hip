// Rowwise MXFP8 quantization: bf16 -> E4M3 codes + one E8M0 scale per 32 elements.
//
// Format from page "transformer_engine/pytorch/ops/basic/grouped_linear.py"
// (_quantize_weights_mxfp8: E4M3 data, one scale per 32 elements of the inner
// dimension); scale rule from OCP MX v1.0: shared exponent floor(log2(amax)) - 8
// clamped to [-127, 127], elements rounded to nearest-even E4M3 and saturated at
// 448.  HBM-bound: each thread owns one 32-element block (64 bytes in, 32 + 1 out),
// so a wave streams 4 KiB of contiguous input.  Everything is exact integer /
// power-of-two arithmetic, bit-identical to the rule.
#include "gl_common.hpp"

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

__global__ __launch_bounds__(kQThreads) void quantize_mxfp8_kernel(const uint16_t *__restrict__ src,
                                                                   int64_t nblocks, uint8_t *__restrict__ data,
                                                                   uint8_t *__restrict__ scale) {
  const int64_t b = (int64_t)blockIdx.x * kQThreads + threadIdx.x;
  if (b >= nblocks) return;
  // blocks are numbered row-major, so block b covers elements [32 b, 32 b + 32)
  const uint4 *in = (const uint4 *)(src + b * 32);
  uint4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = in[i];
  const uint32_t *w = (const uint32_t *)v;
  uint32_t amax = 0;  // |bf16| bit patterns order like magnitudes (Inf 0x7f80, NaN above)
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    amax = max(amax, w[i] & 0x7fffu);
    amax = max(amax, (w[i] >> 16) & 0x7fffu);
  }
  uint32_t out[8];
  uint8_t sbyte;
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
  uint4 *dst = (uint4 *)(data + b * 32);
  dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
  dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
  scale[b] = sbyte;
}

hipError_t launch_quantize_mxfp8(const uint16_t *src, int64_t rows, int64_t cols, uint8_t *data, uint8_t *scale,
                                 hipStream_t s) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return hipSuccess;
  const int64_t grid = (nblocks + kQThreads - 1) / kQThreads;
  hipLaunchKernelGGL(quantize_mxfp8_kernel, dim3((unsigned)grid), dim3(kQThreads), 0, s, src, nblocks, data, scale);
  return hipGetLastError();
}

}  // namespace gl
