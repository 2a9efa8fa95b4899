// SwiGLU between the two grouped GEMMs of the grouped MLP: a = silu(g) * u with g
// and u the two halves of FC1's output h [T, 2F], and its backward.
//
// The grouped MLP of page "[PyTorch] Add optional caller-provided output/grad-input
// buffers to GroupedLinear and fused grouped MLP" is FC1, an activation and FC2 over
// the same splits; the pages do not name the activation, which is taken to be
// SwiGLU on FC1's two output halves (silu(v) = v / (1 + exp(-v))).
//
// HBM-bound elementwise work: each thread moves 16 bytes of each operand (8 columns
// of a 16-bit type, 4 of fp32), math in fp32, one rounding per output.  Per row the
// forward reads 2F and writes F elements; the backward reads 3F and writes 2F.
#include "gl_common.hpp"

namespace gl {

constexpr int kSwThreads = 256;
enum { SW_BF16 = 0, SW_F32 = 1, SW_F16 = 2 };

template <int EL>
struct Vec;  // 16 bytes of elements <-> fp32 values

template <>
struct Vec<SW_F32> {
  static constexpr int n = 4;
  __device__ static void load(const void *p, float *v) {
    const float4 q = *(const float4 *)p;
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  __device__ static void store(void *p, const float *v) { *(float4 *)p = make_float4(v[0], v[1], v[2], v[3]); }
};

template <int EL>
struct Vec16 {
  static constexpr int n = 8;
  static constexpr bool F16 = EL == SW_F16;
  __device__ static void load(const void *p, float *v) {
    const uint4 q = *(const uint4 *)p;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = h16_to_f32<F16>((uint16_t)(w[i] & 0xffffu));
      v[2 * i + 1] = h16_to_f32<F16>((uint16_t)(w[i] >> 16));
    }
  }
  __device__ static void store(void *p, const float *v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = pack_h16x2<F16>(v[2 * i], v[2 * i + 1]);
    *(uint4 *)p = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <>
struct Vec<SW_BF16> : Vec16<SW_BF16> {};
template <>
struct Vec<SW_F16> : Vec16<SW_F16> {};

constexpr int elem_bytes(int el) { return el == SW_F32 ? 4 : 2; }

__device__ __forceinline__ float sigmoid(float v) { return 1.f / (1.f + __expf(-v)); }

template <int EL>
__global__ __launch_bounds__(kSwThreads) void swiglu_fwd_kernel(const char *__restrict__ h, int64_t F, int64_t n,
                                                                 char *__restrict__ a) {
  using V = Vec<EL>;
  constexpr int B = elem_bytes(EL);
  const int64_t per_row = F / V::n;
  const int64_t t = (int64_t)blockIdx.x * kSwThreads + threadIdx.x;
  if (t >= n) return;
  const int64_t r = t / per_row, c = (t - r * per_row) * V::n;
  float g[V::n], u[V::n], o[V::n];
  V::load(h + (r * 2 * F + c) * B, g);
  V::load(h + (r * 2 * F + F + c) * B, u);
#pragma unroll
  for (int i = 0; i < V::n; ++i) o[i] = g[i] * sigmoid(g[i]) * u[i];
  V::store(a + (r * F + c) * B, o);
}

template <int EL>
__global__ __launch_bounds__(kSwThreads) void swiglu_bwd_kernel(const char *__restrict__ h,
                                                                 const char *__restrict__ da, int64_t F, int64_t n,
                                                                 char *__restrict__ dh) {
  using V = Vec<EL>;
  constexpr int B = elem_bytes(EL);
  const int64_t per_row = F / V::n;
  const int64_t t = (int64_t)blockIdx.x * kSwThreads + threadIdx.x;
  if (t >= n) return;
  const int64_t r = t / per_row, c = (t - r * per_row) * V::n;
  float g[V::n], u[V::n], d[V::n], dg[V::n], du[V::n];
  V::load(h + (r * 2 * F + c) * B, g);
  V::load(h + (r * 2 * F + F + c) * B, u);
  V::load(da + (r * F + c) * B, d);
#pragma unroll
  for (int i = 0; i < V::n; ++i) {
    const float s = sigmoid(g[i]);
    dg[i] = d[i] * u[i] * (s + g[i] * s * (1.f - s));
    du[i] = d[i] * g[i] * s;
  }
  V::store(dh + (r * 2 * F + c) * B, dg);
  V::store(dh + (r * 2 * F + F + c) * B, du);
}

// el: 0 bf16, 1 fp32, 2 fp16.  F a multiple of 8 (16-bit) or 4 (fp32).
hipError_t launch_swiglu_fwd(int el, int64_t T, int64_t F, const void *h, void *a, hipStream_t s) {
  const int64_t n = T * (F / (el == SW_F32 ? 4 : 8));
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + kSwThreads - 1) / kSwThreads)), block(kSwThreads);
  if (el == SW_F32)
    hipLaunchKernelGGL(swiglu_fwd_kernel<SW_F32>, grid, block, 0, s, (const char *)h, F, n, (char *)a);
  else if (el == SW_F16)
    hipLaunchKernelGGL(swiglu_fwd_kernel<SW_F16>, grid, block, 0, s, (const char *)h, F, n, (char *)a);
  else
    hipLaunchKernelGGL(swiglu_fwd_kernel<SW_BF16>, grid, block, 0, s, (const char *)h, F, n, (char *)a);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(int el, int64_t T, int64_t F, const void *h, const void *da, void *dh, hipStream_t s) {
  const int64_t n = T * (F / (el == SW_F32 ? 4 : 8));
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + kSwThreads - 1) / kSwThreads)), block(kSwThreads);
  if (el == SW_F32)
    hipLaunchKernelGGL(swiglu_bwd_kernel<SW_F32>, grid, block, 0, s, (const char *)h, (const char *)da, F, n,
                       (char *)dh);
  else if (el == SW_F16)
    hipLaunchKernelGGL(swiglu_bwd_kernel<SW_F16>, grid, block, 0, s, (const char *)h, (const char *)da, F, n,
                       (char *)dh);
  else
    hipLaunchKernelGGL(swiglu_bwd_kernel<SW_BF16>, grid, block, 0, s, (const char *)h, (const char *)da, F, n,
                       (char *)dh);
  return hipGetLastError();
}

}  // namespace gl
