// Bias gradient: per-group column sums of dy (page
// "transformer_engine/pytorch/ops/basic/grouped_linear.py", fuser_backward: the bias
// grad of each split is dy_split.sum(dim=0)).
//
// HBM-bound: dy is read exactly once.  A work item is (group g, a slab of 512
// columns), taken grid-stride by a one-dimensional grid; each of the workgroup's 8
// waves reads 16 bytes per lane of every 8th row of the group, keeping eight rows in
// flight, and the 8 wave partials are combined through
// LDS in a fixed order -- deterministic, no atomics.  An empty group writes zeros.
#include "gl_common.hpp"

namespace gl {

constexpr int kBgThreads = 512, kBgWaves = kBgThreads / 64, kBgCols = 512, kBgUnroll = 8;

// element type of dy and db: 0 bf16, 1 fp32, 2 fp16
enum { BG_BF16 = 0, BG_F32 = 1, BG_F16 = 2 };

template <int EL>
__device__ __forceinline__ void add16(float *a, const uint4 &v) {
  if constexpr (EL == BG_F32) {
    a[0] += __uint_as_float(v.x);
    a[1] += __uint_as_float(v.y);
    a[2] += __uint_as_float(v.z);
    a[3] += __uint_as_float(v.w);
  } else {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[2 * e] += h16_to_f32<EL == BG_F16>(d[e] & 0xffff);
      a[2 * e + 1] += h16_to_f32<EL == BG_F16>(d[e] >> 16);
    }
  }
}

template <int EL>
__global__ __launch_bounds__(kBgThreads) void bgrad_kernel(const void *__restrict__ dy_, void *db_,
                                                           void *const *db_ptrs, int G, int64_t N, int64_t T,
                                                           int slabs, const void *ws_) {
  __shared__ float part[kBgWaves][kBgCols];
  const WsView ws = ws_view(ws_, G);
  if (!ws_usable(ws.hdr, G, T)) return;
  constexpr bool F32 = EL == BG_F32;
  constexpr int kEl = F32 ? 4 : 8;  // elements per 16-byte lane load
  constexpr int kEsz = F32 ? 4 : 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const char *dy = (const char *)dy_;

  // work item = (group g, column slab): items are taken grid-stride, so any number
  // of groups fits a bounded one-dimensional grid
  const int64_t items = (int64_t)G * slabs;
  for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
    const int g = (int)(item / slabs);
    const int64_t c0 = (item - (int64_t)g * slabs) * kBgCols;
    const int64_t lo = ws.off[g], hi = ws.off[g + 1];
    // a wave covers 64 * kEl columns of a row; fp32 takes two sweeps of the slab
    for (int sweep = 0; sweep < kBgCols / (64 * kEl); ++sweep) {
      const int lc = sweep * 64 * kEl + lane * kEl;
      const int64_t col = c0 + lc;
      float a[kEl];
#pragma unroll
      for (int e = 0; e < kEl; ++e) a[e] = 0.f;
      if (col < N) {  // N is a multiple of kEl, so a lane's 16 bytes are all in range
        int64_t r = lo + wave;
        for (; r + (kBgUnroll - 1) * kBgWaves < hi; r += kBgUnroll * kBgWaves) {
          uint4 v[kBgUnroll];
#pragma unroll
          for (int u = 0; u < kBgUnroll; ++u) v[u] = *(const uint4 *)(dy + ((r + u * kBgWaves) * N + col) * kEsz);
#pragma unroll
          for (int u = 0; u < kBgUnroll; ++u) add16<EL>(a, v[u]);
        }
        for (; r < hi; r += kBgWaves) add16<EL>(a, *(const uint4 *)(dy + (r * N + col) * kEsz));
      }
#pragma unroll
      for (int e = 0; e < kEl; ++e) part[wave][lc + e] = a[e];
    }
    __syncthreads();
    for (int c = threadIdx.x; c < kBgCols; c += kBgThreads) {
      const int64_t col = c0 + c;
      if (col >= N) continue;
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kBgWaves; ++w) s += part[w][c];
      char *dst = db_ ? (char *)db_ + ((int64_t)g * N + col) * kEsz : (char *)db_ptrs[g] + col * kEsz;
      if constexpr (F32) *(float *)dst = s;
      else *(uint16_t *)dst = f32_to_h16<EL == BG_F16>(s);
    }
    __syncthreads();  // part[] is rewritten by the next item
  }
}

// el: 0 bf16, 1 fp32, 2 fp16
hipError_t launch_bgrad(int G, int64_t N, int64_t T, int el, const void *dy, void *db, void *const *db_ptrs,
                        const void *ws, hipStream_t s) {
  const int slabs = (int)((N + kBgCols - 1) / kBgCols);
  const int64_t items = (int64_t)G * slabs;
  // enough workgroups to keep every CU streaming; larger launches loop
  const dim3 grid((unsigned)(items < 65536 ? items : 65536));
  if (el == BG_F32)
    hipLaunchKernelGGL(bgrad_kernel<BG_F32>, grid, dim3(kBgThreads), 0, s, dy, db, db_ptrs, G, N, T, slabs, ws);
  else if (el == BG_F16)
    hipLaunchKernelGGL(bgrad_kernel<BG_F16>, grid, dim3(kBgThreads), 0, s, dy, db, db_ptrs, G, N, T, slabs, ws);
  else
    hipLaunchKernelGGL(bgrad_kernel<BG_BF16>, grid, dim3(kBgThreads), 0, s, dy, db, db_ptrs, G, N, T, slabs, ws);
  return hipGetLastError();
}

}  // namespace gl
