// Grouped GEMM for fp32 storage (forward, dgrad, wgrad) on the vector ALUs.
//
// Same contraction and work decomposition as the bf16 MFMA kernel -- C[i][j] =
// sum_p A[i][p] * B[j][p] per group, with either the token rows (row mode) or the
// contraction (contraction mode) grouped -- but operands are addressed through
// general strides and every product is an fp32 FMA.  64x64 tiles, 256 threads each
// computing a 4x4 block, 16-deep contraction slices staged in LDS.  This serves the
// fp32 layer (the reference accepts fp32 parameters); bf16 is the MFMA path.
#include "gl_common.hpp"

namespace gl {

constexpr int kF32Tile = 64, kF32K = 16, kF32Threads = 256;

struct GemmF32Params {
  const float *A;
  int64_t a_si, a_sp;                // A(i, p) = A_base[i * a_si + p * a_sp]
  const float *B;
  const float *const *B_ptrs;
  int64_t b_gstride, b_sj, b_sp;     // B(j, p) = B_g[j * b_sj + p * b_sp]
  float *C;
  float *const *C_ptrs;
  int64_t c_gstride, ldc;
  const float *bias;
  const float *const *bias_ptrs;
  const void *ws;
  int G;
  int64_t T, rows_i, cols_j, P;
  int tiles_i, tiles_j, accumulate, contr;
};

__global__ __launch_bounds__(kF32Threads) void gemm_f32_kernel(GemmF32Params p) {
  __shared__ float sa[kF32K][kF32Tile + 4];
  __shared__ float sb[kF32K][kF32Tile + 4];
  const WsView ws = ws_view(p.ws, p.G);
  if (!ws_usable(ws.hdr, p.G, p.T)) return;
  const int64_t *off = ws.off;
  const int32_t *pre = ws.pre[tile_rows_index(kF32Tile)];
  const int total = p.contr ? p.G * p.tiles_i * p.tiles_j : pre[p.G] * p.tiles_j;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;

  for (int w = blockIdx.x; w < total; w += gridDim.x) {
    int g, it, jt;
    if (p.contr) {
      const int per = p.tiles_i * p.tiles_j;
      g = w / per;
      it = (w - g * per) % p.tiles_i;
      jt = (w - g * per) / p.tiles_i;
    } else {
      const int q = w / p.tiles_j;
      g = find_group(pre, p.G, q);
      const int mt = pre[g + 1] - pre[g];
      const int local = w - pre[g] * p.tiles_j;
      it = local % mt;
      jt = local / mt;
    }
    const int64_t g_off = off[g], g_rows = off[g + 1] - g_off;
    if (p.contr && p.accumulate && g_rows == 0) continue;
    const float *ab, *bb;
    int64_t i_ext, pmax;
    if (p.contr) {
      ab = p.A + g_off * p.a_sp;
      bb = p.B + g_off * p.b_sp;
      i_ext = p.rows_i;
      pmax = g_rows;
    } else {
      ab = p.A + g_off * p.a_si;
      bb = p.B ? p.B + (int64_t)g * p.b_gstride : p.B_ptrs[g];
      i_ext = g_rows;
      pmax = p.P;
    }
    const int64_t i0 = (int64_t)it * kF32Tile, j0 = (int64_t)jt * kF32Tile;
    float acc[4][4] = {};
    for (int64_t k0 = 0; k0 < pmax; k0 += kF32K) {
      for (int e = tid; e < kF32K * kF32Tile; e += kF32Threads) {
        const int kk = e / kF32Tile, rr = e % kF32Tile;
        const int64_t pk = k0 + kk, ia = i0 + rr, jb = j0 + rr;
        sa[kk][rr] = (pk < pmax && ia < i_ext) ? ab[ia * p.a_si + pk * p.a_sp] : 0.f;
        sb[kk][rr] = (pk < pmax && jb < p.cols_j) ? bb[jb * p.b_sj + pk * p.b_sp] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kF32K; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          a[u] = sa[kk][ty * 4 + u];
          b[u] = sb[kk][tx * 4 + u];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] = fmaf(a[u], b[v], acc[u][v]);
      }
      __syncthreads();
    }
    float *cg;
    int64_t row0;
    if (p.contr) {
      cg = p.C ? p.C + (int64_t)g * p.c_gstride : p.C_ptrs[g];
      row0 = i0;
    } else {
      cg = p.C;
      row0 = g_off + i0;
    }
    const float *bias_g = p.bias ? p.bias + (int64_t)g * p.cols_j : (p.bias_ptrs ? p.bias_ptrs[g] : nullptr);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t il = i0 + ty * 4 + u;
      if (il >= i_ext) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t j = j0 + tx * 4 + v;
        if (j >= p.cols_j) continue;
        float r = acc[u][v];
        if (bias_g) r += bias_g[j];
        float *dst = cg + (row0 + ty * 4 + u) * p.ldc + j;
        if (p.accumulate) r += *dst;
        *dst = r;
      }
    }
  }
}

static int grid_for(int64_t items) { return (int)(items < 2048 ? (items > 0 ? items : 1) : 2048); }

hipError_t launch_forward_f32(int G, int64_t K, int64_t N, int64_t T, const float *x, const float *w,
                              const float *const *w_ptrs, const float *bias, const float *const *bias_ptrs,
                              float *y, const void *ws, hipStream_t s) {
  GemmF32Params p{};
  p.A = x; p.a_si = K; p.a_sp = 1;
  p.B = w; p.B_ptrs = w_ptrs; p.b_gstride = N * K; p.b_sj = K; p.b_sp = 1;
  p.C = y; p.ldc = N;
  p.bias = bias; p.bias_ptrs = bias_ptrs;
  p.ws = ws; p.G = G; p.T = T; p.cols_j = N; p.P = K;
  p.tiles_j = (int)((N + kF32Tile - 1) / kF32Tile);
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(grid_for(((T + kF32Tile - 1) / kF32Tile + G) * p.tiles_j)),
                     dim3(kF32Threads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_dgrad_f32(int G, int64_t K, int64_t N, int64_t T, const float *dy, const float *w,
                            const float *const *w_ptrs, float *dx, const void *ws, hipStream_t s) {
  GemmF32Params p{};
  p.A = dy; p.a_si = N; p.a_sp = 1;
  p.B = w; p.B_ptrs = w_ptrs; p.b_gstride = N * K; p.b_sj = 1; p.b_sp = K;
  p.C = dx; p.ldc = K;
  p.ws = ws; p.G = G; p.T = T; p.cols_j = K; p.P = N;
  p.tiles_j = (int)((K + kF32Tile - 1) / kF32Tile);
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(grid_for(((T + kF32Tile - 1) / kF32Tile + G) * p.tiles_j)),
                     dim3(kF32Threads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_wgrad_f32(int G, int64_t K, int64_t N, int64_t T, const float *x, const float *dy, float *dw,
                            float *const *dw_ptrs, int accumulate, const void *ws, hipStream_t s) {
  GemmF32Params p{};
  p.A = dy; p.a_si = 1; p.a_sp = N;
  p.B = x; p.b_sj = 1; p.b_sp = K;
  p.C = dw; p.C_ptrs = dw_ptrs; p.c_gstride = N * K; p.ldc = K;
  p.ws = ws; p.G = G; p.T = T; p.rows_i = N; p.cols_j = K;
  p.tiles_i = (int)((N + kF32Tile - 1) / kF32Tile);
  p.tiles_j = (int)((K + kF32Tile - 1) / kF32Tile);
  p.accumulate = accumulate;
  p.contr = 1;
  hipLaunchKernelGGL(gemm_f32_kernel, dim3(grid_for((int64_t)G * p.tiles_i * p.tiles_j)), dim3(kF32Threads), 0,
                     s, p);
  return hipGetLastError();
}

}  // namespace gl
