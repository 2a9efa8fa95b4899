// Persistent grouped GEMM on gfx950 MFMA: bf16 forward, dgrad and wgrad, and the
// MXFP8 (E4M3 data + E8M0 block scales) forward.
//
// All three passes of the grouped linear layer (page
// "transformer_engine/pytorch/ops/basic/grouped_linear.py", fuser_forward "Perform
// GEMMs" and fuser_backward "Perform dgrad GEMMs" / "Perform wgrad GEMMs") are one
// contraction C[i][j] = sum_p A[i][p] * B[j][p] per group, differing only in which
// index is grouped and how operands sit in memory:
//
//   forward  i = token row of group g, j = n, p = k:  A = x  (k contiguous),  B = W_g (k contiguous)
//   dgrad    i = token row of group g, j = k, p = n:  A = dy (n contiguous),  B = W_g (k contiguous)
//   wgrad    i = n, j = k, p = token row of group g:  A = dy (n contiguous),  B = x   (k contiguous)
//
// "K-major" below means the contraction index p is contiguous in memory, "MN-major"
// that the tile index (i or j) is.  Tiles are always staged in LDS K-major (each
// 256-element tile row holds 64 consecutive p values, 128 bytes), so MN-major
// operands are transposed in registers on their way into LDS.
//
// Work decomposition: 256x256 output tiles, 8 waves of 64 lanes (two per SIMD) in a
// 2x4 grid, each wave owning a 128x64 sub-tile as 4x2 blocks of the 32x32x16 bf16
// MFMA with fp32 accumulation.  The grid is persistent (one workgroup per CU);
// workgroup b walks work items b, b+grid, ... where consecutive items of one XCD
// (blockIdx % 8) are neighbouring tiles of the same group, so they share operand
// panels in that XCD's L2.  In row mode the item -> (group, row tile, column tile)
// map comes from the row-tile prefix table the offsets kernel left in the workspace.
//
// MXFP8 forward: the same tiles and LDS layout (a 128-byte tile row now holds 128
// E4M3 codes, handled by the loader as 64 two-byte units), fed to the scaled
// 32x32x64 f8f6f4 MFMA.  Each 32-wide k block of a row has its own E8M0 scale; in a
// 64-deep MFMA step lane l supplies the scale of block (l / 32) of row l % 32, and
// its 32 operand bytes are 16 codes of each of the step's two blocks.
#include "gl_common.hpp"

namespace gl {

constexpr int kBM = 256, kBN = 256, kBK = 64, kThreads = 512;
constexpr int kTileElems = kBM * kBK;  // bf16 elements of one staged operand tile

enum { MODE_ROWS = 0, MODE_CONTR = 1 };

struct GemmBf16Params {
  const uint16_t *A;
  int64_t lda;
  const uint16_t *B;                 // stacked per-group operand (or shared, in wgrad)
  const uint16_t *const *B_ptrs;     // per-group pointers (row mode only), else nullptr
  int64_t b_gstride;                 // elements between groups of B (row mode)
  int64_t ldb;
  void *C;                           // stacked output (wgrad) or token-row output
  void *const *C_ptrs;               // per-group outputs (wgrad), else nullptr
  int64_t c_gstride;
  int64_t ldc;
  const void *bias;                  // [G, cols] of the output type, or nullptr
  const void *const *bias_ptrs;
  const void *ws;
  int G;
  int64_t T;
  int64_t rows_i;                    // extent of i (contraction mode)
  int64_t cols_j;                    // extent of j
  int64_t P;                         // contraction length (row mode)
  int tiles_i, tiles_j;
  int accumulate;
  int out_f32;
  // MXFP8 only: E8M0 scales, one byte per 32 codes of a row
  const uint8_t *a_scale;            // [T, K/32]
  const uint8_t *b_scale;            // [G, N, K/32] stacked, or
  const uint8_t *const *b_scale_ptrs;
  int64_t scale_ld;                  // K / 32
};

// 16-byte slot swizzle inside a 128-byte LDS tile row: conflict-free for the
// 8-row-apart writes of the transposing loader and the consecutive-row fragment
// reads (both for 8-lane and 16-lane bank groups).
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Loads one 256 x 64 operand tile into registers (4 x 16 bytes per thread) and
// later stores it to LDS in K-major layout.
//   KMAJ:  element (r, p) at base[r * ld + p]; rows >= rv are clamped to rv - 1
//          (their products land in output rows that are never stored).
//   !KMAJ: element (r, p) at base[p * ld + r]; each thread loads a 4 (p) x 8 (r)
//          block and transposes it; columns >= rv are clamped to the last valid
//          8-column chunk.
//   In both, contraction indices p >= pmax read as zero.
template <bool KMAJ>
struct TileLoader {
  uint4 v[4];

  __device__ __forceinline__ void load(const uint16_t *__restrict__ base, int64_t ld, int rv, int64_t p0,
                                       int64_t pmax) {
    const int tid = threadIdx.x;
    if (KMAJ) {
      const int kc = tid & 7;
      const int64_t pp = p0 + kc * 8;
      const bool pin = pp < pmax;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int r = (tid >> 3) + 64 * u;
        r = r < rv ? r : rv - 1;
        v[u] = pin ? *(const uint4 *)(base + (int64_t)r * ld + pp) : make_uint4(0, 0, 0, 0);
      }
    } else {
      const int ib = tid & 31, pb = tid >> 5;
      int c = ib * 8;
      const int clast = ((rv - 1) >> 3) << 3;
      c = c < clast ? c : clast;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t pp = p0 + pb * 4 + q;
        v[q] = pp < pmax ? *(const uint4 *)(base + pp * ld + c) : make_uint4(0, 0, 0, 0);
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t *lds) const {
    const int tid = threadIdx.x;
    if (KMAJ) {
      const int kc = tid & 7;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = (tid >> 3) + 64 * u;
        *(uint4 *)(lds + r * kBK + ((kc ^ swz(r)) << 3)) = v[u];
      }
    } else {
      // 4x8 transpose of 16-bit elements: v[q] holds columns c..c+7 of contraction
      // row p0 + 4*pb + q; LDS row c+e receives those 4 contraction values (8 bytes).
      const int ib = tid & 31, pb = tid >> 5;
      const uint32_t *w = (const uint32_t *)v;  // w[q*4 + d] = columns 2d, 2d+1 of row q
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        uint2 o;
        o.x = __builtin_amdgcn_perm(w[1 * 4 + (e >> 1)], w[0 * 4 + (e >> 1)], sel);
        o.y = __builtin_amdgcn_perm(w[3 * 4 + (e >> 1)], w[2 * 4 + (e >> 1)], sel);
        const int r = ib * 8 + e;
        *(uint2 *)(lds + r * kBK + (((pb >> 1) ^ swz(r)) << 3) + ((pb & 1) << 2)) = o;
      }
    }
  }
};

template <bool A_KMAJ, bool B_KMAJ, int MODE, bool MX>
__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(GemmBf16Params p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kTileElems];

  const WsView ws = ws_view(p.ws, p.G);
  if (!ws_usable(ws.hdr, p.G, p.T)) return;
  const int64_t *__restrict__ off = ws.off;
  const int32_t *__restrict__ pre = ws.pre[tile_rows_index(kBM)];

  const int total = MODE == MODE_ROWS ? pre[p.G] * p.tiles_j : p.G * p.tiles_i * p.tiles_j;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int grid = gridDim.x, b = blockIdx.x;
  const int first = (grid & 7) == 0 ? (b & 7) * (grid >> 3) + (b >> 3) : b;

  for (int w = first; w < total; w += grid) {
    // ------------------------------------------------------------ decode item
    int g, it, jt;
    int64_t g_off, g_rows;
    if (MODE == MODE_ROWS) {
      g = find_group(pre, p.G, w / p.tiles_j);
      const int local = w - pre[g] * p.tiles_j;
      const int mt = pre[g + 1] - pre[g];
      it = local % mt;
      jt = local / mt;
    } else {
      const int per = p.tiles_i * p.tiles_j;
      g = w / per;
      const int local = w - g * per;
      it = local % p.tiles_i;
      jt = local / p.tiles_i;
    }
    g_off = off[g];
    g_rows = off[g + 1] - g_off;
    if (MODE == MODE_CONTR && p.accumulate && g_rows == 0) continue;  // untouched

    const uint16_t *a_base, *b_base;
    int a_rv, b_rv;
    int64_t pmax;
    if (MODE == MODE_ROWS) {
      a_base = p.A + (g_off + (int64_t)it * kBM) * p.lda;
      a_rv = (int)min64(kBM, g_rows - (int64_t)it * kBM);
      const uint16_t *bg = p.B ? p.B + (int64_t)g * p.b_gstride : p.B_ptrs[g];
      b_base = B_KMAJ ? bg + (int64_t)jt * kBN * p.ldb : bg + (int64_t)jt * kBN;
      b_rv = (int)min64(kBN, p.cols_j - (int64_t)jt * kBN);
      pmax = p.P;
    } else {
      a_base = p.A + g_off * p.lda + (int64_t)it * kBM;
      a_rv = (int)min64(kBM, p.rows_i - (int64_t)it * kBM);
      b_base = p.B + g_off * p.ldb + (int64_t)jt * kBN;
      b_rv = (int)min64(kBN, p.cols_j - (int64_t)jt * kBN);
      pmax = g_rows;
    }
    const int nk = (int)((pmax + kBK - 1) / kBK);

    // --------------------------------------------------------------- main loop
    f32x16_t acc[4][2];
#pragma unroll
    for (int ii = 0; ii < 4; ++ii)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[ii][jj][q] = 0.f;

    TileLoader<A_KMAJ> la;
    TileLoader<B_KMAJ> lb;
    // MXFP8: scale dwords (4 blocks = one 128-code k tile) of this lane's A and B rows
    uint32_t sca[4] = {0, 0, 0, 0}, scb[2] = {0, 0};
    const uint8_t *a_srow[4], *b_srow[2];
    if (MX) {
      const uint8_t *bs = p.b_scale ? p.b_scale + (int64_t)g * p.cols_j * p.scale_ld : p.b_scale_ptrs[g];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        int r = wm * 128 + ii * 32 + (lane & 31);
        r = r < a_rv ? r : a_rv - 1;
        a_srow[ii] = p.a_scale + (g_off + (int64_t)it * kBM + r) * p.scale_ld;
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        int r = wn * 64 + jj * 32 + (lane & 31);
        r = r < b_rv ? r : b_rv - 1;
        b_srow[jj] = bs + ((int64_t)jt * kBN + r) * p.scale_ld;
      }
    }
    uint32_t nsca[4], nscb[2];
    if (nk > 0) {
      la.load(a_base, p.lda, a_rv, 0, pmax);
      lb.load(b_base, p.ldb, b_rv, 0, pmax);
      if (MX) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) sca[ii] = *(const uint32_t *)a_srow[ii];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) scb[jj] = *(const uint32_t *)b_srow[jj];
      }
      la.store(lds[0][0]);
      lb.store(lds[0][1]);
      __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        la.load(a_base, p.lda, a_rv, (int64_t)(kt + 1) * kBK, pmax);
        lb.load(b_base, p.ldb, b_rv, (int64_t)(kt + 1) * kBK, pmax);
        if (MX) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) nsca[ii] = *(const uint32_t *)(a_srow[ii] + 4 * (kt + 1));
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) nscb[jj] = *(const uint32_t *)(b_srow[jj] + 4 * (kt + 1));
        }
      }
      const uint16_t *sa = lds[cur][0];
      const uint16_t *sb = lds[cur][1];
      if (!MX) {
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
          const int kc = ks * 2 + (lane >> 5);
          bf16x8_t af[4], bfr[2];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int r = wm * 128 + ii * 32 + (lane & 31);
            af[ii] = *(const bf16x8_t *)(sa + r * kBK + ((kc ^ swz(r)) << 3));
          }
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int r = wn * 64 + jj * 32 + (lane & 31);
            bfr[jj] = *(const bf16x8_t *)(sb + r * kBK + ((kc ^ swz(r)) << 3));
          }
          // operands swapped so each lane ends up with 4 consecutive output columns
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
              acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[jj], af[ii], acc[ii][jj], 0, 0, 0);
        }
      } else {
        const int h = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          // 16-byte chunks of the 128-byte row: block 2ks holds chunks 4ks..4ks+1,
          // block 2ks+1 chunks 4ks+2..4ks+3; lane half h takes one chunk of each
          const int c0 = 4 * ks + h, c1 = 4 * ks + 2 + h;
          i32x8_t af[4], bfr[2];
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            const int r = wm * 128 + ii * 32 + (lane & 31);
            const i32x4_t lo = *(const i32x4_t *)(sa + r * kBK + ((c0 ^ swz(r)) << 3));
            const i32x4_t hi = *(const i32x4_t *)(sa + r * kBK + ((c1 ^ swz(r)) << 3));
            af[ii] = (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int r = wn * 64 + jj * 32 + (lane & 31);
            const i32x4_t lo = *(const i32x4_t *)(sb + r * kBK + ((c0 ^ swz(r)) << 3));
            const i32x4_t hi = *(const i32x4_t *)(sb + r * kBK + ((c1 ^ swz(r)) << 3));
            bfr[jj] = (i32x8_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
          const int sh = 8 * (2 * ks + h);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
              acc[ii][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                  bfr[jj], af[ii], acc[ii][jj], 0, 0, 0, (int)(scb[jj] >> sh), 0, (int)(sca[ii] >> sh));
        }
      }
      if (more) {
        la.store(lds[cur ^ 1][0]);
        lb.store(lds[cur ^ 1][1]);
        if (MX) {
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) sca[ii] = nsca[ii];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) scb[jj] = nscb[jj];
        }
      }
      __syncthreads();
    }

    // ---------------------------------------------------------------- epilogue
    // lane holds C[i][j..j+3] with i = ii*32 + lane%32, j = jj*32 + q4*8 + (lane/32)*4
    char *cbase;
    int64_t row0;
    if (MODE == MODE_ROWS) {
      cbase = (char *)p.C;
      row0 = g_off + (int64_t)it * kBM;
    } else {
      cbase = p.C ? (char *)p.C + (int64_t)g * p.c_gstride * (p.out_f32 ? 4 : 2) : (char *)p.C_ptrs[g];
      row0 = (int64_t)it * kBM;
    }
    const char *bias_g = nullptr;
    if (p.bias) bias_g = (const char *)p.bias + (int64_t)g * p.cols_j * (p.out_f32 ? 4 : 2);
    else if (p.bias_ptrs) bias_g = (const char *)p.bias_ptrs[g];
    const int i_valid = a_rv;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int il = wm * 128 + ii * 32 + (lane & 31);
      if (il >= i_valid) continue;
      const int64_t row = row0 + il;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int jl = wn * 64 + jj * 32 + q4 * 8 + (lane >> 5) * 4;
          if (jl >= b_rv) continue;
          const int64_t col = (int64_t)jt * kBN + jl;
          float v0 = acc[ii][jj][q4 * 4 + 0], v1 = acc[ii][jj][q4 * 4 + 1];
          float v2 = acc[ii][jj][q4 * 4 + 2], v3 = acc[ii][jj][q4 * 4 + 3];
          if (bias_g) {
            if (p.out_f32) {
              const float4 bv = *(const float4 *)(bias_g + col * 4);
              v0 += bv.x; v1 += bv.y; v2 += bv.z; v3 += bv.w;
            } else {
              const uint2 bv = *(const uint2 *)(bias_g + col * 2);
              v0 += bf16_to_f32(bv.x & 0xffff); v1 += bf16_to_f32(bv.x >> 16);
              v2 += bf16_to_f32(bv.y & 0xffff); v3 += bf16_to_f32(bv.y >> 16);
            }
          }
          if (p.out_f32) {
            float4 *dst = (float4 *)(cbase + (row * p.ldc + col) * 4);
            if (p.accumulate) {
              const float4 o = *dst;
              v0 += o.x; v1 += o.y; v2 += o.z; v3 += o.w;
            }
            *dst = make_float4(v0, v1, v2, v3);
          } else {
            uint2 *dst = (uint2 *)(cbase + (row * p.ldc + col) * 2);
            if (p.accumulate) {
              const uint2 o = *dst;
              v0 += bf16_to_f32(o.x & 0xffff); v1 += bf16_to_f32(o.x >> 16);
              v2 += bf16_to_f32(o.y & 0xffff); v3 += bf16_to_f32(o.y >> 16);
            }
            *dst = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
          }
        }
      }
    }
  }
}

// Compute units of the current device (one persistent workgroup per CU).
static int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || n <= 0)
    n = 256;
  return n;
}

static int persistent_grid(int64_t max_items) {
  const int cus = num_cus();
  int64_t g = max_items < cus ? max_items : cus;
  if (g >= 8) g &= ~7;  // keep the XCD-aware remap a bijection
  return (int)(g > 0 ? g : 1);
}

// MXFP8 forward: y = deq(xq) deq(wq)^T (+ b).  Codes travel as two-byte units, so the
// loader sees K/2 units per row; K % 128 == 0 keeps scale dwords aligned.
hipError_t launch_forward_mxfp8(int G, int64_t K, int64_t N, int64_t T, const uint8_t *xq, const uint8_t *xs,
                                const uint8_t *wq, const uint8_t *const *wq_ptrs, const uint8_t *ws_scale,
                                const uint8_t *const *ws_scale_ptrs, const void *bias,
                                const void *const *bias_ptrs, void *y, int out_f32, const void *ws,
                                hipStream_t s) {
  GemmBf16Params p{};
  p.A = (const uint16_t *)xq; p.lda = K / 2;
  p.B = (const uint16_t *)wq; p.B_ptrs = (const uint16_t *const *)wq_ptrs; p.b_gstride = N * K / 2; p.ldb = K / 2;
  p.C = y; p.ldc = N;
  p.bias = bias; p.bias_ptrs = bias_ptrs;
  p.ws = ws; p.G = G; p.T = T;
  p.cols_j = N; p.P = K / 2;
  p.tiles_j = (int)((N + kBN - 1) / kBN);
  p.out_f32 = out_f32;
  p.a_scale = xs; p.b_scale = ws_scale; p.b_scale_ptrs = ws_scale_ptrs; p.scale_ld = K / 32;
  const int64_t max_items = ((T + kBM - 1) / kBM + G) * p.tiles_j;
  hipLaunchKernelGGL((gemm_mfma_kernel<true, true, MODE_ROWS, true>), dim3(persistent_grid(max_items)),
                     dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace gl
