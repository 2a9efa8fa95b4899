// Persistent grouped GEMM for bf16 on gfx950 MFMA: forward, dgrad and wgrad.
//
// All three passes of the grouped linear layer (page
// "transformer_engine/pytorch/ops/basic/grouped_linear.py", fuser_forward "Perform
// GEMMs" and fuser_backward "Perform dgrad GEMMs" / "Perform wgrad GEMMs") are one
// contraction C[i][j] = sum_p A[i][p] * B[j][p] per group, differing only in which
// index is grouped and how the operands sit in memory:
//
//   forward  i = token row of group g, j = n, p = k:  A = x  (p contiguous), B = W_g (p contiguous)
//   dgrad    i = token row of group g, j = k, p = n:  A = dy (p contiguous), B = W_g (j contiguous)
//   wgrad    i = n, j = k, p = token row of group g:  A = dy (i contiguous), B = x   (j contiguous)
//
// Tiles: 256x256 outputs per workgroup, 8 waves (two per SIMD) in a 2x4 grid, each
// wave a 128x64 block of 32x32x16 bf16 MFMAs with fp32 accumulators (GL_WAVES=4
// builds 4 waves of 128x128 instead).
//
// Operand staging: the contraction advances 32 at a time through a 4-stage LDS ring
// (16 KiB per operand per stage), filled by direct global->LDS loads
// (global_load_lds, 16 bytes per lane) issued three tiles ahead of the MFMAs, with a
// single workgroup barrier per tile.  An operand whose contraction index is
// contiguous ("K-major") is staged as 256 rows of 64 bytes and read with 16-byte
// LDS loads; one whose tile index is contiguous ("MN-major") is staged as 32 rows
// of 512 bytes and read with the gfx950 LDS transpose load (ds_read_b64_tr_b16),
// which hands each lane 4 consecutive contraction values of one column -- exactly
// the MFMA operand layout -- so no operand is ever transposed in registers.  Both
// layouts XOR-swizzle 16-byte slots so the fragment reads are bank-conflict free.
//
// Masking: rows past the valid extent of a K-major tile are clamped onto a valid
// row (their products land in output rows that are never stored); columns past an
// MN-major tile's extent are clamped likewise; contraction indices past the end
// (the last tile of a group in wgrad, or a contraction length not a multiple of
// 32) are not loaded -- those lanes write zeros into their LDS slot instead.
//
// Scheduling: persistent grid, one workgroup per CU; workgroup b walks items b,
// b + grid, ...; items are remapped so each XCD (blockIdx % 8) works on a
// contiguous run of neighbouring tiles that share operand panels in its L2.  In row
// mode the item -> (group, row tile, column tile) map comes from the row-tile
// prefix table the offsets kernel left in the workspace.
#include "gl_common.hpp"

namespace gl {

namespace v2 {

#ifndef GL_WAVES
#define GL_WAVES 8
#endif
#ifndef GL_TILE_ORDER
#define GL_TILE_ORDER 1
#endif
#ifndef GL_INTERLEAVE
#define GL_INTERLEAVE 1
#endif

constexpr int kBM = 256, kBN = 256, kBK = 32, kStages = 4;
constexpr int kWaves = GL_WAVES, kThreads = 64 * kWaves;
constexpr int kWM = 2, kWN = kWaves / kWM;           // wave grid
constexpr int kWTM = kBM / kWM, kWTN = kBN / kWN;    // wave tile
constexpr int kNI = kWTM / 32, kNJ = kWTN / 32;      // 32x32 MFMA blocks per wave
constexpr int kOpElems = 256 * kBK;                  // bf16 elements per operand per stage
constexpr int kPieces = kOpElems * 2 / 1024;         // 1 KiB direct-load pieces per operand per stage
constexpr int kLoadsPerTile = 2 * kPieces / kWaves;  // direct-to-LDS instructions per wave per tile
// blocked tile order: each XCD's run of neighbouring work items covers a
// kOrdM x kOrdN block of output tiles
constexpr int kOrdM = 8, kOrdN = 4;

enum { MODE_ROWS = 0, MODE_CONTR = 1 };

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define GL_LDS __attribute__((address_space(3)))

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
};

// 16-byte slot swizzles, chosen for gfx950's LDS (64 banks of 4 bytes; a 16-byte
// read serves 16 lanes per cycle, an 8-byte read 32 lanes).
// K-major rows are 64 bytes (4 slots): chunk c of row r sits in slot c ^ swz_k(r).
// A fragment read takes one chunk of 16 consecutive rows per cycle; rows r and
// r + 4k share a 256-byte bank window, so the slot must differ across r >> 2.
// MN-major rows are 512 bytes (32 slots): chunk c of contraction row p sits in slot
// c ^ swz_m(p).  A transpose read serves 4 rows x 64 bytes per 32 lanes; the rows
// are 512 bytes apart (same banks), so the XOR moves each row's 64 bytes to its own
// quarter of the 256-byte window.
__device__ __forceinline__ int swz_k(int r) { return (r >> 2) & 3; }
__device__ __forceinline__ int swz_m(int p) { return (p & 3) << 2; }

// s_waitcnt immediate for vmcnt(n) that leaves expcnt and lgkmcnt unconstrained
constexpr int vm_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0f70; }

// Wait until at most `tiles` tiles' worth of this wave's direct loads are in flight.
__device__ __forceinline__ void wait_vm_tiles(int tiles) {
  if (tiles <= 0) __builtin_amdgcn_s_waitcnt(vm_imm(0));
  else if (tiles == 1) __builtin_amdgcn_s_waitcnt(vm_imm(kLoadsPerTile));
  else __builtin_amdgcn_s_waitcnt(vm_imm(2 * kLoadsPerTile));
}

__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

constexpr int kQ = kPieces / kWaves;  // direct-load pieces per wave per operand per tile

// Direct global->LDS loads of one operand, one 256 x 32 tile per contraction step.
// A wave owns the 1 KiB pieces wave, wave + kWaves, ... of each 16 KiB operand
// stage; lane l of a piece fills bytes [16 l, 16 l + 16) of it.  Per lane the
// global address of a piece is a fixed 32-bit offset from a wave-uniform tile base
// that advances by `step` bytes per tile, so issuing a full tile is straight-line
// code: no per-lane predicate, no 64-bit address arithmetic.
template <bool KMAJ>
struct Stream {
  const char *base;  // operand tile base for contraction tile 0
  int64_t step;      // bytes per contraction tile
  uint32_t off[kQ];  // lane byte offsets of its pieces
  int pfirst[kQ];    // first contraction index (within the tile) a lane's piece holds

  // K-major: element (r, p) at b[r * ld + p]; rows >= rv clamp to rv - 1.
  // MN-major: element (r, p) at b[p * ld + r]; columns >= rv clamp to the last
  // valid 8-column chunk (rv is a multiple of 8).
  __device__ __forceinline__ void init(const uint16_t *b, int64_t ld, int rv, int wave, int lane) {
    base = (const char *)b;
    step = KMAJ ? kBK * 2 : (int64_t)kBK * ld * 2;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int u = wave + kWaves * q;
      if (KMAJ) {
        const int R = 16 * u + (lane >> 2);
        const int c = (lane & 3) ^ swz_k(R);
        const int r = R < rv ? R : rv - 1;
        off[q] = (uint32_t)(((int64_t)r * ld + c * 8) * 2);
        pfirst[q] = c * 8;
      } else {
        const int prow = 2 * u + (lane >> 5);
        int col = ((lane & 31) ^ swz_m(prow)) * 8;
        col = col < rv - 8 ? col : rv - 8;
        off[q] = (uint32_t)(((int64_t)prow * ld + col) * 2);
        pfirst[q] = prow;
      }
    }
  }

  // All contraction indices of tile t are valid.
  __device__ __forceinline__ void issue_full(int t, char *st, int wave) const {
    const char *tb = base + (int64_t)t * step;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
      __builtin_amdgcn_global_load_lds(tb + off[q], (GL_LDS void *)(st + (wave + kWaves * q) * 1024), 16, 0, 0);
  }

  // The last tile of a contraction: lanes whose piece lies past pmax write zeros
  // into their LDS slot instead of loading.
  __device__ __forceinline__ void issue_masked(int t, int64_t pmax, char *st, int wave, int lane) const {
    const char *tb = base + (int64_t)t * step;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      char *dst = st + (wave + kWaves * q) * 1024;
      if ((int64_t)t * kBK + pfirst[q] < pmax)
        __builtin_amdgcn_global_load_lds(tb + off[q], (GL_LDS void *)dst, 16, 0, 0);
      else
        *(uint4 *)(dst + lane * 16) = make_uint4(0, 0, 0, 0);
    }
  }
};

// MFMA operand fragment (32 rows/columns x 16 contraction values; lane l holds row
// l % 32, contraction values 8 * (l / 32) + 0..7) for contraction step ks of a stage.
__device__ __forceinline__ bf16x8_t frag_kmaj(const uint16_t *st, int row0, int ks, int lane) {
  const int r = row0 + (lane & 31);
  const int c = 2 * ks + (lane >> 5);
  return *(const bf16x8_t *)(st + r * kBK + ((c ^ swz_k(r)) << 3));
}

__device__ __forceinline__ bf16x8_t frag_mnmaj(const uint16_t *st, int col0, int ks, int lane) {
  // 16-lane groups: lanes 0-15 / 16-31 take columns 0-15 / 16-31, lane halves take
  // contraction rows 0-7 / 8-7; lane s of a group names row (s / 4) and columns
  // 4 (s % 4) .. + 3, and the transpose hands lane s column s of those 4 rows.
  const int s = lane & 15, grp = lane >> 4;
  const int col = col0 + ((grp & 1) << 4) + ((s & 3) << 2);
  const int chunk = col >> 3, within = col & 7;
  v4i16 h[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int prow = ks * 16 + (grp >> 1) * 8 + t * 4 + (s >> 2);
    const uint16_t *a = st + prow * 256 + ((chunk ^ swz_m(prow)) << 3) + within;
    h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GL_LDS v4i16 *)a);
  }
  const v4i16 lo = h[0], hi = h[1];
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

template <bool A_KMAJ, bool B_KMAJ, int MODE>
__global__ __launch_bounds__(kThreads) void gemm_bf16_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) uint16_t lds[kStages][2][kOpElems];

  const WsView ws = ws_view(p.ws, p.G);
  if (!ws_usable(ws.hdr, p.G, p.T)) return;
  const int64_t *__restrict__ off = ws.off;
  const int32_t *__restrict__ pre = ws.pre[tile_rows_index(kBM)];

  const int total = MODE == MODE_ROWS ? pre[p.G] * p.tiles_j : p.G * p.tiles_i * p.tiles_j;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / kWN, wn = wave % kWN;
  const int grid = gridDim.x, b = blockIdx.x;
  const int first = (grid & 7) == 0 ? (b & 7) * (grid >> 3) + (b >> 3) : b;

  for (int w = first; w < total; w += grid) {
    // ------------------------------------------------------------ decode item
    int g, local, MT;
    const int NT = p.tiles_j;
    if (MODE == MODE_ROWS) {
      g = find_group(pre, p.G, w / NT);
      local = w - pre[g] * NT;
      MT = pre[g + 1] - pre[g];
    } else {
      const int per = p.tiles_i * NT;
      g = w / per;
      local = w - g * per;
      MT = p.tiles_i;
    }
    int it, jt;
    if (GL_TILE_ORDER == 0) {
      it = local % MT;
      jt = local / MT;
    } else {
      // bands of kOrdN tile columns; inside a band, blocks of kOrdM tile rows;
      // inside a block, row tiles fastest
      const int cb = local / (MT * kOrdN);
      const int bw = min(kOrdN, NT - cb * kOrdN);
      const int l2 = local - cb * MT * kOrdN;
      const int rb = l2 / (kOrdM * bw);
      const int h = min(kOrdM, MT - rb * kOrdM);
      const int l3 = l2 - rb * kOrdM * bw;
      it = rb * kOrdM + l3 % h;
      jt = cb * kOrdN + l3 / h;
    }
    const int64_t g_off = off[g];
    const int64_t g_rows = off[g + 1] - g_off;
    if (MODE == MODE_CONTR && p.accumulate && g_rows == 0) continue;  // main_grad untouched

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

    Stream<A_KMAJ> sa;
    Stream<B_KMAJ> sb;
    sa.init(a_base, p.lda, a_rv, wave, lane);
    sb.init(b_base, p.ldb, b_rv, wave, lane);
    char *const ring = (char *)&lds[0][0][0];
    constexpr int kStageBytes = 2 * kOpElems * 2, kOpBytes = kOpElems * 2;
    const int nfull = (int)(pmax / kBK);  // tiles [0, nfull) are complete; nk - nfull <= 1
    auto issue = [&](int t) {
      char *st = ring + (t % kStages) * kStageBytes;
      if (t < nfull) {
        sa.issue_full(t, st, wave);
        sb.issue_full(t, st + kOpBytes, wave);
      } else {
        sa.issue_masked(t, pmax, st, wave, lane);
        sb.issue_masked(t, pmax, st + kOpBytes, wave, lane);
      }
    };
    // Tiles in (lo, hi] whose loads may still be in flight when every tile up to
    // lo must have landed: only complete tiles count, since a masked tile may
    // have issued fewer loads.
    auto inflight_after = [&](int lo, int hi) {
      const int top = min(hi, nfull - 1);
      return top > lo ? top - lo : 0;
    };

    // -------------------------------------------------------------- main loop
    f32x16_t acc[kNI][kNJ];
#pragma unroll
    for (int ii = 0; ii < kNI; ++ii)
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[ii][jj][q] = 0.f;

    auto load_frags = [&](int t, int ks, bf16x8_t *af, bf16x8_t *bfr) {
      const uint16_t *ta = lds[t % kStages][0];
      const uint16_t *tb = lds[t % kStages][1];
#pragma unroll
      for (int ii = 0; ii < kNI; ++ii)
        af[ii] = A_KMAJ ? frag_kmaj(ta, wm * kWTM + ii * 32, ks, lane) : frag_mnmaj(ta, wm * kWTM + ii * 32, ks, lane);
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj)
        bfr[jj] = B_KMAJ ? frag_kmaj(tb, wn * kWTN + jj * 32, ks, lane) : frag_mnmaj(tb, wn * kWTN + jj * 32, ks, lane);
    };
    auto mfmas = [&](const bf16x8_t *af, const bf16x8_t *bfr) {
      // operands swapped so each lane ends up with 4 consecutive output columns
#pragma unroll
      for (int ii = 0; ii < kNI; ++ii)
#pragma unroll
        for (int jj = 0; jj < kNJ; ++jj)
          acc[ii][jj] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[jj], af[ii], acc[ii][jj], 0, 0, 0);
    };

    // Pipeline: tiles are issued kStages - 1 ahead; the barrier closing iteration
    // kt guarantees tile kt + 2 has landed, so tile kt + 1's first fragments are
    // read during tile kt's last MFMAs and the MFMAs resume right after each
    // barrier.  One barrier per tile.
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s)
      if (s < nk) issue(s);
    bf16x8_t f0a[kNI], f0b[kNJ], f1a[kNI], f1b[kNJ];
    if (nk > 0) {
      wait_vm_tiles(inflight_after(min(1, nk - 1), min(2, nk - 1)));
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      load_frags(0, 0, f0a, f0b);
    }
    int kt = 0;
    // steady state: the tile issued this iteration is complete and a next tile
    // exists -- straight-line code, scheduled as interleaved MFMA / memory groups
    for (; kt + kStages - 1 < nfull; ++kt) {
      char *st = ring + ((kt + kStages - 1) % kStages) * kStageBytes;
      sa.issue_full(kt + kStages - 1, st, wave);
      sb.issue_full(kt + kStages - 1, st + kOpBytes, wave);
      load_frags(kt, 1, f1a, f1b);
      mfmas(f0a, f0b);
      load_frags(kt + 1, 0, f0a, f0b);
      mfmas(f1a, f1b);
      if (GL_INTERLEAVE) {
        // 16 MFMAs; between them the 2 kQ direct loads and the 2 (kNI + kNJ)
        // fragment reads (fragment reads of tile kt + 1 can only follow the
        // eighth MFMA, the last reader of the registers they refill)
#pragma unroll
        for (int i = 0; i < 2 * kQ; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 2 * kQ; i < 16; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      wait_vm_tiles(1);
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
    }
    for (; kt < nk; ++kt) {
      if (kt + kStages - 1 < nk) issue(kt + kStages - 1);
      load_frags(kt, 1, f1a, f1b);
      mfmas(f0a, f0b);
      if (kt + 1 < nk) load_frags(kt + 1, 0, f0a, f0b);
      mfmas(f1a, f1b);
      wait_vm_tiles(inflight_after(kt + 2, min(kt + kStages - 1, nk - 1)));
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
    }
    __builtin_amdgcn_s_barrier();  // every wave is done with the ring before it is refilled

    // --------------------------------------------------------------- epilogue
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
#pragma unroll
    for (int ii = 0; ii < kNI; ++ii) {
      const int il = wm * kWTM + ii * 32 + (lane & 31);
      if (il >= a_rv) continue;
      const int64_t row = row0 + il;
#pragma unroll
      for (int jj = 0; jj < kNJ; ++jj) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int jl = wn * kWTN + jj * 32 + q4 * 8 + (lane >> 5) * 4;
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
  if (g >= 8) g &= ~7;  // keeps the XCD-aware remap a bijection
  return (int)(g > 0 ? g : 1);
}

}  // namespace v2

// forward: y = x W^T (+ b); A = x [T,K], B = W [N,K]
hipError_t launch_forward_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *x, const uint16_t *w,
                               const uint16_t *const *w_ptrs, const void *bias, const void *const *bias_ptrs,
                               uint16_t *y, const void *ws, hipStream_t s) {
  using namespace v2;
  Params p{};
  p.A = x; p.lda = K;
  p.B = w; p.B_ptrs = w_ptrs; p.b_gstride = N * K; p.ldb = K;
  p.C = y; p.ldc = N;
  p.bias = bias; p.bias_ptrs = bias_ptrs;
  p.ws = ws; p.G = G; p.T = T;
  p.cols_j = N; p.P = K;
  p.tiles_j = (int)((N + kBN - 1) / kBN);
  const int64_t max_items = ((T + kBM - 1) / kBM + G) * p.tiles_j;
  hipLaunchKernelGGL((gemm_bf16_kernel<true, true, MODE_ROWS>), dim3(persistent_grid(max_items)), dim3(kThreads), 0,
                     s, p);
  return hipGetLastError();
}

// dgrad: dx = dy W; A = dy [T,N] (n contiguous), B[j=k][p=n] = W[n][k] (k contiguous)
hipError_t launch_dgrad_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *dy, const uint16_t *w,
                             const uint16_t *const *w_ptrs, uint16_t *dx, const void *ws, hipStream_t s) {
  using namespace v2;
  Params p{};
  p.A = dy; p.lda = N;
  p.B = w; p.B_ptrs = w_ptrs; p.b_gstride = N * K; p.ldb = K;
  p.C = dx; p.ldc = K;
  p.ws = ws; p.G = G; p.T = T;
  p.cols_j = K; p.P = N;
  p.tiles_j = (int)((K + kBN - 1) / kBN);
  const int64_t max_items = ((T + kBM - 1) / kBM + G) * p.tiles_j;
  hipLaunchKernelGGL((gemm_bf16_kernel<true, false, MODE_ROWS>), dim3(persistent_grid(max_items)), dim3(kThreads), 0,
                     s, p);
  return hipGetLastError();
}

// wgrad: dW_g[n][k] = sum_r dy[r][n] x[r][k]; A[i=n][p=r] (n contiguous), B[j=k][p=r] (k contiguous)
hipError_t launch_wgrad_bf16(int G, int64_t K, int64_t N, int64_t T, const uint16_t *x, const uint16_t *dy,
                             void *dw, void *const *dw_ptrs, int out_f32, int accumulate, const void *ws,
                             hipStream_t s) {
  using namespace v2;
  Params p{};
  p.A = dy; p.lda = N;
  p.B = x; p.ldb = K;
  p.C = dw; p.C_ptrs = dw_ptrs; p.c_gstride = N * K; p.ldc = K;
  p.ws = ws; p.G = G; p.T = T;
  p.rows_i = N; p.cols_j = K;
  p.tiles_i = (int)((N + kBM - 1) / kBM);
  p.tiles_j = (int)((K + kBN - 1) / kBN);
  p.accumulate = accumulate;
  p.out_f32 = out_f32;
  const int64_t max_items = (int64_t)G * p.tiles_i * p.tiles_j;
  hipLaunchKernelGGL((gemm_bf16_kernel<false, false, MODE_CONTR>), dim3(persistent_grid(max_items)), dim3(kThreads),
                     0, s, p);
  return hipGetLastError();
}

}  // namespace gl
