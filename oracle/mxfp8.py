"""Float64 CPU oracle of MXFP8 group quantization -- test infrastructure only.

Format (page "transformer_engine/pytorch/ops/basic/grouped_linear.py",
``_quantize_weights_mxfp8``): E4M3 data bytes with one shared scale per block of
32 consecutive elements along the inner (in_features) dimension; the rowwise
scale tensor has in_features // 32 columns.  The pages do not state how the
shared scale is chosen; the workload names OCP MX, so this follows the OCP
Microscaling Formats v1.0 conversion (section on converting vectors to MX):

1. amax = max |v| over the 32 block values;
2. shared exponent e = floor(log2(amax)) - 8, where 8 is the largest exponent
   of an E4M3 normal (448 = 1.75 * 2^8); e is clamped to [-127, 127]; an all-zero
   block takes e = -127; the scale byte is the E8M0 code e + 127;
3. each element is v * 2^-e rounded to E4M3 by round-to-nearest-even, with
   magnitudes above 448 saturated to 448 and the sign of zero kept;
4. a block holding NaN or Inf gets scale byte 0xFF and NaN codes 0x7F | sign.

E4M3 ("fn" variant): 1 sign, 4 exponent (bias 7), 3 mantissa bits; normals
2^-6 .. 448, subnormals k * 2^-9 (k = 1..7), no infinities, NaN = S.1111.111.
"""
from __future__ import annotations

import numpy as np

from . import grouped_linear

E4M3_MAX = 448.0
BLOCK = 32


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2(a)) for finite a > 0, exact (taken from the binary exponent)."""
    _, ex = np.frexp(a)          # a = mant * 2^ex with mant in [0.5, 1)
    return ex.astype(np.int64) - 1


def e4m3_round(s) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value (ties to even), saturating
    magnitudes above 448 to 448.  Returns float64 values that E4M3 represents
    exactly; the sign of zero is kept."""
    s = np.asarray(s, dtype=np.float64)
    a = np.minimum(np.abs(s), E4M3_MAX)
    safe = np.where(a > 0, a, 1.0)
    # Spacing of E4M3 values around a: 2^(E-3) in binade [2^E, 2^(E+1)), E >= -6;
    # below 2^-6 the subnormal spacing 2^-9.
    E = np.maximum(_floor_log2(safe), -6)
    quantum = np.ldexp(1.0, E - 3)
    r = np.rint(a / quantum) * quantum        # a / quantum is exact; rint ties to even
    r = np.minimum(r, E4M3_MAX)
    r = np.where(a > 0, r, 0.0)
    return np.copysign(r, s)


def e4m3_encode(v) -> np.ndarray:
    """Byte code of float64 values that are exactly representable in E4M3."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.uint8) << 7
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = (a > 0) & (a < 2.0 ** -6)
    code[sub] = np.rint(a[sub] / 2.0 ** -9).astype(np.int64)
    nrm = a >= 2.0 ** -6
    E = _floor_log2(np.where(nrm, a, 1.0))
    mant = np.rint((a / np.ldexp(1.0, E) - 1.0) * 8.0).astype(np.int64)
    code = np.where(nrm, ((E + 7) << 3) | mant, code)
    if np.any(code > 0x7E) or np.any((a > 0) & ~nrm & (code > 7)):
        raise ValueError("value not representable in E4M3")
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """Float64 value of E4M3 byte codes (0x7F / 0xFF decode to NaN)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def quantize_mxfp8(src):
    """Rowwise MXFP8 quantization of a [rows, K] array (K a multiple of 32).

    Returns (codes uint8 [rows, K], scales uint8 [rows, K // 32]).  Each row is
    cut into blocks of 32 consecutive elements; blocks never straddle rows, so
    the result does not depend on how rows are split into groups.
    """
    v = np.asarray(src, dtype=np.float64)
    rows, K = v.shape
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blk = v.reshape(rows, K // BLOCK, BLOCK)
    finite = np.isfinite(blk).all(axis=2)
    amax = np.abs(np.where(np.isfinite(blk), blk, 0.0)).max(axis=2)
    e = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)) - 8, -127)
    e = np.clip(e, -127, 127)
    scales = (e + 127).astype(np.uint8)
    scaled = blk * np.ldexp(1.0, -e)[:, :, None]
    scaled = np.where(np.isfinite(blk), scaled, 0.0)
    codes = e4m3_encode(e4m3_round(np.clip(scaled, -E4M3_MAX, E4M3_MAX)))
    nan_code = (np.signbit(blk).astype(np.uint8) << 7) | np.uint8(0x7F)
    codes = np.where(finite[:, :, None], codes, nan_code).astype(np.uint8)
    scales = np.where(finite, scales, np.uint8(0xFF)).astype(np.uint8)
    return codes.reshape(rows, K), scales


def dequantize_mxfp8(codes, scales) -> np.ndarray:
    """value(code) * 2^(scale - 127) per element; scale byte 0xFF is NaN."""
    c = np.asarray(codes)
    s = np.asarray(scales, dtype=np.int64)
    rows, K = c.shape
    mult = np.where(s == 0xFF, np.nan, np.ldexp(1.0, s - 127))
    return (e4m3_decode(c).reshape(rows, K // BLOCK, BLOCK) * mult[:, :, None]).reshape(rows, K)


def forward_mxfp8(xq, xs, wq, ws, b, m_splits, rows=None) -> np.ndarray:
    """MXFP8 grouped forward: the grouped forward evaluated on the dequantized
    operands, i.e. on exactly the rounded values the quantized GEMM consumes.

    xq/xs: [T, K] codes and [T, K/32] scales; wq/ws: [G, N, K] and [G, N, K/32]
    (or per-group sequences).  Dequantization is exact in float64.
    """
    x = dequantize_mxfp8(xq, xs)

    class _Groups:  # dequantizes one group's weight when the forward asks for it
        def __len__(self):
            return len(m_splits)

        def __getitem__(self, g):
            return dequantize_mxfp8(wq[g], ws[g])

    return grouped_linear.forward(x, _Groups(), b, m_splits, rows=rows)


# ---------------------------------------------------------------- columnwise
# The backward pass of the quantized GroupedLinear (page
# "transformer_engine/pytorch/ops/basic/grouped_linear.py", op_forward / fuser_backward:
# the input and grad-output quantizers take columnwise usage when the weight needs a
# gradient, the weight quantizer when the input does; split_quantize quantizes each
# split on its own) contracts over token rows in wgrad and over out_features in dgrad,
# so those operands are quantized in blocks of 32 along the rows instead.
#
# Layout (a reading of this library, not of the pages): columnwise codes are stored
# transposed, so the 32 values of a block are contiguous.  For activations split into
# groups the transposed matrix is [cols, ld]; group g's rows start at column
# COLWISE_ALIGN-aligned offset poff[g] and are followed by zero padding up to the next
# multiple of COLWISE_ALIGN.  A group's last block may hold fewer than 32 real rows;
# the zero padding leaves its amax unchanged, so it is quantized as the padded block.
# Padding blocks are all zero: codes 0, scale byte 0 (the OCP code of an all-zero
# block, 2^-127, finite).

COLWISE_ALIGN = 128


def colwise_offsets(m_splits) -> np.ndarray:
    """Start column of each group's rows in the transposed columnwise layout:
    exclusive prefix of ceil(m_g / 128) * 128, with the total last."""
    m = np.asarray(m_splits, dtype=np.int64)
    pad = -(-m // COLWISE_ALIGN) * COLWISE_ALIGN
    return np.concatenate([[0], np.cumsum(pad)]).astype(np.int64)


def quantize_mxfp8_colwise(src, m_splits, ld=None):
    """Columnwise MXFP8 group quantization of a [T, C] array split into row groups.

    Returns (codes uint8 [C, ld], scales uint8 [C, ld // 32], poff int64 [G + 1]):
    per group and column, blocks of 32 consecutive rows of the group, stored
    transposed from column poff[g].  ld defaults to poff[G]; columns past poff[G]
    are zero here (the library leaves them untouched).
    """
    v = np.asarray(src, dtype=np.float64)
    T, C = v.shape
    m = np.asarray(m_splits, dtype=np.int64)
    if m.sum() != T:
        raise ValueError("split sizes must add up to the row count")
    off = np.concatenate([[0], np.cumsum(m)])
    poff = colwise_offsets(m)
    ld = int(poff[-1]) if ld is None else int(ld)
    if ld < poff[-1] or ld % BLOCK:
        raise ValueError("ld must hold every padded group and be a multiple of 32")
    codes = np.zeros((C, ld), dtype=np.uint8)
    scales = np.zeros((C, ld // BLOCK), dtype=np.uint8)
    for g in range(len(m)):
        width = int(poff[g + 1] - poff[g])
        if width == 0:
            continue
        block = np.zeros((C, width))
        block[:, : m[g]] = v[off[g]: off[g + 1]].T
        q, s = quantize_mxfp8(block)
        codes[:, poff[g]: poff[g + 1]] = q
        scales[:, poff[g] // BLOCK: poff[g + 1] // BLOCK] = s
    return codes, scales, poff


def quantize_mxfp8_colwise_weights(w):
    """Columnwise MXFP8 of grouped weights [G, N, K] (blocks of 32 along N, the
    dgrad contraction), stored transposed: codes [G, K, N], scales [G, K, N // 32]."""
    w = np.asarray(w, dtype=np.float64)
    G, N, K = w.shape
    if N % BLOCK:
        raise ValueError("N must be a multiple of 32")
    codes = np.zeros((G, K, N), dtype=np.uint8)
    scales = np.zeros((G, K, N // BLOCK), dtype=np.uint8)
    for g in range(G):
        codes[g], scales[g] = quantize_mxfp8(w[g].T)
    return codes, scales


def dgrad_mxfp8(dyq, dys, wtq, wts, m_splits, rows=None) -> np.ndarray:
    """MXFP8 grouped dgrad dx_g = dy_g W_g on the dequantized operands: dy from its
    rowwise codes [T, N] (blocks along N), W_g from its columnwise codes stored
    transposed [K, N] (per group, or [G, K, N])."""
    dy = dequantize_mxfp8(dyq, dys)

    class _Groups:
        def __len__(self):
            return len(m_splits)

        def __getitem__(self, g):
            return dequantize_mxfp8(wtq[g], wts[g]).T   # [N, K]

    return grouped_linear.dgrad(dy, _Groups(), m_splits, rows=rows)


def wgrad_mxfp8(dytq, dyts, xtq, xts, m_splits, main_grad=None, accumulate: bool = False, groups=None,
                out_rows=None) -> np.ndarray:
    """MXFP8 grouped wgrad dW_g = dy_g^T x_g on the dequantized columnwise operands:
    dy from codes [N, ld] and x from codes [K, ld] in the transposed group layout."""
    m = np.asarray(m_splits, dtype=np.int64)
    poff = colwise_offsets(m)
    dyT = dequantize_mxfp8(dytq, dyts)
    xT = dequantize_mxfp8(xtq, xts)
    dy = np.concatenate([dyT[:, poff[g]: poff[g] + m[g]].T for g in range(len(m))], axis=0)
    x = np.concatenate([xT[:, poff[g]: poff[g] + m[g]].T for g in range(len(m))], axis=0)
    return grouped_linear.wgrad(x, dy, m, main_grad=main_grad, accumulate=accumulate, groups=groups,
                                out_rows=out_rows)
