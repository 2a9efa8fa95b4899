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
