"""Pins of the CPU oracle's MXFP8 quantizer against things other than itself.

* hand-worked blocks (tests/golden/mxfp8_hand_worked.json) under the OCP MX v1.0
  rule the oracle states (shared exponent floor(log2 amax) - 8, RNE, saturation);
* every finite bf16 value at several shared exponents, against torch's own
  float8_e4m3fn conversion of the clamped scaled value (a library routine that
  rounds to nearest-even);
* all 256 E4M3 codes decoded against torch's float8_e4m3fn -> float conversion;
* the OCP scale invariant 2^8 <= amax * 2^-e < 2^9 and the E4M3 round-trip bound;
* independence from the split sizes (rowwise blocks never straddle rows);
* planted mistakes (ceil exponent, truncation, no saturation, wrong block) that
  these pins must catch.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import mxfp8 as mx
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp8_hand_worked.json")


def _golden_blocks():
    d = json.load(open(GOLDEN))
    out = []
    for c in d["cases"]:
        vals = [1.0] * 32 if c["values"] == "ones32" else [float(v) for v in c["values"]]
        blk = np.zeros(32, dtype=np.float64)
        blk[: len(vals)] = vals
        # the fixture's values are bf16 numbers; check that claim rather than assume it
        as_bf16 = torch.tensor(blk, dtype=torch.float64).to(torch.bfloat16).double().numpy()
        assert np.array_equal(as_bf16, blk, equal_nan=True) or np.isnan(blk).any()
        codes = list(c["codes"])
        filler = 0x7F if c["scale"] == 255 else 0x00
        codes += [filler] * (32 - len(codes))
        if c["values"] == "ones32":
            codes = [c["codes"][0]] * 32
        out.append((c["why"], blk, c["scale"], codes))
    return out


def _golden_pins_hold(quant) -> bool:
    try:
        for _, blk, scale, codes in _golden_blocks():
            q, s = quant(blk[None, :])
            if int(s[0, 0]) != scale or q[0].tolist() != codes:
                return False
        return True
    except Exception:
        return False


@pytest.mark.parametrize("case", _golden_blocks(), ids=lambda c: c[0][:40])
def test_hand_worked_block(case):
    why, blk, scale, codes = case
    q, s = oracle.quantize_mxfp8(blk[None, :])
    assert int(s[0, 0]) == scale, why
    assert q[0].tolist() == codes, why


def _torch_e4m3_codes(v64: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v64, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("e", [-127, -20, -8, -3, 0, 5, 40, 119])
def test_element_rounding_matches_torch_for_every_bf16(e):
    v = synth.special_bf16_block_values().double().numpy()
    scaled = np.clip(v * math.ldexp(1.0, -e), -448.0, 448.0)
    fp32_exact = np.abs(scaled) >= 2.0 ** -126   # below that the float32 input itself would round first
    ours = mx.e4m3_encode(mx.e4m3_round(scaled))
    ref = _torch_e4m3_codes(scaled)
    assert np.array_equal(ours[fp32_exact], ref[fp32_exact])
    tiny = ~fp32_exact   # far below E4M3's smallest subnormal: a signed zero
    assert np.array_equal(ours[tiny] & 0x7F, np.zeros(tiny.sum(), np.uint8))


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    ours = mx.e4m3_decode(codes)
    assert np.array_equal(ours, ref, equal_nan=True)
    finite = ~np.isnan(ours)
    assert np.array_equal(mx.e4m3_encode(ours[finite]), codes[finite])


def test_scale_invariant_and_round_trip_bound():
    rng = np.random.default_rng(3)
    mags = np.ldexp(1.0, rng.integers(-140, 120, size=(400, 1)))
    v = torch.from_numpy(rng.standard_normal((400, 256)) * mags).to(torch.bfloat16).double().numpy()
    v[5, 32:64] = 0.0
    q, s = oracle.quantize_mxfp8(v)
    blk = v.reshape(400, 8, 32)
    amax = np.abs(blk).max(axis=2)
    e = s.astype(np.int64) - 127
    nz = (amax > 0) & (e > -127)
    r = amax[nz] * np.ldexp(1.0, -e[nz])
    assert ((r >= 256.0) & (r < 512.0)).all()
    assert (s[amax == 0] == 0).all()
    deq = oracle.dequantize_mxfp8(q, s).reshape(400, 8, 32)
    scaled = np.abs(blk) * np.ldexp(1.0, -e)[:, :, None]
    err = np.abs(deq - blk)
    unit = np.ldexp(1.0, e)[:, :, None]
    normal = (scaled >= 2.0 ** -6) & (scaled <= 448.0)
    assert (err[normal] <= 2.0 ** -4 * np.abs(blk[normal])).all()
    sub = scaled < 2.0 ** -6
    assert (err <= 2.0 ** -10 * unit)[sub].all()
    sat = scaled > 448.0
    assert np.array_equal(np.abs(deq[sat]), (448.0 * unit * np.ones_like(deq))[sat])


def test_independent_of_split_sizes():
    rng = np.random.default_rng(5)
    v = torch.from_numpy(rng.standard_normal((40, 128))).to(torch.bfloat16).double().numpy()
    q, s = oracle.quantize_mxfp8(v)
    parts = [oracle.quantize_mxfp8(p) for p in np.split(v, [7, 7, 30])]
    assert np.array_equal(q, np.concatenate([p[0] for p in parts]))
    assert np.array_equal(s, np.concatenate([p[1] for p in parts]))


def test_rejects_ragged_blocks():
    with pytest.raises(ValueError):
        oracle.quantize_mxfp8(np.zeros((2, 48)))


def test_mx_forward_is_forward_on_decoded_operands():
    rng = np.random.default_rng(9)
    m = [3, 0, 5]
    x = torch.from_numpy(rng.standard_normal((8, 64))).to(torch.bfloat16).double().numpy()
    w = torch.from_numpy(rng.standard_normal((3, 16, 64)) * 0.02).to(torch.bfloat16).double().numpy()
    xq, xs = oracle.quantize_mxfp8(x)
    wqs = [oracle.quantize_mxfp8(w[g]) for g in range(3)]
    y = oracle.forward_mxfp8(xq, xs, [a for a, _ in wqs], [b for _, b in wqs], None, m)
    # decode through torch's own float8 type, independent of the oracle's decoder
    def dec(q, s):
        vals = torch.from_numpy(q).view(torch.float8_e4m3fn).double()
        return (vals.reshape(q.shape[0], -1, 32) * torch.pow(2.0, torch.from_numpy(s.astype(np.float64)) - 127)[
            :, :, None]).reshape(q.shape)
    xd = dec(xq, xs)
    ref = torch.cat([torch.nn.functional.linear(p, dec(*wqs[g])) for g, p in enumerate(torch.split(xd, m))])
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


# --------------------------------------------------------- planted bugs ----

def test_pins_accept_the_oracle():
    assert _golden_pins_hold(oracle.quantize_mxfp8)


def _ceil_log2(a):
    return np.ceil(np.log2(a)).astype(np.int64)


def _truncating_round(s):
    s = np.asarray(s, dtype=np.float64)
    a = np.minimum(np.abs(s), 448.0)
    E = np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), -6)
    q = np.ldexp(1.0, (E - 3).astype(np.int64))
    return np.copysign(np.floor(a / q) * q, s)


def _non_saturating_round(s):
    s = np.asarray(s, dtype=np.float64)
    out = mx.e4m3_round(s)
    return np.where(np.abs(s) > 448.0, np.nan, out)


@pytest.mark.parametrize("attr,value", [
    ("_floor_log2", _ceil_log2),
    ("e4m3_round", _truncating_round),
    ("BLOCK", 16),
])
def test_golden_pins_catch_planted_mistake(monkeypatch, attr, value):
    monkeypatch.setattr(mx, attr, value)
    assert not _golden_pins_hold(mx.quantize_mxfp8)


def test_golden_pins_catch_missing_saturation(monkeypatch):
    real_clip = np.clip

    def no_clip_quant(src):
        monkeypatch.setattr(mx.np, "clip", lambda a, lo, hi: a if lo == -448.0 else real_clip(a, lo, hi))
        monkeypatch.setattr(mx, "e4m3_round", _non_saturating_round)
        try:
            return mx.quantize_mxfp8(src)
        finally:
            monkeypatch.setattr(mx.np, "clip", real_clip)

    assert not _golden_pins_hold(no_clip_quant)
