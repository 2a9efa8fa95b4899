"""Pins of the oracle's columnwise MXFP8 group quantization and its MXFP8 dgrad /
wgrad, against things other than themselves:

* a hand-worked example (tests/golden/mxfp8_colwise_hand_worked.json) with an
  unaligned group start, a partial last block and saturation;
* exactness: on inputs that MX represents exactly (integers in [-14, 14], every
  block holding an element of magnitude 8, so every value times 2^5 is an E4M3
  code) the MXFP8 dgrad and wgrad must equal the bf16-path oracle (itself pinned
  by the split/Linear/concat identity and autograd) exactly -- this checks every
  transposition, group offset and padding rule;
* invariants: groups do not leak into each other, padding is zero codes with scale
  byte 0, and the round trip stays within the E4M3 error bound;
* planted mistakes (blocks aligned to the global row instead of the group start,
  unpadded group offsets) that these pins must catch.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import mxfp8 as mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp8_colwise_hand_worked.json")


def test_golden_colwise_example():
    d = json.load(open(GOLDEN))
    codes, scales, poff = oracle.quantize_mxfp8_colwise(np.array(d["x"]), d["m_splits"])
    assert poff.tolist() == d["poff"]
    assert np.array_equal(codes, np.array(d["codes"], dtype=np.uint8))
    assert np.array_equal(scales, np.array(d["scales"], dtype=np.uint8))


def test_golden_weights_example():
    # one group, N = 32, K = 2: column k = 0 holds 1.0 everywhere (e = -8, byte 119,
    # codes 256 -> 0x78), column k = 1 is zero but for n = 5 = -448 (e = 0, byte 127,
    # code 0xFE); stored transposed [K, N]
    w = np.zeros((1, 32, 2))
    w[0, :, 0] = 1.0
    w[0, 5, 1] = -448.0
    q, s = oracle.quantize_mxfp8_colwise_weights(w)
    exp_q = np.zeros((1, 2, 32), dtype=np.uint8)
    exp_q[0, 0, :] = 0x78
    exp_q[0, 1, 5] = 0xFE
    assert np.array_equal(q, exp_q)
    assert s.tolist() == [[[119], [127]]]


def representable(rng, rows, cols, block_axis, starts=None):
    """Integers in [-14, 14] with an element of magnitude 8 at the start of every
    32-block along block_axis (0: rows, blocks restarting at each group start)."""
    v = rng.integers(-14, 15, size=(rows, cols)).astype(np.float64)
    if block_axis == 1:
        v[:, ::32] = 8.0
    else:
        for a, b in zip(starts[:-1], starts[1:]):
            v[a:b:32, :] = -8.0
    return v


@pytest.mark.parametrize("m", [[3, 33, 0, 70], [0, 128, 1], [64, 64], [200]])
def test_mx_backward_exact_on_representable_inputs(m):
    rng = np.random.default_rng(len(m) * 100 + sum(m))
    G, K, N = len(m), 64, 96
    T = sum(m)
    off = np.concatenate([[0], np.cumsum(m)])
    dy_row = representable(rng, T, N, 1)                        # rowwise blocks along N
    x = representable(rng, T, K, 0, off)                        # columnwise blocks along rows
    dy_col = representable(rng, T, N, 0, off)
    w = np.stack([representable(rng, K, N, 1).T for _ in range(G)])  # [G, N, K], blocks along N
    # dgrad: dy rowwise, W columnwise
    dq, ds = oracle.quantize_mxfp8(dy_row)
    wq, ws = oracle.quantize_mxfp8_colwise_weights(w)
    assert np.array_equal(oracle.dequantize_mxfp8(dq, ds), dy_row)
    got = oracle.dgrad_mxfp8(dq, ds, wq, ws, m)
    assert np.array_equal(got, oracle.dgrad(dy_row, w, m))
    # wgrad: dy and x columnwise
    dyq, dys, poff = oracle.quantize_mxfp8_colwise(dy_col, m)
    xq, xs, _ = oracle.quantize_mxfp8_colwise(x, m, ld=int(poff[-1]) + 64)
    got = oracle.wgrad_mxfp8(dyq, dys, xq[:, : poff[-1]], xs[:, : poff[-1] // 32], m)
    assert np.array_equal(got, oracle.wgrad(x, dy_col, m))
    mg = rng.standard_normal((G, N, K))
    got = oracle.wgrad_mxfp8(dyq, dys, xq[:, : poff[-1]], xs[:, : poff[-1] // 32], m, main_grad=mg,
                             accumulate=True)
    assert np.array_equal(got, oracle.wgrad(x, dy_col, m, main_grad=mg, accumulate=True))


def test_groups_do_not_leak_and_padding_is_zero():
    rng = np.random.default_rng(5)
    m = [40, 0, 130, 7]
    T, C = sum(m), 48
    v = rng.standard_normal((T, C))
    q1, s1, poff = oracle.quantize_mxfp8_colwise(v, m)
    v2 = v.copy()
    v2[40:170] *= 1000.0          # group 2 only
    q2, s2, _ = oracle.quantize_mxfp8_colwise(v2, m)
    for g in (0, 3):
        a, b = poff[g], poff[g + 1]
        assert np.array_equal(q1[:, a:b], q2[:, a:b]) and np.array_equal(s1[:, a // 32: b // 32], s2[:, a // 32: b // 32])
    for g, mg in enumerate(m):
        pad_start = poff[g] + mg
        assert not q1[:, pad_start: poff[g + 1]].any()
        first_pad_block = -(-pad_start // 32)
        assert not s1[:, first_pad_block: poff[g + 1] // 32].any()


def test_round_trip_within_e4m3_bound():
    rng = np.random.default_rng(9)
    m = [33, 100, 1]
    v = rng.standard_normal((sum(m), 64)) * np.exp(rng.uniform(-4, 4, size=(1, 64)))
    q, s, poff = oracle.quantize_mxfp8_colwise(v, m)
    deq = oracle.dequantize_mxfp8(q, s)
    off = np.concatenate([[0], np.cumsum(m)])
    for g in range(len(m)):
        back = deq[:, poff[g]: poff[g] + m[g]].T
        e = (s[:, poff[g] // 32: (poff[g] + m[g] + 31) // 32].astype(np.int64) - 127)
        e_rows = np.repeat(e, 32, axis=1)[:, : m[g]].T              # block exponent per element
        a = np.abs(v[off[g]: off[g + 1]])
        bound = 2.0 ** -4 * a + np.ldexp(1.0, e_rows - 10)
        # the floor rule lets the largest elements of a block saturate at 448 * 2^e
        sat = a > 448.0 * np.ldexp(1.0, e_rows)
        bound = np.where(sat, a - 448.0 * np.ldexp(1.0, e_rows), bound)
        assert (np.abs(back - v[off[g]: off[g + 1]]) <= bound * (1 + 1e-12)).all()


def test_planted_mistakes_are_caught(monkeypatch):
    d = json.load(open(GOLDEN))
    x, m = np.array(d["x"]), d["m_splits"]

    # blocks cut at global rows instead of at each group's start: golden codes differ
    v = np.pad(x, ((0, -len(x) % 32), (0, 0))).T
    q, _ = mx.quantize_mxfp8(v)
    assert q.shape != (2, 256) or not np.array_equal(q, np.array(d["codes"], dtype=np.uint8))

    # groups aligned to 32 instead of 128 columns: golden offsets differ
    with monkeypatch.context() as mp:
        mp.setattr(mx, "COLWISE_ALIGN", 32)
        with pytest.raises(AssertionError):
            test_golden_colwise_example()

    # wgrad reading each group from the unpadded row offset: the exactness pin fails
    def bad_wgrad(dytq, dyts, xtq, xts, m_splits, **kw):
        mm = np.asarray(m_splits)
        off = np.concatenate([[0], np.cumsum(mm)])
        dyT, xT = mx.dequantize_mxfp8(dytq, dyts), mx.dequantize_mxfp8(xtq, xts)
        dy = np.concatenate([dyT[:, off[g]: off[g] + mm[g]].T for g in range(len(mm))])
        xx = np.concatenate([xT[:, off[g]: off[g] + mm[g]].T for g in range(len(mm))])
        return oracle.wgrad(xx, dy, mm, **kw)

    with monkeypatch.context() as mp:
        mp.setattr(oracle, "wgrad_mxfp8", bad_wgrad)
        with pytest.raises(AssertionError):
            test_mx_backward_exact_on_representable_inputs([3, 33, 0, 70])
