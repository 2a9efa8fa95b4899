"""Pins of the CPU oracle's grouped-linear functions against things other than itself.

* the page's own statement of the method: splitting the rows, applying one
  ``torch.nn.Linear`` per split and concatenating (GroupedLinear class docstring);
* torch autograd through that same split/Linear/concat expression for dgrad,
  wgrad and bias grad;
* a single group reducing to ``torch.nn.Linear``;
* a hand-worked example with integer values (tests/golden);
* the offsets' closed form against ``itertools.accumulate`` at the sizes the
  offsets kernel was tested with (page "Single parameter for GroupedLinear
  module", files table row for test_cumsum.cu: 1, 2, 17, 256, 257, 513, 1024);
* planted mistakes (a dropped term, a wrong index, a transposed operand) that the
  pins above must catch.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import grouped_linear as gl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "grouped_linear_hand_worked.json")


def _case(seed, G, K, N, m):
    g = torch.Generator().manual_seed(seed)
    T = int(sum(m))
    x = torch.randn(T, K, generator=g, dtype=torch.float64)
    w = torch.randn(G, N, K, generator=g, dtype=torch.float64)
    b = torch.randn(G, N, generator=g, dtype=torch.float64)
    dy = torch.randn(T, N, generator=g, dtype=torch.float64)
    mg = torch.randn(G, N, K, generator=g, dtype=torch.float64)
    return x, w, b, dy, mg


CASES = [
    (0, 4, 64, 32, [5, 0, 17, 10]),
    (1, 3, 7, 5, [0, 4, 3]),          # empty first group
    (2, 3, 6, 9, [4, 3, 0]),          # empty last group
    (3, 5, 8, 8, [2, 0, 0, 6, 1]),    # adjacent empty groups, square
    (4, 1, 16, 12, [9]),              # a single group
    (5, 2, 4, 4, [0, 0]),             # no rows at all
]


def _split_linear_cat(x, w, b, m):
    parts = [F.linear(xs, w[g], None if b is None else b[g]) for g, xs in enumerate(torch.split(x, m))]
    return torch.cat(parts) if parts else x.new_zeros((0, w.shape[1]))


# ---------------------------------------------------------------- golden ----

def test_hand_worked_example():
    d = json.load(open(GOLDEN))
    m, e = d["m_splits"], d["expect"]
    x, W, b, dy, mg = (np.array(d[k], dtype=np.float64) for k in ("x", "W", "b", "dy", "main_grad"))
    assert oracle.offsets(m, 3, 3).tolist() == e["offsets"]
    assert oracle.forward(x, W, b, m).tolist() == e["y"]
    assert oracle.dgrad(dy, W, m).tolist() == e["dx"]
    assert oracle.wgrad(x, dy, m).tolist() == e["dW"]
    assert oracle.wgrad(x, dy, m, main_grad=mg, accumulate=True).tolist() == e["dW_accumulated"]
    assert oracle.bgrad(dy, m).tolist() == e["db"]


# --------------------------------------------------------------- offsets ----

@pytest.mark.parametrize("n", [1, 2, 17, 256, 257, 513, 1024])
def test_offsets_closed_form(n):
    rng = np.random.default_rng(n)
    m = rng.integers(0, 50, size=n)
    m[rng.integers(0, n, size=max(1, n // 5))] = 0
    ref = list(itertools.accumulate(m.tolist(), initial=0))
    assert oracle.offsets(m, n, int(m.sum())).tolist() == ref


def test_offsets_known_values():
    assert oracle.offsets([5, 0, 17, 10], 4, 32).tolist() == [0, 5, 5, 22, 32]
    assert oracle.offsets([0, 0, 3], 3, 3).tolist() == [0, 0, 0, 3]
    assert oracle.offsets([3, 0, 0], 3, 3).tolist() == [0, 3, 3, 3]
    assert oracle.offsets([0], 1, 0).tolist() == [0, 0]


@pytest.mark.parametrize("m,G,T", [([1, 2], 3, 3), ([1, -1, 3], 3, 3), ([1, 2, 3], 3, 7)])
def test_offsets_rejects(m, G, T):
    with pytest.raises(ValueError):
        oracle.offsets(m, G, T)


def test_group_of_rows_skips_empty_groups():
    off = oracle.offsets([5, 0, 17, 10], 4, 32)
    assert gl.group_of_rows(off, [0, 4, 5, 21, 22, 31]).tolist() == [0, 0, 2, 2, 3, 3]


# ------------------------------------------------ identity and autograd ----

@pytest.mark.parametrize("seed,G,K,N,m", CASES)
def test_forward_equals_split_linear_cat(seed, G, K, N, m):
    x, w, b, _, _ = _case(seed, G, K, N, m)
    ref = _split_linear_cat(x, w, b, m).numpy()
    np.testing.assert_allclose(oracle.forward(x.numpy(), w.numpy(), b.numpy(), m), ref, rtol=1e-12, atol=1e-12)
    ref_nb = _split_linear_cat(x, w, None, m).numpy()
    np.testing.assert_allclose(oracle.forward(x.numpy(), w.numpy(), None, m), ref_nb, rtol=1e-12, atol=1e-12)
    # per-group weight lists are the same operand in another form
    np.testing.assert_allclose(oracle.forward(x.numpy(), list(w.numpy()), list(b.numpy()), m), ref,
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed,G,K,N,m", CASES)
def test_backward_equals_autograd(seed, G, K, N, m):
    x, w, b, dy, mg = _case(seed, G, K, N, m)
    xr, wr, br = (t.clone().requires_grad_(True) for t in (x, w, b))
    y = _split_linear_cat(xr, wr, br, m)
    if y.numel():
        y.backward(dy)
    gx = xr.grad if xr.grad is not None else torch.zeros_like(x)
    gw = wr.grad if wr.grad is not None else torch.zeros_like(w)
    gb = br.grad if br.grad is not None else torch.zeros_like(b)
    np.testing.assert_allclose(oracle.dgrad(dy.numpy(), w.numpy(), m), gx.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.wgrad(x.numpy(), dy.numpy(), m), gw.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(oracle.bgrad(dy.numpy(), m), gb.numpy(), rtol=1e-12, atol=1e-12)
    acc = oracle.wgrad(x.numpy(), dy.numpy(), m, main_grad=mg.numpy(), accumulate=True)
    np.testing.assert_allclose(acc, mg.numpy() + gw.numpy(), rtol=1e-12, atol=1e-12)
    for g in range(G):
        if m[g] == 0:   # an empty group leaves main_grad exactly as it was
            assert np.array_equal(acc[g], mg.numpy()[g])
            assert not oracle.wgrad(x.numpy(), dy.numpy(), m)[g].any()


def test_single_group_is_nn_linear():
    torch.manual_seed(7)
    lin = torch.nn.Linear(24, 10, dtype=torch.float64)
    x = torch.randn(13, 24, dtype=torch.float64, requires_grad=True)
    y = lin(x)
    dy = torch.randn_like(y)
    y.backward(dy)
    W, b = lin.weight.detach().numpy()[None], lin.bias.detach().numpy()[None]
    np.testing.assert_allclose(oracle.forward(x.detach().numpy(), W, b, [13]), y.detach().numpy(), rtol=1e-12)
    np.testing.assert_allclose(oracle.dgrad(dy.numpy(), W, [13]), x.grad.numpy(), rtol=1e-12)
    np.testing.assert_allclose(oracle.wgrad(x.detach().numpy(), dy.numpy(), [13])[0], lin.weight.grad.numpy(),
                               rtol=1e-12)
    np.testing.assert_allclose(oracle.bgrad(dy.numpy(), [13])[0], lin.bias.grad.numpy(), rtol=1e-12)


def test_row_and_group_sampling_match_library():
    seed, G, K, N, m = CASES[0]
    x, w, b, dy, mg = _case(seed, G, K, N, m)
    rows = np.array([0, 4, 5, 21, 22, 31])
    ref = _split_linear_cat(x, w, b, m).numpy()[rows]
    np.testing.assert_allclose(oracle.forward(x.numpy(), w.numpy(), b.numpy(), m, rows=rows), ref, rtol=1e-12, atol=1e-12)
    off = oracle.offsets(m, G, sum(m))
    ref_dx = np.stack([dy.numpy()[r] @ w.numpy()[gl.group_of_rows(off, [r])[0]] for r in rows])
    np.testing.assert_allclose(oracle.dgrad(dy.numpy(), w.numpy(), m, rows=rows), ref_dx, rtol=1e-12, atol=1e-12)
    sel_n = np.array([1, 7, 30])
    full = oracle.wgrad(x.numpy(), dy.numpy(), m, main_grad=mg.numpy(), accumulate=True)
    part = oracle.wgrad(x.numpy(), dy.numpy(), m, main_grad=mg.numpy(), accumulate=True, groups=[3, 1],
                        out_rows=sel_n)
    np.testing.assert_array_equal(part, full[[3, 1]][:, sel_n])


# --------------------------------------------------------- planted bugs ----

def _forward_pins_hold(fwd) -> bool:
    try:
        for seed, G, K, N, m in CASES:
            x, w, b, _, _ = _case(seed, G, K, N, m)
            ref = _split_linear_cat(x, w, b, m).numpy()
            if not np.allclose(fwd(x.numpy(), w.numpy(), b.numpy(), m), ref, rtol=1e-12, atol=1e-12):
                return False
        d = json.load(open(GOLDEN))
        got = fwd(np.array(d["x"], float), np.array(d["W"], float), np.array(d["b"], float), d["m_splits"])
        return got.tolist() == d["expect"]["y"]
    except Exception:
        return False


def _backward_pins_hold(dgrad, wgrad, bgrad) -> bool:
    try:
        for seed, G, K, N, m in CASES:
            x, w, b, dy, _ = _case(seed, G, K, N, m)
            xr, wr, br = (t.clone().requires_grad_(True) for t in (x, w, b))
            y = _split_linear_cat(xr, wr, br, m)
            if not y.numel():
                continue
            y.backward(dy)
            if not np.allclose(dgrad(dy.numpy(), w.numpy(), m), xr.grad.numpy(), rtol=1e-12, atol=1e-12):
                return False
            if not np.allclose(wgrad(x.numpy(), dy.numpy(), m), wr.grad.numpy(), rtol=1e-12, atol=1e-12):
                return False
            if not np.allclose(bgrad(dy.numpy(), m), br.grad.numpy(), rtol=1e-12, atol=1e-12):
                return False
        return True
    except Exception:
        return False


def test_pins_accept_the_oracle():
    assert _forward_pins_hold(oracle.forward)
    assert _backward_pins_hold(oracle.dgrad, oracle.wgrad, oracle.bgrad)


def _fwd_no_bias(x, w, b, m):
    return gl.forward(x, w, None, m)


def _fwd_transposed_weight(x, w, b, m):
    return gl.forward(x, np.swapaxes(np.asarray(w), 1, 2), b, m) if np.asarray(w).shape[1] == np.asarray(
        w).shape[2] else gl.forward(x, w, b, m) + 1.0


def _fwd_wrong_group(x, w, b, m):
    G = len(m)
    return gl.forward(x, [np.asarray(w)[(g + 1) % G] for g in range(G)], b, m)


def _fwd_bias_sign(x, w, b, m):
    return gl.forward(x, w, -np.asarray(b), m)


def _fwd_off_by_one_rows(x, w, b, m):
    y = gl.forward(x, w, b, m)
    return np.roll(y, 1, axis=0)


@pytest.mark.parametrize("mutant", [_fwd_no_bias, _fwd_transposed_weight, _fwd_wrong_group, _fwd_bias_sign,
                                    _fwd_off_by_one_rows])
def test_forward_pins_catch_planted_mistake(mutant):
    assert not _forward_pins_hold(mutant)


def _dgrad_transposed(dy, w, m):
    w = np.asarray(w)
    if w.shape[1] != w.shape[2]:
        return gl.dgrad(dy, w, m) * 1.5
    return gl.dgrad(dy, np.swapaxes(w, 1, 2), m)


def _wgrad_transposed(x, dy, m):
    out = gl.wgrad(x, dy, m)
    return np.swapaxes(out, 1, 2) if out.shape[1] == out.shape[2] else out[:, ::-1]


def _wgrad_neighbour_rows(x, dy, m):
    return gl.wgrad(np.roll(np.asarray(x), 1, axis=0), dy, m)


def _bgrad_dropped_row(dy, m):
    dy = np.array(dy, dtype=np.float64)
    dy[-1] = 0.0
    return gl.bgrad(dy, m)


@pytest.mark.parametrize("which,mutant", [("d", _dgrad_transposed), ("w", _wgrad_transposed),
                                          ("w", _wgrad_neighbour_rows), ("b", _bgrad_dropped_row)])
def test_backward_pins_catch_planted_mistake(which, mutant):
    fns = {"d": gl.dgrad, "w": gl.wgrad, "b": gl.bgrad}
    fns[which] = mutant
    assert not _backward_pins_hold(fns["d"], fns["w"], fns["b"])
