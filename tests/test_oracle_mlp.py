"""Pins of the grouped-MLP oracle (FC1 -> SwiGLU -> FC2) against things other than
itself: torch's own silu and autograd in float64, closed forms of silu and its
derivative, hand-rounded storage values, and the one-group case written as
torch.nn.Linear -> silu * up -> torch.nn.Linear."""
import numpy as np
import pytest
import torch

import oracle


def test_silu_matches_torch_and_closed_forms():
    v = np.concatenate([np.linspace(-30, 30, 1201), [0.0, 1e-9, -1e-9, 80.0, -80.0]])
    ref = torch.nn.functional.silu(torch.from_numpy(v)).numpy()
    assert np.allclose(oracle.silu(v), ref, rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(40.0) - 40.0) < 1e-15 * 40
    assert abs(oracle.silu(-40.0)) < 1e-15


def test_swiglu_halves_and_backward_closed_form():
    h = np.array([[0.0, 2.0, 1.0, -3.0]])          # F = 2: gate (0, 2), up (1, -3)
    a = oracle.swiglu(h)
    assert a.shape == (1, 2)
    assert a[0, 0] == 0.0                            # silu(0) * 1
    assert np.isclose(a[0, 1], 2.0 / (1 + np.exp(-2.0)) * -3.0)
    dh = oracle.swiglu_backward(h, np.ones((1, 2)))
    assert np.isclose(dh[0, 0], 0.5)                 # d silu/dg at 0 is 1/2, times up = 1
    assert dh[0, 2] == 0.0                           # d/d up = silu(0) = 0
    assert np.isclose(dh[0, 3], 2.0 / (1 + np.exp(-2.0)))


def test_swiglu_backward_matches_autograd():
    rng = np.random.default_rng(0)
    h = rng.normal(0, 3, (37, 2 * 19))
    da = rng.normal(0, 1, (37, 19))
    ht = torch.from_numpy(h).requires_grad_(True)
    g, u = ht[:, :19], ht[:, 19:]
    (torch.nn.functional.silu(g) * u).backward(torch.from_numpy(da))
    assert np.allclose(oracle.swiglu_backward(h, da), ht.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(oracle.swiglu(h), (torch.nn.functional.silu(g) * u).detach().numpy(), rtol=1e-14)


def test_store_rounds_to_nearest_even():
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -9), 65520.0, 1.0 + 2.0 ** -12])
    assert oracle.store(v, "bf16").tolist() == [1.0, 1.015625, -1.0, 65536.0, 1.0]
    assert oracle.store(v, "f16")[4] == 1.0 and np.isinf(oracle.store(v, "f16")[3])
    assert oracle.store(v, "f64").tolist() == v.tolist()


def _torch_mlp(x, w1, b1, w2, b2, m):
    """Split rows by m; per group Linear -> silu(first half) * second half -> Linear."""
    outs = []
    for g, xs in enumerate(torch.split(x, list(m))):
        h = torch.nn.functional.linear(xs, w1[g], None if b1 is None else b1[g])
        F = h.shape[1] // 2
        a = torch.nn.functional.silu(h[:, :F]) * h[:, F:]
        outs.append(torch.nn.functional.linear(a, w2[g], None if b2 is None else b2[g]))
    return torch.cat(outs)


@pytest.mark.parametrize("m,bias", [([23], True), ([5, 0, 17, 9], True), ([0, 12, 0], False)])
def test_mlp_forward_backward_match_torch_autograd(m, bias):
    rng = np.random.default_rng(1)
    G, K, F, N = len(m), 11, 7, 13
    T = sum(m)
    x, dy = rng.normal(0, 1, (T, K)), rng.normal(0, 1, (T, N))
    w1, w2 = rng.normal(0, 0.3, (G, 2 * F, K)), rng.normal(0, 0.3, (G, N, F))
    b1 = rng.normal(0, 0.1, (G, 2 * F)) if bias else None
    b2 = rng.normal(0, 0.1, (G, N)) if bias else None
    h, a, y = oracle.mlp_forward(x, w1, b1, w2, b2, m, "f64")
    t = {k: torch.from_numpy(v).requires_grad_(True) for k, v in
         dict(x=x, w1=w1, w2=w2, **({"b1": b1, "b2": b2} if bias else {})).items()}
    yt = _torch_mlp(t["x"], t["w1"], t.get("b1"), t["w2"], t.get("b2"), m)
    assert np.allclose(y, yt.detach().numpy(), rtol=1e-12, atol=1e-12)
    yt.backward(torch.from_numpy(dy))
    dx, dw1, db1, dw2, db2, da, dh = oracle.mlp_backward(x, w1, w2, h, a, dy, m, "f64")
    for got, key in ((dx, "x"), (dw1, "w1"), (dw2, "w2")):
        assert np.allclose(got, t[key].grad.numpy(), rtol=1e-11, atol=1e-11), key
    if bias:
        assert np.allclose(db1, t["b1"].grad.numpy(), rtol=1e-11, atol=1e-11)
        assert np.allclose(db2, t["b2"].grad.numpy(), rtol=1e-11, atol=1e-11)
    for g in range(G):   # empty groups: zero weight and bias gradients
        if m[g] == 0:
            assert not dw1[g].any() and not dw2[g].any() and not db1[g].any() and not db2[g].any()


def test_mlp_storage_points_round_h_and_a():
    rng = np.random.default_rng(2)
    m, K, F, N = [9, 4], 8, 5, 6
    x = rng.normal(0, 1, (13, K))
    w1, w2 = rng.normal(0, 0.5, (2, 2 * F, K)), rng.normal(0, 0.5, (2, N, F))
    h, a, _ = oracle.mlp_forward(x, w1, None, w2, None, m, "bf16")
    assert np.array_equal(h, oracle.store(h, "bf16")) and np.array_equal(a, oracle.store(a, "bf16"))
    h64, _, _ = oracle.mlp_forward(x, w1, None, w2, None, m, "f64")
    assert not np.array_equal(h, h64) and np.allclose(h, h64, rtol=2 ** -8)
