"""GPU parity of the grouped MLP (FC1 -> SwiGLU -> FC2, page "[PyTorch] Add optional
caller-provided output/grad-input buffers to GroupedLinear and fused grouped MLP";
the activation, which the pages leave open, is SwiGLU).

Each step is checked against the oracle on the GPU's own stored intermediates
(h, a, da, dh are stored in the layer dtype, as the oracle's definition says) with
the usual element-wise bound, and the whole forward and backward end to end
against the oracle's own chain with a bound scaled by each output's RMS.
Caller buffers: only rows < T of y and dx are written.
"""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
from gl_testutil import TOL_BF16, TOL_F32, assert_bits_equal, assert_close, nan_tail, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {torch.bfloat16: TOL_BF16, torch.float16: 2e-3, torch.float32: TOL_F32}
NAME = {torch.bfloat16: "bf16", torch.float16: "f16", torch.float32: "f32"}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def assert_close_chain(got, ref, rel, what):
    """End-to-end bound: the GPU chain rounds h, a, da and dh to the layer dtype at
    values that differ from the oracle chain's by an ulp here and there, and a
    result summed over many rows carries that difference at the scale of its
    typical magnitude, not of each element; so the bound is rel * (|ref| + rms(ref) + 1)."""
    g = to64(got)
    ref = np.asarray(ref, dtype=np.float64)
    lim = rel * (np.abs(ref) + np.sqrt(np.mean(ref ** 2)) + 1.0)
    bad = ~(np.abs(g - ref) <= lim)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} elements outside the end-to-end bound"


def workspace_for(m):
    ws = gl.new_workspace(len(m))
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), int(sum(m)), ws)
    return ws


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_swiglu_forward_backward(dtype):
    T, F = 301, 200
    g = torch.Generator().manual_seed(31)
    h = (torch.randn(T, 2 * F, generator=g) * 4).to(dtype)
    h[0, :8] = torch.tensor([0.0, -0.0, 30.0, -30.0, 88.0, -88.0, 1e-3, -1e-3]).to(dtype)
    da = torch.randn(T, F, generator=g).to(dtype)
    hd, dad = h.to(DEV), da.to(DEV)
    a = torch.empty(T, F, dtype=dtype, device=DEV)
    dh = torch.empty(T, 2 * F, dtype=dtype, device=DEV)
    gl.gl_swiglu_forward(hd, a)
    gl.gl_swiglu_backward(hd, dad, dh)
    torch.cuda.synchronize()
    H, DA = to64(h), to64(da)
    assert_close(a, oracle.swiglu(H), TOL[dtype], "a")
    assert_close(dh, oracle.swiglu_backward(H, DA), TOL[dtype], "dh")


SHAPES = [
    # (G, K, F, N, m): ragged and empty groups, partial tiles in every dimension
    (4, 128, 96, 136, [50, 0, 300, 77]),
    (3, 512, 512, 256, [700, 0, 333]),
]


def mlp_case(seed, G, K, F, N, m, dtype):
    g = torch.Generator().manual_seed(seed)
    T = sum(m)
    r = lambda *s, std=1.0: (torch.randn(*s, generator=g) * std).to(dtype)
    return (r(T, K), r(G, 2 * F, K, std=0.08), r(G, 2 * F, std=0.1), r(G, N, F, std=0.08), r(G, N, std=0.1),
            r(T, N))


@pytest.mark.parametrize("G,K,F,N,m", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_grouped_mlp_forward_backward(G, K, F, N, m, dtype):
    say(f"grouped MLP {dtype} G={G} K={K} F={F} N={N} m={m}")
    x, w1, b1, w2, b2, dy = mlp_case(32, G, K, F, N, m, dtype)
    T = sum(m)
    ws = workspace_for(m)
    xd, w1d, b1d, w2d, b2d, dyd = (t.to(DEV) for t in (x, w1, b1, w2, b2, dy))
    h = torch.empty(T, 2 * F, dtype=dtype, device=DEV)
    a = torch.empty(T, F, dtype=dtype, device=DEV)
    y = nan_tail(T + 5, N, T, dtype, DEV)
    y_tail = y[T:].clone()
    gl.gl_grouped_mlp_forward(xd, w1d, w2d, h, a, y, ws, b1=b1d, b2=b2d)
    da = torch.empty(T, F, dtype=dtype, device=DEV)
    dh = torch.empty(T, 2 * F, dtype=dtype, device=DEV)
    dx = nan_tail(T + 3, K, T, dtype, DEV)
    dx_tail = dx[T:].clone()
    dw1 = torch.full((G, 2 * F, K), float("nan"), dtype=dtype, device=DEV)
    dw2 = torch.full((G, N, F), float("nan"), dtype=dtype, device=DEV)
    db1 = torch.full((G, 2 * F), float("nan"), dtype=dtype, device=DEV)
    db2 = torch.full((G, N), float("nan"), dtype=dtype, device=DEV)
    gl.gl_grouped_mlp_backward(xd, w1d, w2d, h, a, dyd, da, dh, dx, dw1, dw2, ws, db1=db1, db2=db2)
    torch.cuda.synchronize()
    assert gl.gl_read_status(ws) == 0
    tol = TOL[dtype]
    X, W1, B1, W2, B2, DY = (to64(t) for t in (x, w1, b1, w2, b2, dy))
    Hg, Ag, DAg, DHg = (to64(t) for t in (h, a, da, dh))
    # each step on the GPU's own stored inputs
    assert_close(h, oracle.forward(X, W1, B1, m), tol, "h = FC1(x)")
    assert_close(a, oracle.swiglu(Hg), tol, "a = SwiGLU(h)")
    assert_close(y[:T], oracle.forward(Ag, W2, B2, m), tol, "y = FC2(a)")
    assert_close(dw2, oracle.wgrad(Ag, DY, m), tol, "dW2")
    assert_close(db2, oracle.bgrad(DY, m), tol, "db2")
    assert_close(da, oracle.dgrad(DY, W2, m), tol, "da")
    assert_close(dh, oracle.swiglu_backward(Hg, DAg), tol, "dh")
    assert_close(dw1, oracle.wgrad(X, DHg, m), tol, "dW1")
    assert_close(db1, oracle.bgrad(DHg, m), tol, "db1")
    assert_close(dx[:T], oracle.dgrad(DHg, W1, m), tol, "dx")
    assert_bits_equal(y[T:], y_tail, "y tail untouched")
    assert_bits_equal(dx[T:], dx_tail, "dx tail untouched")
    # end to end against the oracle's own chain
    ho, ao, yo = oracle.mlp_forward(X, W1, B1, W2, B2, m, NAME[dtype])
    assert_close_chain(y[:T], yo, tol, "y end to end")
    dxo, dw1o, db1o, dw2o, db2o, _, _ = oracle.mlp_backward(X, W1, W2, ho, ao, DY, m, NAME[dtype])
    for got, ref, what in ((dx[:T], dxo, "dx"), (dw1, dw1o, "dW1"), (db1, db1o, "db1"), (dw2, dw2o, "dW2"),
                           (db2, db2o, "db2")):
        assert_close_chain(got, ref, tol, f"{what} end to end")


def test_grouped_mlp_per_group_weights_and_main_grad_accumulate():
    G, K, F, N, m = 3, 136, 64, 96, [40, 0, 201]
    dtype = torch.bfloat16
    x, w1, b1, w2, b2, dy = mlp_case(33, G, K, F, N, m, dtype)
    T = sum(m)
    ws = workspace_for(m)
    xd, dyd = x.to(DEV), dy.to(DEV)
    w1l, w2l = [t.to(DEV) for t in w1], [t.to(DEV) for t in w2]
    h = torch.empty(T, 2 * F, dtype=dtype, device=DEV)
    a = torch.empty(T, F, dtype=dtype, device=DEV)
    y = torch.empty(T, N, dtype=dtype, device=DEV)
    gl.gl_grouped_mlp_forward(xd, w1l, w2l, h, a, y, ws)
    y_stacked = torch.empty_like(y)
    gl.gl_grouped_mlp_forward(xd, w1.to(DEV), w2.to(DEV), torch.empty_like(h), torch.empty_like(a), y_stacked, ws)
    g = torch.Generator().manual_seed(34)
    mg1, mg2 = torch.randn(G, 2 * F, K, generator=g), torch.randn(G, N, F, generator=g)
    mg1d, mg2d = [t.to(DEV) for t in mg1], [t.to(DEV) for t in mg2]
    da = torch.empty(T, F, dtype=dtype, device=DEV)
    dh = torch.empty(T, 2 * F, dtype=dtype, device=DEV)
    dx = torch.empty(T, K, dtype=dtype, device=DEV)
    gl.gl_grouped_mlp_backward(xd, w1l, w2l, h, a, dyd, da, dh, dx, mg1d, mg2d, ws, accumulate=True)
    torch.cuda.synchronize()
    assert_bits_equal(y, y_stacked, "per-group vs stacked weights")
    Ag, DHg = to64(a), to64(dh)
    assert_close(torch.stack(mg2d), oracle.wgrad(Ag, to64(dy), m, main_grad=mg2.numpy(), accumulate=True),
                 TOL_F32, "main_grad 2")
    assert_close(torch.stack(mg1d), oracle.wgrad(to64(x), DHg, m, main_grad=mg1.numpy(), accumulate=True),
                 TOL_F32, "main_grad 1")
    assert_bits_equal(mg1d[1], mg1[1].to(DEV), "empty group main_grad 1 untouched")
    assert_bits_equal(mg2d[1], mg2[1].to(DEV), "empty group main_grad 2 untouched")
