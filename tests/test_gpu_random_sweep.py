"""A seeded random sweep of the grouped-linear path on the GPU against the oracle:
shapes, group counts, split patterns (empty, one-row, ragged, tile-multiple
groups), weight and bias forms, element types and accumulate modes drawn per case,
so that combinations the fixed cases do not name are still checked.  Every case
prints its parameters before it runs.  Bounds as everywhere: bf16 2e-2, fp16 2e-3,
fp32 1e-4, each times (|ref| + 1); MXFP8 codes bit-exact and its GEMMs at the bf16
bound on the dequantized operands (page "transformer_engine/pytorch/ops/basic/
grouped_linear.py": forward, dgrad, wgrad, bias grad; MXFP8 forward and backward)."""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
from gl_testutil import TOL_BF16, TOL_F32, assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {torch.bfloat16: TOL_BF16, torch.float16: 2e-3, torch.float32: TOL_F32}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def draw_splits(rng, G, scale):
    kind = rng.integers(0, 4)
    if kind == 0:
        m = rng.integers(0, scale, G)
    elif kind == 1:  # many empty groups
        m = rng.integers(0, scale, G) * (rng.random(G) < 0.4)
    elif kind == 2:  # tile multiples and one-row groups
        m = rng.choice([0, 1, 255, 256, 257, 512], G)
    else:  # one large group
        m = rng.integers(0, 8, G)
        m[rng.integers(0, G)] = scale * 3
    return [int(v) for v in m]


CASES = list(range(40))


@pytest.mark.parametrize("case", CASES)
def test_random_grouped_linear(case):
    rng = np.random.default_rng(1000 + case)
    dtype = [torch.bfloat16, torch.float16, torch.float32][case % 3]
    G = int(rng.integers(1, 12))
    K = int(rng.integers(1, 48)) * 8
    N = int(rng.integers(1, 48)) * 8
    if dtype == torch.float32:
        K, N = max(4, K // 2 // 4 * 4), max(4, N // 2 // 4 * 4)
    m = draw_splits(rng, G, 400)
    T = sum(m)
    per_group = bool(rng.integers(0, 2))
    with_bias = bool(rng.integers(0, 2))
    accumulate = bool(rng.integers(0, 2))
    say(f"case {case}: {dtype} G={G} K={K} N={N} m={m} per_group={per_group} bias={with_bias} acc={accumulate}")
    g = torch.Generator().manual_seed(2000 + case)
    x = torch.randn(T, K, generator=g).to(dtype)
    dy = torch.randn(T, N, generator=g).to(dtype)
    w = (torch.randn(G, N, K, generator=g) * 0.05).to(dtype)
    b = (torch.randn(G, N, generator=g) * 0.1).to(dtype)
    mg = torch.randn(G, N, K, generator=g)
    ws = gl.new_workspace(G)
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), T, ws)
    xd, dyd = x.to(DEV), dy.to(DEV)
    wd = [t.to(DEV) for t in w] if per_group else w.to(DEV)
    bd = ([t.to(DEV) for t in b] if per_group else b.to(DEV)) if with_bias else None
    y = torch.full((T + 3, N), float("nan"), dtype=dtype, device=DEV)
    gl.gl_forward(xd, wd, y, ws, bias=bd)
    dx = torch.full((T + 2, K), float("nan"), dtype=dtype, device=DEV)
    gl.gl_dgrad(dyd, wd, dx, ws)
    if accumulate:
        dw = [t.to(DEV) for t in mg] if per_group else mg.to(DEV)
    else:
        dw = [torch.empty(N, K, dtype=dtype, device=DEV) for _ in range(G)] if per_group else \
            torch.empty(G, N, K, dtype=dtype, device=DEV)
    db = torch.empty(G, N, dtype=dtype, device=DEV)
    gl.gl_wgrad_bgrad(xd, dyd, dw, db, ws, accumulate=accumulate)
    torch.cuda.synchronize()
    assert gl.gl_read_status(ws) == 0
    tol = TOL[dtype]
    X, DY, W, B = to64(x), to64(dy), to64(w), to64(b)
    assert_close(y[:T], oracle.forward(X, W, B if with_bias else None, m), tol, "y")
    assert torch.isnan(y[T:]).all() and torch.isnan(dx[T:]).all(), "rows past T written"
    assert_close(dx[:T], oracle.dgrad(DY, W, m), tol, "dx")
    dws = torch.stack(dw) if per_group else dw
    ref = oracle.wgrad(X, DY, m, main_grad=mg.numpy(), accumulate=accumulate)
    # an fp32 main_grad (accumulate) is held to the fp32 bound whatever the input type
    assert_close(dws, ref, TOL_F32 if accumulate else tol, "dW")
    assert_close(db, oracle.bgrad(DY, m), tol, "db")


@pytest.mark.parametrize("case", list(range(12)))
def test_random_mxfp8_path(case):
    rng = np.random.default_rng(3000 + case)
    G = int(rng.integers(1, 10))
    K = int(rng.integers(1, 5)) * 128
    N = int(rng.integers(1, 5)) * 128
    m = draw_splits(rng, G, 300)
    T = sum(m)
    say(f"mxfp8 case {case}: G={G} K={K} N={N} m={m}")
    g = torch.Generator().manual_seed(4000 + case)
    x = (torch.randn(T, K, generator=g) * 2).to(torch.bfloat16)
    dy = torch.randn(T, N, generator=g).to(torch.bfloat16)
    w = (torch.randn(G, N, K, generator=g) * 0.05).to(torch.bfloat16)
    u8 = dict(dtype=torch.uint8, device=DEV)
    ws = gl.new_workspace(G)
    md = torch.tensor(m, dtype=torch.int64, device=DEV)
    ld = gl.gl_colwise_ld(G, T)
    xq, xs, xtq, xts = torch.empty(T, K, **u8), torch.empty(T, K // 32, **u8), torch.zeros(K, ld, **u8), \
        torch.zeros(K, ld // 32, **u8)
    gl.gl_offsets_quantize_mxfp8_rowwise_colwise(md, x.to(DEV), ws, xq, xs, xtq, xts)
    wq, wsc = torch.empty(G, N, K, **u8), torch.empty(G, N, K // 32, **u8)
    wtq, wts = torch.empty(G, K, N, **u8), torch.empty(G, K, N // 32, **u8)
    gl.gl_quantize_mxfp8_weights(w.to(DEV), wq, wsc, wtq, wts)
    y = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    gl.gl_forward(xq, wq, y, ws, x_scale=xs, w_scale=wsc)
    dq, ds, dtq, dts = torch.empty(T, N, **u8), torch.empty(T, N // 32, **u8), torch.zeros(N, ld, **u8), \
        torch.zeros(N, ld // 32, **u8)
    gl.gl_group_quantize_mxfp8_rowwise_colwise(dy.to(DEV), dq, ds, dtq, dts, ws, G)
    dx = torch.empty(T, K, dtype=torch.bfloat16, device=DEV)
    gl.gl_dgrad_mxfp8(dq, ds, wtq, wts, dx, ws)
    dw = torch.empty(G, N, K, dtype=torch.bfloat16, device=DEV)
    gl.gl_wgrad_mxfp8(dtq, dts, xtq, xts, dw, ws, T)
    torch.cuda.synchronize()
    assert gl.gl_read_status(ws) == 0
    X, DY, W = to64(x), to64(dy), to64(w)
    rxq, rxs = oracle.quantize_mxfp8(X)
    assert np.array_equal(xq.cpu().numpy(), rxq) and np.array_equal(xs.cpu().numpy(), rxs)
    Xd = oracle.dequantize_mxfp8(rxq, rxs)
    rwq, rws = oracle.quantize_mxfp8(W.reshape(G * N, K))
    Wd = oracle.dequantize_mxfp8(rwq, rws).reshape(G, N, K)
    assert_close(y, oracle.forward(Xd, Wd, None, m), TOL_BF16, "MX y")
    rdq, rds = oracle.quantize_mxfp8(DY)
    DYd = oracle.dequantize_mxfp8(rdq, rds)
    wtq_ref, wts_ref = oracle.quantize_mxfp8_colwise_weights(W)
    Wtd = np.stack([oracle.dequantize_mxfp8(wtq_ref[i], wts_ref[i]) for i in range(G)])  # [G, K, N]
    assert_close(dx, oracle.dgrad(DYd, np.transpose(Wtd, (0, 2, 1)), m), TOL_BF16, "MX dx")
    cxq, cxs, poff = oracle.quantize_mxfp8_colwise(X, m, ld=ld)
    cdq, cds, _ = oracle.quantize_mxfp8_colwise(DY, m, ld=ld)
    Xtd, DYtd = oracle.dequantize_mxfp8(cxq, cxs), oracle.dequantize_mxfp8(cdq, cds)
    ref = np.zeros((G, N, K))
    for gi in range(G):
        lo, n = int(poff[gi]), m[gi]
        if n:
            ref[gi] = DYtd[:, lo:lo + n] @ Xtd[:, lo:lo + n].T
    assert_close(dw, ref, TOL_BF16, "MX dW")
