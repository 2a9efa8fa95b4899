"""GPU parity of the fp16 paths (forward + bias, dgrad, wgrad, bias grad) against
the CPU oracle through the C ABI.  Tolerance: fp16 outputs carry an 11-bit
significand, so rounding the fp32 accumulator costs at most 2^-11 ~ 4.9e-4 relative;
fp32 accumulation over these contraction lengths adds far less; |err| <=
2e-3 (|ref| + 1) leaves a 4x margin.  Integer-valued inputs are exact in fp16 and
every sum is exact in fp32, so those must match bit for bit."""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
from gl_testutil import assert_close, nan_tail, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL_F16 = 2e-3
F16 = torch.float16

SHAPES = [
    # groups of at most 256 rows on average (the forward's deeper weight ring) ...
    (5, 200, 264, [0, 300, 1, 0, 513]),
    (3, 256, 512, [256, 257, 255]),
    (8, 136, 72, [3, 0, 0, 70, 260, 1, 0, 90]),
    # ... and larger ones (its default ring)
    (2, 200, 264, [700, 301]),
]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def workspace_for(m, T):
    ws = gl.new_workspace(len(m))
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), T, ws)
    return ws


def run_all(x, w, b, dy, mg, m):
    T, K = x.shape
    G, N, _ = w.shape
    ws = workspace_for(m, T)
    xd, wd, bd, dyd = x.to(DEV), w.to(DEV), b.to(DEV), dy.to(DEV)
    y = nan_tail(T + 3, N, T, F16, DEV)
    gl.gl_forward(xd, wd, y, ws, bias=bd)
    dx = nan_tail(T + 3, K, T, F16, DEV)
    gl.gl_dgrad(dyd, wd, dx, ws)
    dw = torch.full((G, N, K), float("nan"), dtype=F16, device=DEV)
    gl.gl_wgrad(xd, dyd, dw, ws)
    mgd = mg.to(DEV)
    gl.gl_wgrad(xd, dyd, mgd, ws, accumulate=True)
    db = torch.empty(G, N, dtype=F16, device=DEV)
    gl.gl_bgrad(dyd, db, ws)
    torch.cuda.synchronize()
    assert torch.isnan(y[T:]).all() and torch.isnan(dx[T:]).all(), "wrote past the valid rows"
    X, W, B, DY, MG = (to64(t) for t in (x, w, b, dy, mg))
    return dict(y=(y[:T], oracle.forward(X, W, B, m)), dx=(dx[:T], oracle.dgrad(DY, W, m)),
                dw=(dw, oracle.wgrad(X, DY, m)), mg=(mgd, oracle.wgrad(X, DY, m, main_grad=MG, accumulate=True)),
                db=(db, oracle.bgrad(DY, m)))


@pytest.mark.parametrize("G,K,N,m", SHAPES)
def test_fp16_all_passes(G, K, N, m):
    say(f"fp16 G={G} K={K} N={N} m={m}")
    T = sum(m)
    g = torch.Generator().manual_seed(G + K)
    x = torch.randn(T, K, generator=g).to(F16)
    w = (torch.randn(G, N, K, generator=g) * 0.05).to(F16)
    b = (torch.randn(G, N, generator=g) * 0.1).to(F16)
    dy = torch.randn(T, N, generator=g).to(F16)
    mg = torch.randn(G, N, K, generator=g)
    for name, (got, ref) in run_all(x, w, b, dy, mg, m).items():
        assert_close(got, ref, TOL_F16, f"fp16 {name}")


def test_fp16_integer_cases_bit_exact():
    G, K, N, m = 5, 200, 264, [0, 300, 1, 0, 513]
    T = sum(m)
    g = torch.Generator().manual_seed(4)
    r = lambda *s: torch.randint(-3, 4, s, generator=g).to(F16)
    x, w, b, dy = r(T, K), r(G, N, K), r(G, N), r(T, N)
    mg = torch.randint(-3, 4, (G, N, K), generator=g).float()
    for name, (got, ref) in run_all(x, w, b, dy, mg, m).items():
        assert np.array_equal(to64(got), ref), f"fp16 {name} not exact"
