"""GPU edge cases through the C ABI: GEMMs over many groups (1300: past one
1024-group scan chunk, most groups empty or a few rows), and zero total rows for every entry point
(forward/dgrad write nothing, wgrad stores zeros or leaves main_grad untouched, the
bias gradient is zero)."""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
from gl_testutil import TOL_BF16, TOL_F32, assert_bits_equal, assert_close, nan_tail, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def workspace_for(m):
    ws = gl.new_workspace(len(m))
    gl.gl_offsets(torch.tensor(np.asarray(m), dtype=torch.int64, device=DEV), int(np.sum(m)), ws)
    return ws


def test_1300_groups_mostly_tiny_or_empty():
    rng = np.random.default_rng(41)
    G, K, N = 1300, 136, 264
    m = rng.integers(0, 9, G) * (rng.random(G) < 0.6)
    m[[0, 1029, 1299]] = [0, 300, 0]
    T = int(m.sum())
    say(f"1300 groups: T={T}, empty={int((m == 0).sum())}")
    g = torch.Generator().manual_seed(42)
    x, dy = torch.randn(T, K, generator=g).to(torch.bfloat16), torch.randn(T, N, generator=g).to(torch.bfloat16)
    w = (torch.randn(G, N, K, generator=g) * 0.05).to(torch.bfloat16)
    b = (torch.randn(G, N, generator=g) * 0.1).to(torch.bfloat16)
    ws = workspace_for(m)
    xd, dyd, wd, bd = x.to(DEV), dy.to(DEV), w.to(DEV), b.to(DEV)
    y = nan_tail(T + 7, N, T, torch.bfloat16, DEV)
    gl.gl_forward(xd, wd, y, ws, bias=bd)
    dx = torch.empty(T, K, dtype=torch.bfloat16, device=DEV)
    gl.gl_dgrad(dyd, wd, dx, ws)
    dw = torch.full((G, N, K), float("nan"), dtype=torch.bfloat16, device=DEV)
    db = torch.full((G, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    gl.gl_wgrad_bgrad(xd, dyd, dw, db, ws)
    torch.cuda.synchronize()
    assert gl.gl_read_status(ws) == 0
    X, DY, W = to64(x), to64(dy), to64(w)
    assert_close(y[:T], oracle.forward(X, W, to64(b), m), TOL_BF16, "y")
    assert torch.isnan(y[T:]).all()
    assert_close(dx, oracle.dgrad(DY, W, m), TOL_BF16, "dx")
    groups = [1, 2, 1023, 1024, 1029, 1298] + [int(i) for i in np.nonzero(m)[0][:5]]
    assert_close(dw[groups], oracle.wgrad(X, DY, m, groups=groups), TOL_BF16, "dW (selected groups)")
    assert not dw[torch.from_numpy(np.nonzero(m == 0)[0]).to(DEV)].float().abs().sum().item()
    # bias grad over 100 000 groups: the standalone kernel (bf16) and the fp32
    # wgrad + bias grad call, whose bias grad is a launch of its own
    say("100k groups: bias grad, fp32 wgrad + bias grad")
    db = torch.full((G, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    gl.gl_bgrad(dyd, db, ws)
    x32, dy32 = xd.float(), dyd.float()
    dw32 = torch.full((G, N, K), float("nan"), device=DEV)
    db32 = torch.full((G, N), float("nan"), device=DEV)
    gl.gl_wgrad_bgrad(x32, dy32, dw32, db32, ws)
    torch.cuda.synchronize()
    ref_db = oracle.bgrad(DY, m)
    assert_close(db, ref_db, TOL_BF16, "db (bf16, every group)")
    assert_close(db32, ref_db, TOL_F32, "db (fp32, every group)")
    assert_close(dw32[groups], oracle.wgrad(X, DY, m, groups=groups), TOL_F32, "dW fp32 (selected groups)")
    assert not dw32[torch.from_numpy(np.nonzero(m == 0)[0]).to(DEV)].abs().sum().item()
    assert_close(db, oracle.bgrad(DY, m), TOL_BF16, "db")


class LazyGroups:
    """Per-group float64 views of a stacked CPU tensor, converted when asked for."""

    def __init__(self, t):
        self.t = t

    def __len__(self):
        return self.t.shape[0]

    def __getitem__(self, g):
        return self.t[g].double().numpy()


def test_100k_groups_offsets_and_passes():
    """100 000 groups, 95% empty, a few large ones: the scan's chunk carries over 98
    workgroup-sized chunks (offsets bit-exact against the oracle's), and the GEMMs'
    group lookup over a tile table that long."""
    rng = np.random.default_rng(43)
    G, K, N = 100_000, 32, 40
    m = rng.integers(1, 4, G) * (rng.random(G) < 0.05)
    m[[0, 1023, 1024, 50_000, G - 1]] = [0, 257, 1, 600, 3]
    T = int(m.sum())
    say(f"100k groups: T={T}, empty={int((m == 0).sum())}")
    ws = workspace_for(m)
    torch.cuda.synchronize()
    assert gl.gl_read_status(ws) == 0
    assert np.array_equal(gl.workspace_offsets(ws, G).cpu().numpy(), oracle.offsets(m.tolist(), G, T))
    g = torch.Generator().manual_seed(44)
    x, dy = torch.randn(T, K, generator=g).to(torch.bfloat16), torch.randn(T, N, generator=g).to(torch.bfloat16)
    w = (torch.randn(G, N, K, generator=g) * 0.05).to(torch.bfloat16)
    xd, dyd, wd = x.to(DEV), dy.to(DEV), w.to(DEV)
    y = nan_tail(T + 5, N, T, torch.bfloat16, DEV)
    gl.gl_forward(xd, wd, y, ws)
    dx = torch.empty(T, K, dtype=torch.bfloat16, device=DEV)
    gl.gl_dgrad(dyd, wd, dx, ws)
    dw = torch.full((G, N, K), float("nan"), dtype=torch.bfloat16, device=DEV)
    gl.gl_wgrad(xd, dyd, dw, ws)
    torch.cuda.synchronize()
    X, DY = to64(x), to64(dy)
    W = LazyGroups(w)
    assert_close(y[:T], oracle.forward(X, W, None, m), TOL_BF16, "y")
    assert torch.isnan(y[T:]).all()
    assert_close(dx, oracle.dgrad(DY, W, m), TOL_BF16, "dx")
    groups = [0, 1, 1023, 1024, 50_000, G - 1] + [int(i) for i in np.nonzero(m)[0][:5]]
    assert_close(dw[groups], oracle.wgrad(X, DY, m, groups=groups), TOL_BF16, "dW (selected groups)")
    assert not dw[torch.from_numpy(np.nonzero(m == 0)[0]).to(DEV)].float().abs().sum().item()
    # bias grad over 100 000 groups: the standalone kernel (bf16) and the fp32
    # wgrad + bias grad call, whose bias grad is a launch of its own
    say("100k groups: bias grad, fp32 wgrad + bias grad")
    db = torch.full((G, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    gl.gl_bgrad(dyd, db, ws)
    x32, dy32 = xd.float(), dyd.float()
    dw32 = torch.full((G, N, K), float("nan"), device=DEV)
    db32 = torch.full((G, N), float("nan"), device=DEV)
    gl.gl_wgrad_bgrad(x32, dy32, dw32, db32, ws)
    torch.cuda.synchronize()
    ref_db = oracle.bgrad(DY, m)
    assert_close(db, ref_db, TOL_BF16, "db (bf16, every group)")
    assert_close(db32, ref_db, TOL_F32, "db (fp32, every group)")
    assert_close(dw32[groups], oracle.wgrad(X, DY, m, groups=groups), TOL_F32, "dW fp32 (selected groups)")
    assert not dw32[torch.from_numpy(np.nonzero(m == 0)[0]).to(DEV)].abs().sum().item()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_zero_total_rows(dtype):
    G, K, N = 3, 64, 96
    m = [0, 0, 0]
    ws = workspace_for(m)
    x = torch.empty(0, K, dtype=dtype, device=DEV)
    dy = torch.empty(0, N, dtype=dtype, device=DEV)
    w = torch.randn(G, N, K, device=DEV).to(dtype)
    y = torch.full((5, N), float("nan"), dtype=dtype, device=DEV)
    dx = torch.full((5, K), float("nan"), dtype=dtype, device=DEV)
    gl.gl_forward(x, w, y, ws)
    gl.gl_dgrad(dy, w, dx, ws)
    dw = torch.full((G, N, K), float("nan"), dtype=dtype, device=DEV)
    db = torch.full((G, N), float("nan"), dtype=dtype, device=DEV)
    gl.gl_wgrad_bgrad(x, dy, dw, db, ws)
    mg = torch.randn(G, N, K, device=DEV)
    mg0 = mg.clone()
    gl.gl_wgrad(x, dy, mg, ws, accumulate=True)
    db2 = torch.full((G, N), float("nan"), dtype=dtype, device=DEV)
    gl.gl_bgrad(dy, db2, ws)
    torch.cuda.synchronize()
    assert gl.gl_read_status(ws) == 0
    assert torch.isnan(y).all() and torch.isnan(dx).all(), "nothing to write for zero rows"
    assert not dw.float().abs().sum().item() and not db.float().abs().sum().item()
    assert not db2.float().abs().sum().item()
    assert_bits_equal(mg, mg0, "main_grad untouched")


def test_zero_total_rows_mxfp8_and_mlp():
    G, K, F, N = 2, 128, 64, 256
    m = [0, 0]
    ws = workspace_for(m)
    u8 = dict(dtype=torch.uint8, device=DEV)
    x = torch.empty(0, K, dtype=torch.bfloat16, device=DEV)
    xq, xs = torch.empty(0, K, **u8), torch.empty(0, K // 32, **u8)
    gl.gl_offsets_quantize_mxfp8(torch.zeros(G, dtype=torch.int64, device=DEV), x, ws, xq, xs)
    w = (torch.randn(G, N, K, device=DEV) * 0.05).to(torch.bfloat16)
    wq, wsc = torch.empty(G, N, K, **u8), torch.empty(G, N, K // 32, **u8)
    wtq, wts = torch.empty(G, K, N, **u8), torch.empty(G, K, N // 32, **u8)
    gl.gl_quantize_mxfp8_weights(w, wq, wsc, wtq, wts)
    y = torch.full((4, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    gl.gl_forward(xq, wq, y, ws, x_scale=xs, w_scale=wsc)
    ld = gl.gl_colwise_ld(G, 0)
    dytq, dyts = torch.zeros(N, ld, **u8), torch.zeros(N, ld // 32, **u8)
    xtq, xts = torch.zeros(K, ld, **u8), torch.zeros(K, ld // 32, **u8)
    dw = torch.full((G, N, K), float("nan"), dtype=torch.bfloat16, device=DEV)
    gl.gl_wgrad_mxfp8(dytq, dyts, xtq, xts, dw, ws, 0)
    w1 = (torch.randn(G, 2 * F, K, device=DEV) * 0.05).to(torch.bfloat16)
    w2 = (torch.randn(G, N, F, device=DEV) * 0.05).to(torch.bfloat16)
    h, a = torch.empty(0, 2 * F, dtype=torch.bfloat16, device=DEV), torch.empty(0, F, dtype=torch.bfloat16, device=DEV)
    ym = torch.full((3, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    gl.gl_grouped_mlp_forward(x, w1, w2, h, a, ym, ws)
    dw1 = torch.full_like(w1, float("nan"))
    dw2 = torch.full_like(w2, float("nan"))
    dxm = torch.full((3, K), float("nan"), dtype=torch.bfloat16, device=DEV)
    gl.gl_grouped_mlp_backward(x, w1, w2, h, a, torch.empty(0, N, dtype=torch.bfloat16, device=DEV),
                               torch.empty(0, F, dtype=torch.bfloat16, device=DEV), torch.empty_like(h), dxm, dw1,
                               dw2, ws)
    torch.cuda.synchronize()
    assert torch.isnan(y).all() and torch.isnan(ym).all() and torch.isnan(dxm).all()
    assert not dw.float().abs().sum().item()
    assert not dw1.float().abs().sum().item() and not dw2.float().abs().sum().item()
