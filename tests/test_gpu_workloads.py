"""GPU parity at the workloads' full sizes, through the C ABI, in the same launch
configuration the benchmark times.

Outputs are checked on samples the oracle computes one by one (rows, wgrad rows of
selected groups) and, where cheap, in full (bias grad, the untouched tail of a
caller buffer, untouched main_grad of empty groups).  Inputs come from the seeded
generators; the oracle quantizes and computes on its own.
"""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
import synth
from gl_testutil import TOL_BF16, assert_bits_equal, assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


class LazyGroups:
    """Per-group float64 views of a stacked CPU tensor, converted when asked for."""

    def __init__(self, t):
        self.t = t

    def __len__(self):
        return self.t.shape[0]

    def __getitem__(self, g):
        return self.t[g].double().numpy()


def sample_rows(m, n_random=48, seed=0, groups=None):
    """First two and last two rows of every (listed) non-empty group, plus random
    rows of those groups."""
    off = np.concatenate([[0], np.cumsum(m)])
    groups = range(len(m)) if groups is None else groups
    rows = set()
    rng = np.random.default_rng(seed)
    nonempty = [g for g in groups if m[g]]
    for g in nonempty:
        for r in (off[g], off[g] + 1, off[g + 1] - 2, off[g + 1] - 1):
            if off[g] <= r < off[g + 1]:
                rows.add(int(r))
    for _ in range(n_random):
        g = nonempty[rng.integers(0, len(nonempty))]
        rows.add(int(rng.integers(off[g], off[g + 1])))
    return np.array(sorted(rows), dtype=np.int64)


def some_groups(G, k, seed=1):
    """Group 0, the last group and k - 2 others."""
    rng = np.random.default_rng(seed)
    return sorted({0, G - 1, *rng.choice(np.arange(1, G - 1), size=k - 2, replace=False).tolist()})


def workspace(m, T):
    ws = gl.new_workspace(len(m))
    gl.gl_offsets(torch.from_numpy(np.asarray(m, dtype=np.int64)).to(DEV), T, ws)
    assert gl.gl_read_status(ws) == 0
    return ws


def test_bf16_train_g8_all_passes():
    wl = synth.WORKLOADS["bf16_train_g8_k4096_n14336"]
    say(f"workload {wl.name}: generating")
    m = synth.split_sizes(wl)
    x, w, b, dy = synth.x(wl), synth.weight(wl), synth.bias(wl), synth.dy(wl)
    xd, wd, bd, dyd = (t.to(DEV) for t in (x, w, b, dy))
    ws = workspace(m, wl.T)
    y = torch.empty(wl.T, wl.N, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty(wl.T, wl.K, dtype=torch.bfloat16, device=DEV)
    dw = torch.empty(wl.G, wl.N, wl.K, dtype=torch.bfloat16, device=DEV)
    db = torch.empty(wl.G, wl.N, dtype=torch.bfloat16, device=DEV)
    say("  launching offsets/forward/dgrad/wgrad/bgrad")
    gl.gl_forward(xd, wd, y, ws, bias=bd)
    gl.gl_dgrad(dyd, wd, dx, ws)
    gl.gl_wgrad(xd, dyd, dw, ws)
    gl.gl_bgrad(dyd, db, ws)
    torch.cuda.synchronize()
    say("  checking against the oracle")
    rows = sample_rows(m)
    X, DY = x.float().numpy(), dy.float().numpy()
    W = LazyGroups(w)
    assert_close(y[torch.from_numpy(rows).to(DEV)], oracle.forward(X, W, to64(b), m, rows=rows), TOL_BF16, "y rows")
    assert_close(dx[torch.from_numpy(rows).to(DEV)], oracle.dgrad(DY, W, m, rows=rows), TOL_BF16, "dx rows")
    groups = [int(np.argmax(m)), int(np.argmin(m)), 3]
    nsel = np.array([0, 1, 255, 256, 7000, wl.N - 1])
    ref = oracle.wgrad(X, DY, m, groups=groups, out_rows=nsel)
    got = dw[groups][:, torch.from_numpy(nsel).to(DEV)]
    assert_close(got, ref, TOL_BF16, "dW rows")
    assert_close(db, oracle.bgrad(DY, m), TOL_BF16, "db")


def test_bf16_zipf_g64_main_grad_accumulate():
    wl = synth.WORKLOADS["bf16_zipf_g64_k2048_n1536"]
    say(f"workload {wl.name}: generating")
    m = synth.split_sizes(wl)
    assert (m == 0).sum() >= 4 and m.max() > 15000
    x, w, dy, mg = synth.x(wl), synth.weight(wl), synth.dy(wl), synth.main_grad(wl)
    xd, wd, dyd, mgd = (t.to(DEV) for t in (x, w, dy, mg))
    ws = workspace(m, wl.T)
    y = torch.empty(wl.T, wl.N, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty(wl.T, wl.K, dtype=torch.bfloat16, device=DEV)
    say("  launching forward/dgrad/wgrad(accumulate)")
    gl.gl_forward(xd, wd, y, ws)
    gl.gl_dgrad(dyd, wd, dx, ws)
    gl.gl_wgrad(xd, dyd, mgd, ws, accumulate=True)
    torch.cuda.synchronize()
    say("  checking against the oracle")
    rows = sample_rows(m)
    X, DY = x.float().numpy(), dy.float().numpy()
    W = LazyGroups(w)
    idx = torch.from_numpy(rows).to(DEV)
    assert_close(y[idx], oracle.forward(X, W, None, m, rows=rows), TOL_BF16, "y rows")
    assert_close(dx[idx], oracle.dgrad(DY, W, m, rows=rows), TOL_BF16, "dx rows")
    nz = np.nonzero(m)[0]
    groups = [int(np.argmax(m)), int(nz[np.argmin(m[nz])]), int(nz[len(nz) // 2])]
    nsel = np.array([0, 5, 511, 1535])
    ref = oracle.wgrad(X, DY, m, main_grad=mg.numpy(), accumulate=True, groups=groups, out_rows=nsel)
    assert_close(mgd[groups][:, torch.from_numpy(nsel).to(DEV)], ref, TOL_BF16, "main_grad rows")
    for g in np.nonzero(m == 0)[0]:
        assert_bits_equal(mgd[int(g)], mg[int(g)], f"empty group {g} main_grad")


def test_bf16_fwd_g256_caller_buffer_per_group_weights():
    wl = synth.WORKLOADS["bf16_fwd_g256_k7168_n2048_outbuf"]
    say(f"workload {wl.name}: generating")
    m = synth.split_sizes(wl)
    x, w = synth.x(wl), synth.weight(wl)
    xd = x.to(DEV)
    wd = w.to(DEV)
    wlist = [wd[g] for g in range(wl.G)]  # the per-group pointer form
    ws = workspace(m, wl.T)
    y = torch.full((wl.out_rows, wl.N), float("nan"), dtype=torch.bfloat16, device=DEV)
    y[: wl.T] = 0.0
    tail_before = y[wl.T:].clone()
    say("  launching forward into the caller buffer")
    gl.gl_forward(xd, wlist, y, ws)
    y_stacked = torch.empty(wl.T, wl.N, dtype=torch.bfloat16, device=DEV)
    gl.gl_forward(xd, wd, y_stacked, ws)
    torch.cuda.synchronize()
    say("  checking against the oracle")
    assert_bits_equal(y[wl.T:], tail_before, "padded tail")
    assert_bits_equal(y[: wl.T], y_stacked, "per-group pointers vs stacked weight")
    rows = sample_rows(m, n_random=32, groups=some_groups(wl.G, 16))
    X = x.float().numpy()
    assert_close(y[torch.from_numpy(rows).to(DEV)], oracle.forward(X, LazyGroups(w), None, m, rows=rows), TOL_BF16,
                 "y rows")


def test_mxfp8_fwd_g32_quantize_and_forward():
    wl = synth.WORKLOADS["mxfp8_fwd_g32_k4096_n4096"]
    say(f"workload {wl.name}: generating")
    m = synth.split_sizes(wl)
    x, w = synth.x(wl), synth.weight(wl)
    xd, wd = x.to(DEV), w.to(DEV)
    ws = workspace(m, wl.T)
    xq = torch.empty(wl.T, wl.K, dtype=torch.uint8, device=DEV)
    xs = torch.empty(wl.T, wl.K // 32, dtype=torch.uint8, device=DEV)
    wq = torch.empty(wl.G, wl.N, wl.K, dtype=torch.uint8, device=DEV)
    wsc = torch.empty(wl.G, wl.N, wl.K // 32, dtype=torch.uint8, device=DEV)
    say("  launching quantize(W), quantize(x), MXFP8 forward")
    gl.gl_group_quantize_mxfp8(wd, wq, wsc)
    gl.gl_group_quantize_mxfp8(xd, xq, xs)
    y = torch.empty(wl.T, wl.N, dtype=torch.bfloat16, device=DEV)
    gl.gl_forward(xq, wq, y, ws, x_scale=xs, w_scale=wsc)
    torch.cuda.synchronize()
    say("  checking against the oracle")
    rows = sample_rows(m, n_random=24, groups=some_groups(wl.G, 4))
    off = np.concatenate([[0], np.cumsum(m)])
    gs = oracle.group_of_rows(off, rows)
    xq_c, xs_c = xq.cpu().numpy(), xs.cpu().numpy()
    ref_rows = np.zeros((rows.size, wl.N))
    for g in np.unique(gs):
        g = int(g)
        sel = np.nonzero(gs == g)[0]
        qx, sx = oracle.quantize_mxfp8(x[torch.from_numpy(rows[sel])].double().numpy())
        assert np.array_equal(xq_c[rows[sel]], qx) and np.array_equal(xs_c[rows[sel]], sx), f"x codes, group {g}"
        qw, sw = oracle.quantize_mxfp8(w[g].double().numpy())
        if g in (int(gs[0]), int(gs[-1])):  # whole-group weight codes, bit for bit
            assert np.array_equal(wq[g].cpu().numpy(), qw) and np.array_equal(wsc[g].cpu().numpy(), sw)
        # rows are independent: each sampled row is a one-group problem of its own
        ref_rows[sel] = oracle.forward_mxfp8(qx, sx, [qw], [sw], None, [len(sel)])
    assert_close(y[torch.from_numpy(rows).to(DEV)], ref_rows, TOL_BF16, "MXFP8 y rows")
