"""GPU parity at the longest rows the bf16 GEMMs take: in_features or out_features
of 2^22 elements, the bound of their 32-bit stage offsets (a 256-row K-major stage
then spans just under 2 GiB).  Forward with bias, dgrad, and wgrad with the fused
bias grad over two groups of 37 and 263 rows (a ragged row tile in each), checked
on sampled rows and columns the oracle computes one by one: every pass is row- or
column-separable, so a sample is the same definition on fewer outputs (page
"transformer_engine/pytorch/ops/basic/grouped_linear.py": forward, dgrad, wgrad,
bias grad)."""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
import synth
from gl_testutil import TOL_BF16, assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
LONG = 1 << 22


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


def sample(n, rng):
    """Both ends, the 256-element tile edges near the middle and random indices."""
    if n <= 256:
        return np.arange(n)
    idx = {0, 1, 7, 8, 255, 256, n // 2 - 1, n // 2, n - 257, n - 256, n - 9, n - 8, n - 2, n - 1}
    idx.update(rng.integers(0, n, 40).tolist())
    return np.array(sorted(idx), dtype=np.int64)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("K,N", [(LONG, 64), (64, LONG)])
def test_bf16_rows_of_2_to_the_22(K, N):
    wl = synth.WORKLOADS["bf16_train_g8_k4096_n14336"].scaled(
        name=f"bf16_g2_k{K}_n{N}", G=2, K=K, N=N, T=300, m_law="fixed", m_fixed=(37, 263))
    m = [int(v) for v in synth.split_sizes(wl)]
    G, T = wl.G, wl.T
    say(f"K={K} N={N} m={m}: generating")
    x, w, b, dy = synth.x(wl), synth.weight(wl), synth.bias(wl), synth.dy(wl)
    xd, wd, bd, dyd = (t.to(DEV) for t in (x, w, b, dy))
    ws = gl.new_workspace(G)
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), T, ws)
    bf = dict(dtype=torch.bfloat16, device=DEV)
    y, dx = torch.empty(T, N, **bf), torch.empty(T, K, **bf)
    dw, db = torch.empty(G, N, K, **bf), torch.empty(G, N, **bf)
    say("  launching forward, dgrad, wgrad with bias grad")
    gl.gl_forward(xd, wd, y, ws, bias=bd)
    gl.gl_dgrad(dyd, wd, dx, ws)
    gl.gl_wgrad_bgrad(xd, dyd, dw, db, ws)
    torch.cuda.synchronize()
    assert gl.gl_read_status(ws) == 0
    del xd, dyd, wd
    say("  checking sampled outputs against the oracle")
    rng = np.random.default_rng(7)
    rows = np.array([0, 1, 35, 36, 37, 38, 200, 291, 292, 293, 294, 298, 299])  # group and row-tile edges
    m_rows = [int((rows < m[0]).sum()), int((rows >= m[0]).sum())]
    rsel = torch.from_numpy(rows)
    W = LazyGroups(w)
    assert_close(y[rsel.to(DEV)], oracle.forward(to64(x[rsel]), W, to64(b), m_rows), TOL_BF16, "y rows")
    assert_close(dx[rsel.to(DEV)], oracle.dgrad(to64(dy[rsel]), W, m_rows), TOL_BF16, "dx rows")
    kc, nc = torch.from_numpy(sample(K, rng)), torch.from_numpy(sample(N, rng))
    ref = oracle.wgrad(to64(x[:, kc]), to64(dy[:, nc]), m)
    assert_close(dw[:, nc.to(DEV)][:, :, kc.to(DEV)], ref, TOL_BF16, "dW sample")
    assert_close(db[:, nc.to(DEV)], oracle.bgrad(to64(dy[:, nc]), m), TOL_BF16, "db sample")
