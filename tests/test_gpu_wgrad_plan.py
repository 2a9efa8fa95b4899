"""GPU parity of the wgrad contraction plan's split parts.

A wgrad launch orders the groups by stage count (64 rows a stage) and cuts the tiles
of every group above a cap (two thirds of the average stages per workgroup) into
parts over the contraction, whose fp32 partials are added in part order by the part
that arrives last.  The cases below give one group far more rows than the others:
with 24 tiles (one workgroup each) the 9000-row group's 141 stages are cut into
parts of at most 25.  On integer inputs every sum is exact in fp32, so the split
results must equal the oracle bit for bit in every output form; on random inputs
they meet the bf16 bound, gl_wgrad_bgrad's dW equals gl_wgrad's bit for bit, and a
repeated launch gives the same bits.
"""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
from gl_testutil import TOL_BF16, assert_bits_equal, assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
G, K, N, M = 4, 264, 520, [9000, 0, 130, 64]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def workspace_for(m):
    ws = gl.new_workspace(len(m))
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), int(sum(m)), ws)
    return ws


# The long group's split parts carry its bias grad: in tile column 0, then (group 1, with
# column g mod 2 = 1) in the partial second column of K = 264.
@pytest.mark.parametrize("m", [M, [64, 9000, 0, 130]])
def test_plan_splits_exact_on_integers(m):
    say(f"wgrad plan, integer inputs G={G} K={K} N={N} m={m}")
    g = torch.Generator().manual_seed(31)
    T = sum(m)
    r = lambda *s: torch.randint(-3, 4, s, generator=g)
    x, dy = r(T, K).to(torch.bfloat16), r(T, N).to(torch.bfloat16)
    mg = r(G, N, K).float()
    X, DY, MG = to64(x), to64(dy), to64(mg)
    ref_dw = oracle.wgrad(X, DY, m)
    ref_db = oracle.bgrad(DY, m)
    ws = workspace_for(m)
    xd, dyd = x.to(DEV), dy.to(DEV)

    dw32 = torch.empty(G, N, K, device=DEV)
    db32 = torch.empty(G, N, device=DEV)
    gl.gl_wgrad_bgrad(xd, dyd, dw32, db32, ws)
    dw16 = torch.empty(G, N, K, dtype=torch.bfloat16, device=DEV)
    db16 = torch.empty(G, N, dtype=torch.bfloat16, device=DEV)
    gl.gl_wgrad_bgrad(xd, dyd, dw16, db16, ws)
    mgd = mg.to(DEV)
    gl.gl_wgrad(xd, dyd, mgd, ws, accumulate=True)
    torch.cuda.synchronize()
    assert np.array_equal(dw32.cpu().numpy(), ref_dw), "fp32 dW (split parts) not exact"
    assert np.array_equal(db32.cpu().numpy(), ref_db), "fp32 db (split parts) not exact"
    # the exact sums rounded once to bf16, as the oracle's exact values round
    assert_bits_equal(dw16, torch.from_numpy(ref_dw).to(torch.bfloat16), "bf16 dW")
    assert_bits_equal(db16, torch.from_numpy(ref_db).to(torch.bfloat16), "bf16 db")
    ref_mg = oracle.wgrad(X, DY, m, main_grad=MG, accumulate=True)
    assert np.array_equal(mgd.cpu().numpy(), ref_mg), "main_grad accumulate (split parts) not exact"
    e = m.index(0)
    assert bool((mgd[e] == mg[e].to(DEV)).all()), "empty group's main_grad touched"


def test_plan_splits_random_bf16():
    say(f"wgrad plan, random inputs G={G} K={K} N={N} m={M}")
    g = torch.Generator().manual_seed(32)
    T = sum(M)
    x = torch.randn(T, K, generator=g).to(torch.bfloat16)
    dy = torch.randn(T, N, generator=g).to(torch.bfloat16)
    ws = workspace_for(M)
    xd, dyd = x.to(DEV), dy.to(DEV)
    dw_a = torch.empty(G, N, K, dtype=torch.bfloat16, device=DEV)
    gl.gl_wgrad(xd, dyd, dw_a, ws)
    outs = []
    for _ in range(2):
        dw = torch.empty(G, N, K, dtype=torch.bfloat16, device=DEV)
        db = torch.empty(G, N, dtype=torch.bfloat16, device=DEV)
        gl.gl_wgrad_bgrad(xd, dyd, dw, db, ws)
        outs.append((dw, db))
    torch.cuda.synchronize()
    X, DY = to64(x), to64(dy)
    assert_close(dw_a, oracle.wgrad(X, DY, M), TOL_BF16, "dW")
    assert_close(outs[0][1], oracle.bgrad(DY, M), TOL_BF16, "db")
    assert_bits_equal(outs[0][0], dw_a, "gl_wgrad_bgrad dW vs gl_wgrad dW")
    assert_bits_equal(outs[0][0], outs[1][0], "repeated dW")
    assert_bits_equal(outs[0][1], outs[1][1], "repeated db")
