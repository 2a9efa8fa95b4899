"""GPU parity of the deferred-wgrad queue: calls put in the backward and run later
(page "transformer_engine/pytorch/ops/basic/grouped_linear.py", delay_wgrad_compute
and backward_dw) give bit for bit what the same calls give when run at once, in put
order, also with unrelated work queued in between, on a side stream, into an fp32
main_grad, for per-group gradient lists and for the MXFP8 wgrad."""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
from gl_testutil import TOL_BF16, TOL_F32, assert_bits_equal, assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def workspace_for(m):
    ws = gl.new_workspace(len(m))
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), int(sum(m)), ws)
    return ws


def rand(g, *shape, dtype=torch.bfloat16, std=1.0):
    return (torch.randn(*shape, generator=g) * std).to(dtype).to(DEV)


def test_deferred_equals_immediate_and_runs_in_order():
    g = torch.Generator().manual_seed(51)
    m1, m2 = [300, 0, 77, 513], [40, 900]
    K1, N1, K2, N2 = 200, 264, 512, 136
    ws1, ws2 = workspace_for(m1), workspace_for(m2)
    x1, dy1 = rand(g, sum(m1), K1), rand(g, sum(m1), N1)
    x2, dy2 = rand(g, sum(m2), K2), rand(g, sum(m2), N2)
    say("deferred wgrad: two layers, stacked + per-group, bias grad on the first")
    # immediate
    dw1_ref = torch.empty(4, N1, K1, dtype=torch.bfloat16, device=DEV)
    db1_ref = torch.empty(4, N1, dtype=torch.bfloat16, device=DEV)
    gl.gl_wgrad_bgrad(x1, dy1, dw1_ref, db1_ref, ws1)
    dw2_ref = [torch.empty(N2, K2, dtype=torch.bfloat16, device=DEV) for _ in m2]
    gl.gl_wgrad(x2, dy2, dw2_ref, ws2)
    # deferred, with unrelated work in between
    q = gl.WgradQueue()
    dw1 = torch.full((4, N1, K1), float("nan"), dtype=torch.bfloat16, device=DEV)
    db1 = torch.full((4, N1), float("nan"), dtype=torch.bfloat16, device=DEV)
    dw2 = [torch.full((N2, K2), float("nan"), dtype=torch.bfloat16, device=DEV) for _ in m2]
    q.put(x1, dy1, dw1, ws1, db=db1)
    q.put(x2, dy2, dw2, ws2)
    assert len(q) == 2
    y_other = torch.empty(sum(m1), N1, dtype=torch.bfloat16, device=DEV)
    gl.gl_forward(x1, rand(g, 4, N1, K1, std=0.05), y_other, ws1)
    torch.cuda.synchronize()
    assert torch.isnan(dw1).all() and torch.isnan(dw2[0]).all(), "a put must not run anything"
    q.run_next()
    torch.cuda.synchronize()
    assert len(q) == 1
    assert_bits_equal(dw1, dw1_ref, "first deferred dW")
    assert_bits_equal(db1, db1_ref, "first deferred db")
    assert torch.isnan(dw2[1]).all(), "run_next runs only the oldest call"
    q.flush()
    torch.cuda.synchronize()
    assert len(q) == 0
    for a, b in zip(dw2, dw2_ref):
        assert_bits_equal(a, b, "second deferred dW")
    assert_close(dw1, oracle.wgrad(to64(x1), to64(dy1), m1), TOL_BF16, "deferred dW vs oracle")
    q.close()


def test_deferred_accumulate_on_side_stream():
    g = torch.Generator().manual_seed(52)
    m = [0, 250, 31, 600]
    K, N = 136, 200
    ws = workspace_for(m)
    x, dy = rand(g, sum(m), K), rand(g, sum(m), N)
    mg0 = torch.randn(len(m), N, K, generator=g)
    mg_ref = [t.to(DEV) for t in mg0]
    gl.gl_wgrad(x, dy, mg_ref, ws, accumulate=True)
    mg = [t.to(DEV) for t in mg0]
    q = gl.WgradQueue()
    q.put(x, dy, mg, ws, accumulate=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    q.flush(stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for a, b in zip(mg, mg_ref):
        assert_bits_equal(a, b, "deferred main_grad accumulate")
    assert_bits_equal(mg[0], mg0[0].to(DEV), "empty group's main_grad untouched")
    assert_close(torch.stack(mg), oracle.wgrad(to64(x), to64(dy), m, main_grad=mg0.numpy(), accumulate=True),
                 TOL_F32, "deferred main_grad vs oracle")
    q.close()


def test_deferred_mxfp8_wgrad():
    g = torch.Generator().manual_seed(53)
    m = [100, 0, 333]
    G, K, N, T = len(m), 256, 128, sum(m)
    ws = workspace_for(m)
    x, dy = rand(g, T, K), rand(g, T, N)
    ld = gl.gl_colwise_ld(G, T)
    u8 = dict(dtype=torch.uint8, device=DEV)
    xq, xs = torch.zeros(K, ld, **u8), torch.zeros(K, ld // 32, **u8)
    dyq, dys = torch.zeros(N, ld, **u8), torch.zeros(N, ld // 32, **u8)
    gl.gl_group_quantize_mxfp8_colwise(x, xq, xs, ws, G)
    gl.gl_group_quantize_mxfp8_colwise(dy, dyq, dys, ws, G)
    ref = torch.empty(G, N, K, dtype=torch.bfloat16, device=DEV)
    gl.gl_wgrad_mxfp8(dyq, dys, xq, xs, ref, ws, T)
    dw = torch.full((G, N, K), float("nan"), dtype=torch.bfloat16, device=DEV)
    q = gl.WgradQueue()
    q.put_mxfp8(dyq, dys, xq, xs, dw, ws, T)
    q.run_next()
    torch.cuda.synchronize()
    assert len(q) == 0
    assert_bits_equal(dw, ref, "deferred MXFP8 dW")
    assert not dw[1].float().abs().sum().item()
    q.close()
