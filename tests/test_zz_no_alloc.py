"""The allocation-free forward (gl_forward_noalloc) through the C ABI against the
workspace forward (gl_offsets + gl_forward) on the same inputs, and against the
oracle: three calls in a row on the one device array, each smaller than the one
before, so every call must rewrite what the previous left there."""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
import synth
from gl_testutil import TOL_BF16, TOL_F32, assert_bits_equal, assert_close, nan_tail, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def case(seed, G, K, N, m, dtype=torch.bfloat16, bias=True):
    g = torch.Generator().manual_seed(seed)
    T = sum(m)
    x = torch.randn(T, K, generator=g).to(dtype)
    w = (torch.randn(G, N, K, generator=g) * 0.05).to(dtype)
    b = (torch.randn(G, N, generator=g) * 0.1).to(dtype) if bias else None
    return x, w, b


def run_both(x, w, b, m, tail=7):
    """y of the allocation-free call (into a caller buffer with a NaN tail) and of
    the workspace call."""
    T, N = x.shape[0], w.shape[1]
    md = torch.tensor(m, dtype=torch.int64, device=DEV)
    xd, wd = x.to(DEV), w.to(DEV)
    bd = b.to(DEV) if b is not None else None
    y = nan_tail(T + tail, N, T, x.dtype, DEV)
    gl.gl_forward_noalloc(md, xd, wd, y, bias=bd)
    ws = gl.new_workspace(len(m))
    gl.gl_offsets(md, T, ws)
    y_ws = torch.empty(T, N, dtype=x.dtype, device=DEV)
    gl.gl_forward(xd, wd, y_ws, ws, bias=bd)
    torch.cuda.synchronize()
    assert torch.isnan(y[T:]).all(), "rows past T written"
    return y[:T], y_ws


def test_noalloc_forward_calls_in_a_row():
    # 1: 8 groups, one empty; the workspace forward splits its tail round over the
    #    contraction, the allocation-free one (fewer partial slots) may not: the two
    #    agree within the bf16 bound
    G, K, N, m = 8, 512, 1024, [700, 0, 300, 511, 1, 900, 257, 64]
    say(f"noalloc call 1: G={G} K={K} N={N} m={m}")
    x, w, b = case(1, G, K, N, m)
    y, y_ws = run_both(x, w, b, m)
    ref = oracle.forward(to64(x), to64(w), to64(b), m)
    assert_close(y, to64(y_ws), TOL_BF16, "noalloc vs workspace forward (call 1)")
    assert_close(y, ref, TOL_BF16, "noalloc vs oracle (call 1)")

    # 2: smaller, 3 groups; both paths split the 6 tiles into the same parts, so the
    #    results are bit-identical (and the split counters left by call 1 were reset)
    G, K, N, m = 3, 1024, 512, [0, 300, 77]
    say(f"noalloc call 2: G={G} K={K} N={N} m={m}")
    x, w, b = case(2, G, K, N, m)
    y, y_ws = run_both(x, w, b, m)
    assert_bits_equal(y, y_ws, "noalloc vs workspace forward (call 2)")
    assert_close(y, oracle.forward(to64(x), to64(w), to64(b), m), TOL_BF16, "noalloc vs oracle (call 2)")

    # 3: smaller again, the fp32 workload with an empty group
    wl = synth.WORKLOADS["fwd_f32_g4_k64_n32"]
    m = synth.split_sizes(wl).tolist()
    say(f"noalloc call 3: {wl.name} m={m}")
    x, w, b = synth.x(wl), synth.weight(wl), synth.bias(wl)
    y, y_ws = run_both(x, w, b, m, tail=3)
    assert_bits_equal(y, y_ws, "noalloc vs workspace forward (call 3, fp32)")
    assert_close(y, oracle.forward(to64(x), to64(w), to64(b), m), TOL_F32, "noalloc vs oracle (call 3)")


def test_noalloc_forward_mxfp8_and_invalid_splits():
    """The MXFP8 form, then splits that do not add up to T: the forward writes
    nothing, and a following valid call is unaffected."""
    G, K, N, m = 4, 256, 256, [100, 0, 129, 30]
    T = sum(m)
    say(f"noalloc MXFP8: G={G} K={K} N={N} m={m}")
    x, w, _ = case(3, G, K, N, m, bias=False)
    xq, xs = torch.empty(T, K, dtype=torch.uint8, device=DEV), torch.empty(T, K // 32, dtype=torch.uint8, device=DEV)
    wq = torch.empty(G, N, K, dtype=torch.uint8, device=DEV)
    wsc = torch.empty(G, N, K // 32, dtype=torch.uint8, device=DEV)
    gl.gl_group_quantize_mxfp8(x.to(DEV), xq, xs)
    gl.gl_group_quantize_mxfp8(w.to(DEV), wq, wsc)
    md = torch.tensor(m, dtype=torch.int64, device=DEV)
    y = nan_tail(T + 2, N, T, torch.bfloat16, DEV)
    gl.gl_forward_noalloc(md, xq, wq, y, x_scale=xs, w_scale=wsc)
    ws = gl.new_workspace(G)
    gl.gl_offsets(md, T, ws)
    y_ws = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    gl.gl_forward(xq, wq, y_ws, ws, x_scale=xs, w_scale=wsc)
    torch.cuda.synchronize()
    assert_bits_equal(y[:T], y_ws, "MXFP8 noalloc vs workspace forward")
    assert torch.isnan(y[T:]).all()

    say("noalloc with splits that do not add up to T")
    bad = torch.tensor([100, 0, 129, 31], dtype=torch.int64, device=DEV)
    y_bad = nan_tail(T, N, 0, torch.bfloat16, DEV)
    gl.gl_forward_noalloc(bad, xq, wq, y_bad, x_scale=xs, w_scale=wsc)
    torch.cuda.synchronize()
    assert torch.isnan(y_bad).all(), "invalid splits: nothing written"
    y2 = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    gl.gl_forward_noalloc(md, xq, wq, y2, x_scale=xs, w_scale=wsc)
    torch.cuda.synchronize()
    assert_bits_equal(y2, y_ws, "valid call after an invalid one")
