"""GPU parity at the workloads' full sizes, through the C ABI, in the same launch
configuration the benchmark times.

Every element of every output is compared with the float64 oracle, which runs one
group at a time (tests/full_check.py).  Quantized codes and scales are compared
bit for bit with the oracle's own quantization of the same inputs before the
oracle's GEMMs consume them.  Inputs come from the seeded generators in synth.py.
"""
import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
import synth
from full_check import assert_codes_equal, check_chunks, group_bounds, pool_map, say
from gl_testutil import TOL_BF16, assert_bits_equal, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


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
    dw_sep = torch.empty_like(dw)
    db_sep = torch.empty_like(db)
    say("  launching offsets/forward/dgrad/wgrad+bgrad (fused, as timed) and wgrad, bgrad alone")
    gl.gl_forward(xd, wd, y, ws, bias=bd)
    gl.gl_dgrad(dyd, wd, dx, ws)
    gl.gl_wgrad_bgrad(xd, dyd, dw, db, ws)
    gl.gl_wgrad(xd, dyd, dw_sep, ws)
    gl.gl_bgrad(dyd, db_sep, ws)
    torch.cuda.synchronize()
    assert_bits_equal(dw, dw_sep, "dW of the fused call vs gl_wgrad")
    say("  checking every element against the oracle")
    X, DY, B = x.float().numpy(), dy.float().numpy(), to64(b)
    yc, dxc = y.cpu(), dx.cpu()
    bounds = group_bounds(m)

    def fwd_chunks():
        for g, lo, hi in bounds:
            Wg = w[g].double().numpy()
            yield g, yc[lo:hi], oracle.forward(X[lo:hi], [Wg], [B[g]], [hi - lo])

    def dgrad_chunks():
        for g, lo, hi in bounds:
            Wg = w[g].double().numpy()
            yield g, dxc[lo:hi], oracle.dgrad(DY[lo:hi], [Wg], [hi - lo])

    def wgrad_chunks():
        for g, lo, hi in bounds:
            yield g, dw[g].cpu(), oracle.wgrad(X[lo:hi], DY[lo:hi], [hi - lo])[0]

    check_chunks("y", TOL_BF16, fwd_chunks())
    check_chunks("dx", TOL_BF16, dgrad_chunks())
    check_chunks("dW", TOL_BF16, wgrad_chunks())
    ref_db = oracle.bgrad(DY, m)
    check_chunks("db (fused)", TOL_BF16, [("all", db, ref_db)])
    check_chunks("db (gl_bgrad)", TOL_BF16, [("all", db_sep, ref_db)])


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
    say("  checking every element against the oracle")
    X, DY = x.float().numpy(), dy.float().numpy()
    yc, dxc, mgc = y.cpu(), dx.cpu(), mgd.cpu()
    bounds = [(g, lo, hi) for g, lo, hi in group_bounds(m) if hi > lo]
    check_chunks("y", TOL_BF16,
                 ((g, yc[lo:hi], oracle.forward(X[lo:hi], [w[g].double().numpy()], None, [hi - lo]))
                  for g, lo, hi in bounds))
    check_chunks("dx", TOL_BF16,
                 ((g, dxc[lo:hi], oracle.dgrad(DY[lo:hi], [w[g].double().numpy()], [hi - lo]))
                  for g, lo, hi in bounds))
    # fp32 main_grad of a bf16 GEMM: the products are exact in fp32, but the longest
    # group contracts over about 19 900 rows in one fp32 accumulator, and elements
    # whose sum cancels to near zero keep the rounding of partial sums of order 100.
    # Held to the bf16 GEMM bound on every element, and at least 99.99% of the
    # elements to the fp32 bound (measured: 99.9994%, worst err/limit 4.6); a
    # result rounded through 16 bits anywhere would fall far below that share.
    check_chunks("main_grad (fp32, accumulate)", TOL_BF16,
                 ((g, mgc[g], oracle.wgrad(X[lo:hi], DY[lo:hi], [hi - lo], main_grad=mg[g:g + 1].numpy(),
                                           accumulate=True)[0])
                  for g, lo, hi in bounds), f32_floor=0.9999)
    for g in np.nonzero(m == 0)[0]:
        assert_bits_equal(mgc[int(g)], mg[int(g)], f"empty group {g} main_grad")


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
    assert_bits_equal(y[wl.T:], tail_before, "padded tail")
    assert_bits_equal(y[: wl.T], y_stacked, "per-group pointers vs stacked weight")
    say("  checking every row against the oracle")
    X = x.float().numpy()
    yc = y[: wl.T].cpu()
    check_chunks("y", TOL_BF16,
                 ((g, yc[lo:hi], oracle.forward(X[lo:hi], [w[g].double().numpy()], None, [hi - lo]))
                  for g, lo, hi in group_bounds(m) if hi > lo))


def _rowwise_codes_check(what, src, q, s, block_rows=1024):
    """Rowwise codes and scales of src [rows, K] against the oracle, bit for bit,
    in blocks of rows on host threads."""
    qc, sc = q.cpu().numpy(), s.cpu().numpy()
    rows = src.shape[0]

    def one(lo):
        hi = min(rows, lo + block_rows)
        rq, rs = oracle.quantize_mxfp8(src[lo:hi].double().numpy())
        assert_codes_equal(f"{what} codes rows {lo}..{hi}", qc[lo:hi], rq)
        assert_codes_equal(f"{what} scales rows {lo}..{hi}", sc[lo:hi], rs)

    pool_map(one, range(0, rows, block_rows))
    say(f"  {what}: codes and scales of {rows} rows bit-exact")


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
    say("  checking every code against the oracle's quantization")
    _rowwise_codes_check("x", x, xq, xs)
    _rowwise_codes_check("W", w.view(wl.G * wl.N, wl.K), wq.view(wl.G * wl.N, wl.K),
                         wsc.view(wl.G * wl.N, wl.K // 32))
    say("  checking every element of y against the oracle on the dequantized operands")
    xq_c, xs_c, wq_c, ws_c = xq.cpu().numpy(), xs.cpu().numpy(), wq.cpu().numpy(), wsc.cpu().numpy()
    yc = y.cpu()
    check_chunks("MXFP8 y", TOL_BF16,
                 ((g, yc[lo:hi], oracle.forward_mxfp8(xq_c[lo:hi], xs_c[lo:hi], [wq_c[g]], [ws_c[g]], None,
                                                      [hi - lo]))
                  for g, lo, hi in group_bounds(m) if hi > lo))
