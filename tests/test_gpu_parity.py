"""GPU parity of every library entry point against the CPU oracle, through the C ABI.

Oracle-sized cases that still span several 256x256 tiles, ragged row tiles,
partial column tiles and partial contraction tiles, with empty groups at the
start, middle and end.  Integer-valued cases must match bit for bit (every sum is
exact in fp32 and bf16); random cases meet the fp32 / bf16 tolerances.
"""
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


def workspace_for(m, T):
    G = len(m)
    ws = gl.new_workspace(G)
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), T, ws)
    return ws


def rand_case(seed, G, K, N, m, dtype, scale_w=0.05):
    g = torch.Generator().manual_seed(seed)
    T = int(sum(m))
    x = torch.randn(T, K, generator=g).to(dtype)
    w = (torch.randn(G, N, K, generator=g) * scale_w).to(dtype)
    b = (torch.randn(G, N, generator=g) * 0.1).to(dtype)
    dy = torch.randn(T, N, generator=g).to(dtype)
    mg = torch.randn(G, N, K, generator=g)
    return x, w, b, dy, mg


def int_case(seed, G, K, N, m, dtype):
    g = torch.Generator().manual_seed(seed)
    T = int(sum(m))
    r = lambda *s: torch.randint(-3, 4, s, generator=g).to(dtype)
    return r(T, K), r(G, N, K), r(G, N), r(T, N), torch.randint(-3, 4, (G, N, K), generator=g).float()


SHAPES = [
    # (G, K, N, m): ragged rows, partial k tile (K % 64), partial n tile, empty groups.
    # The first four average at most 256 rows per group (the forward's deeper weight
    # ring), the last two more (its default ring).
    (5, 200, 264, [0, 300, 1, 0, 513]),
    (3, 256, 512, [256, 257, 255]),
    (1, 64, 8, [37]),
    (8, 136, 72, [3, 0, 0, 70, 260, 1, 0, 90]),
    # several full 256-row tiles in a group, then a ragged one
    (2, 200, 264, [700, 301]),
    (3, 136, 72, [600, 0, 517]),
]


# --------------------------------------------------------------------- offsets

@pytest.mark.parametrize("n", [1, 2, 17, 256, 257, 513, 1024, 3000])
def test_offsets_bit_exact(n):
    say(f"offsets n={n}")
    rng = np.random.default_rng(n)
    m = rng.integers(0, 700, size=n)
    m[rng.integers(0, n, size=max(1, n // 4))] = 0
    if n > 2:
        m[0] = m[-1] = 0
        m[n // 2: n // 2 + 2] = 0
    T = int(m.sum())
    ws = workspace_for(m.tolist(), T)
    assert gl.gl_read_status(ws) == 0
    got = gl.workspace_offsets(ws, n).cpu().numpy()
    assert np.array_equal(got, oracle.offsets(m, n, T))
    # row-tile tables: exclusive prefix of ceil(m / rows) for each tile height
    for i, rows in enumerate((32, 64, 128, 256)):
        base = 32 + 8 * (n + 1) + i * 4 * (n + 1)
        tab = ws[base: base + 4 * (n + 1)].view(torch.int32).cpu().numpy()
        ref = np.concatenate([[0], np.cumsum((m + rows - 1) // rows)])
        assert np.array_equal(tab, ref)


@pytest.mark.parametrize("m,T,bit", [([3, -1, 4], 6, 1), ([3, 1, 4], 9, 2), ([-2, 5], 0, 3)])
def test_invalid_splits_set_status_and_write_nothing(m, T, bit):
    say(f"invalid splits m={m} T={T}")
    G, K, N = len(m), 64, 64
    ws = workspace_for(m, T)
    assert gl.gl_read_status(ws) & bit == bit
    rows = max(T, 1)
    x = torch.ones(rows, K, dtype=torch.bfloat16, device=DEV)[:T]
    w = torch.ones(G, N, K, dtype=torch.bfloat16, device=DEV)
    y = nan_tail(rows, N, 0, torch.bfloat16, DEV)
    before = y.clone()
    gl.gl_forward(x, w, y, ws)
    gl.gl_dgrad(torch.ones(T, N, dtype=torch.bfloat16, device=DEV), w, y[:, :K], ws)
    mg = torch.full((G, N, K), 7.0, device=DEV)
    gl.gl_wgrad(x, torch.ones(T, N, dtype=torch.bfloat16, device=DEV), mg, ws, accumulate=False)
    db = torch.full((G, N), 3.0, dtype=torch.bfloat16, device=DEV)
    gl.gl_bgrad(torch.ones(T, N, dtype=torch.bfloat16, device=DEV), db, ws)
    torch.cuda.synchronize()
    assert_bits_equal(y, before, "forward output after invalid splits")
    assert bool((mg == 7.0).all()) and bool((db == 3.0).all())


def test_workspace_for_other_sizes_is_refused():
    say("workspace mismatch")
    m = [4, 4]
    ws = workspace_for(m, 8)
    x = torch.ones(9, 64, dtype=torch.bfloat16, device=DEV)
    w = torch.ones(2, 64, 64, dtype=torch.bfloat16, device=DEV)
    y = nan_tail(9, 64, 0, torch.bfloat16, DEV)
    before = y.clone()
    gl.gl_forward(x, w, y, ws)  # 9 rows against a workspace built for 8
    assert gl.gl_read_status(ws) & gl.GL_STATUS_WORKSPACE
    assert_bits_equal(y, before, "output after workspace mismatch")


# -------------------------------------------------------------- bit-exact ints

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_integer_cases_bit_exact(dtype):
    G, K, N, m = 3, 16, 16, [5, 0, 6]
    say(f"integer case {dtype}")
    x, w, b, dy, mg = int_case(1, G, K, N, m, dtype)
    T = sum(m)
    ws = workspace_for(m, T)
    xd, wd, bd, dyd = (t.to(DEV) for t in (x, w, b, dy))
    y = torch.empty(T, N, dtype=dtype, device=DEV)
    gl.gl_forward(xd, wd, y, ws, bias=bd)
    dx = torch.empty(T, K, dtype=dtype, device=DEV)
    gl.gl_dgrad(dyd, wd, dx, ws)
    dw = torch.empty(G, N, K, dtype=dtype, device=DEV)
    gl.gl_wgrad(xd, dyd, dw, ws)
    mgd = mg.to(DEV)
    gl.gl_wgrad(xd, dyd, mgd, ws, accumulate=True)
    db = torch.empty(G, N, dtype=dtype, device=DEV)
    gl.gl_bgrad(dyd, db, ws)
    torch.cuda.synchronize()
    X, W, B, DY, MG = (to64(t) for t in (x, w, b, dy, mg))
    assert np.array_equal(to64(y), oracle.forward(X, W, B, m))
    assert np.array_equal(to64(dx), oracle.dgrad(DY, W, m))
    assert np.array_equal(to64(dw), oracle.wgrad(X, DY, m))
    assert np.array_equal(to64(mgd), oracle.wgrad(X, DY, m, main_grad=MG, accumulate=True))
    assert np.array_equal(to64(db), oracle.bgrad(DY, m))


# ------------------------------------------------------------ random, ragged

@pytest.mark.parametrize("G,K,N,m", SHAPES)
def test_forward_bf16(G, K, N, m):
    say(f"forward bf16 G={G} K={K} N={N} m={m}")
    x, w, b, _, _ = rand_case(2, G, K, N, m, torch.bfloat16)
    T = sum(m)
    ws = workspace_for(m, T)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    y = nan_tail(T + 37, N, T, torch.bfloat16, DEV)
    gl.gl_forward(xd, wd, y, ws, bias=bd)
    y_exact = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    gl.gl_forward(xd, [wd[g] for g in range(G)], y_exact, ws, bias=[bd[g] for g in range(G)])
    y_nb = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    gl.gl_forward(xd, wd, y_nb, ws)
    torch.cuda.synchronize()
    X, Wt, B = to64(x), to64(w), to64(b)
    assert_close(y[:T], oracle.forward(X, Wt, B, m), TOL_BF16, "y (stacked, bias)")
    assert torch.isnan(y[T:]).all() and bool((y[T:].view(torch.int16) == y[T:].view(torch.int16)[0, 0]).all())
    assert_bits_equal(y[:T], y_exact, "caller buffer vs exact-size buffer / per-group pointers")
    assert_close(y_nb, oracle.forward(X, Wt, None, m), TOL_BF16, "y (no bias)")


@pytest.mark.parametrize("G,K,N,m", SHAPES)
def test_dgrad_bf16(G, K, N, m):
    say(f"dgrad bf16 G={G} K={K} N={N} m={m}")
    _, w, _, dy, _ = rand_case(3, G, K, N, m, torch.bfloat16)
    T = sum(m)
    ws = workspace_for(m, T)
    dx = nan_tail(T + 5, K, T, torch.bfloat16, DEV)
    gl.gl_dgrad(dy.to(DEV), w.to(DEV), dx, ws)
    dx2 = torch.empty(T, K, dtype=torch.bfloat16, device=DEV)
    gl.gl_dgrad(dy.to(DEV), [t.to(DEV) for t in w], dx2, ws)
    torch.cuda.synchronize()
    assert_close(dx[:T], oracle.dgrad(to64(dy), to64(w), m), TOL_BF16, "dx")
    assert torch.isnan(dx[T:]).all()
    assert_bits_equal(dx[:T], dx2, "dgrad caller buffer vs exact / per-group pointers")


@pytest.mark.parametrize("G,K,N,m", SHAPES)
def test_wgrad_bf16(G, K, N, m):
    say(f"wgrad bf16 G={G} K={K} N={N} m={m}")
    x, _, _, dy, mg = rand_case(4, G, K, N, m, torch.bfloat16)
    T = sum(m)
    ws = workspace_for(m, T)
    xd, dyd = x.to(DEV), dy.to(DEV)
    dw = torch.full((G, N, K), float("nan"), dtype=torch.bfloat16, device=DEV)
    gl.gl_wgrad(xd, dyd, dw, ws)
    mgd = mg.to(DEV)
    gl.gl_wgrad(xd, dyd, mgd, ws, accumulate=True)
    dwf = [torch.full((N, K), 5.0, device=DEV) for _ in range(G)]
    gl.gl_wgrad(xd, dyd, dwf, ws)
    torch.cuda.synchronize()
    X, DY, MG = to64(x), to64(dy), to64(mg)
    ref = oracle.wgrad(X, DY, m)
    assert_close(dw, ref, TOL_BF16, "dW bf16 store")
    assert_close(torch.stack(dwf), ref, TOL_F32, "dW fp32 per-group store")
    assert_close(mgd, oracle.wgrad(X, DY, m, main_grad=MG, accumulate=True), TOL_F32, "main_grad accumulate")
    for g in range(G):
        if m[g] == 0:
            assert_bits_equal(mgd[g], mg[g].to(DEV), f"empty group {g} main_grad untouched")
            assert not dw[g].float().abs().sum().item()


@pytest.mark.parametrize("G,K,N,m", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_bgrad(G, K, N, m, dtype):
    say(f"bgrad {dtype} G={G} N={N} m={m}")
    _, _, _, dy, _ = rand_case(5, G, K, N, m, dtype)
    T = sum(m)
    ws = workspace_for(m, T)
    db = torch.full((G, N), float("nan"), dtype=dtype, device=DEV)
    gl.gl_bgrad(dy.to(DEV), db, ws)
    torch.cuda.synchronize()
    assert_close(db, oracle.bgrad(to64(dy), m), TOL_BF16 if dtype == torch.bfloat16 else TOL_F32, "db")


def test_wgrad_deterministic():
    G, K, N, m = 8, 136, 72, [3, 0, 0, 70, 260, 1, 0, 90]
    say("wgrad determinism")
    x, _, _, dy, _ = rand_case(6, G, K, N, m, torch.bfloat16)
    ws = workspace_for(m, sum(m))
    a = torch.zeros(G, N, K, device=DEV)
    b = torch.zeros(G, N, K, device=DEV)
    gl.gl_wgrad(x.to(DEV), dy.to(DEV), a, ws)
    gl.gl_wgrad(x.to(DEV), dy.to(DEV), b, ws)
    torch.cuda.synchronize()
    assert_bits_equal(a, b, "two wgrad runs")


# ----------------------------------------------------------------- fp32 path

def test_fp32_tiny_workload():
    wl = synth.WORKLOADS["fwd_f32_g4_k64_n32"]
    say(f"workload {wl.name}")
    m = synth.split_sizes(wl).tolist()
    x, w, b = synth.x(wl), synth.weight(wl), synth.bias(wl)
    ws = workspace_for(m, wl.T)
    y = torch.empty(wl.T, wl.N, dtype=torch.float32, device=DEV)
    gl.gl_forward(x.to(DEV), w.to(DEV), y, ws, bias=b.to(DEV))
    torch.cuda.synchronize()
    assert_close(y, oracle.forward(to64(x), to64(w), to64(b), m), TOL_F32, "fp32 forward")


@pytest.mark.parametrize("G,K,N,m", [(5, 70, 33, [0, 40, 1, 0, 90]), (2, 64, 32, [30, 34])])
def test_fp32_all_passes(G, K, N, m):
    say(f"fp32 passes G={G} K={K} N={N} m={m}")
    x, w, b, dy, mg = rand_case(7, G, K, N, m, torch.float32)
    T = sum(m)
    ws = workspace_for(m, T)
    y = nan_tail(T + 3, N, T, torch.float32, DEV)
    gl.gl_forward(x.to(DEV), w.to(DEV), y, ws, bias=b.to(DEV))
    dx = torch.empty(T, K, device=DEV)
    gl.gl_dgrad(dy.to(DEV), w.to(DEV), dx, ws)
    mgd = mg.to(DEV)
    gl.gl_wgrad(x.to(DEV), dy.to(DEV), mgd, ws, accumulate=True)
    torch.cuda.synchronize()
    X, Wt, B, DY, MG = (to64(t) for t in (x, w, b, dy, mg))
    assert_close(y[:T], oracle.forward(X, Wt, B, m), TOL_F32, "fp32 y")
    assert torch.isnan(y[T:]).all()
    assert_close(dx, oracle.dgrad(DY, Wt, m), TOL_F32, "fp32 dx")
    assert_close(mgd, oracle.wgrad(X, DY, m, main_grad=MG, accumulate=True), TOL_F32, "fp32 main_grad")


# --------------------------------------------------------------------- MXFP8

def test_quantize_every_bf16_pattern_bit_exact():
    say("quantize exhaustive")
    v = synth.special_bf16_block_values()
    n = (v.numel() // 256) * 256
    rng = np.random.default_rng(11)
    mixed = v[torch.from_numpy(rng.permutation(v.numel())[:n])]
    ordered = v[torch.argsort(v.float().abs())][:n]   # blocks of like magnitudes: every scale
    src = torch.cat([mixed, ordered]).reshape(-1, 256)
    # blocks at several magnitudes, an all-zero block and NaN / Inf blocks
    src[0, :32] = 0.0
    src[1, 32:64] = float("inf")
    src[2, 64:96] = float("nan")
    src[3, :32] = torch.linspace(-1, 1, 32).to(torch.bfloat16) * 2.0 ** -130
    data = torch.empty(src.shape, dtype=torch.uint8, device=DEV)
    scale = torch.empty(src.shape[0], src.shape[1] // 32, dtype=torch.uint8, device=DEV)
    gl.gl_group_quantize_mxfp8(src.to(DEV), data, scale)
    torch.cuda.synchronize()
    q, s = oracle.quantize_mxfp8(src.double().numpy())
    assert np.array_equal(scale.cpu().numpy(), s)
    assert np.array_equal(data.cpu().numpy(), q)


@pytest.mark.parametrize("e", [0, 16])
def test_quantize_every_scaled_value_bit_exact(e):
    """Every value the E4M3 rounding can be handed: a block whose first element is
    1.5 * 2^(8+e) has shared exponent e, so its other 31 elements (every finite bf16
    of magnitude at most that) reach the rounding as v * 2^-e.  e = 0 and e = 16
    together cover every value of 8 significant bits from 2^-149 to 2^8, both signs."""
    say(f"quantize every scaled value, e={e}")
    v = synth.special_bf16_block_values()
    head = 1.5 * 2.0 ** (8 + e)
    v = v[v.float().abs() <= head]
    n = (v.numel() + 30) // 31
    body = torch.zeros(n * 31, dtype=torch.bfloat16)
    body[: v.numel()] = v
    src = torch.cat([torch.full((n, 1), head, dtype=torch.bfloat16), body.reshape(n, 31)], dim=1)
    src = src.reshape(-1, 32 * 8) if n % 8 == 0 else torch.cat(
        [src, torch.full((8 - n % 8, 32), head, dtype=torch.bfloat16)]).reshape(-1, 32 * 8)
    data = torch.empty(src.shape, dtype=torch.uint8, device=DEV)
    scale = torch.empty(src.shape[0], src.shape[1] // 32, dtype=torch.uint8, device=DEV)
    gl.gl_group_quantize_mxfp8(src.to(DEV), data, scale)
    torch.cuda.synchronize()
    q, s = oracle.quantize_mxfp8(src.double().numpy())
    assert (s == 127 + e).all(), "every block has the intended shared exponent"
    assert np.array_equal(scale.cpu().numpy(), s)
    assert np.array_equal(data.cpu().numpy(), q)


@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("G,K,N,m", [(3, 256, 264, [0, 300, 77]), (4, 128, 512, [256, 1, 0, 257])])
def test_mxfp8_forward(G, K, N, m, out):
    """bf16 output at the bf16 bound; fp32 output (bias added to the fp32 accumulator,
    stored unrounded) at the fp32 bound, since the products of decoded codes are
    exact and only the fp32 summation order differs from the oracle."""
    say(f"mxfp8 forward G={G} K={K} N={N} m={m} out={out}")
    x, w, b, _, _ = rand_case(8, G, K, N, m, torch.bfloat16, scale_w=0.02)
    T = sum(m)
    ws = workspace_for(m, T)
    xq = torch.empty(T, K, dtype=torch.uint8, device=DEV)
    xs = torch.empty(T, K // 32, dtype=torch.uint8, device=DEV)
    gl.gl_group_quantize_mxfp8(x.to(DEV), xq, xs)
    wq = torch.empty(G, N, K, dtype=torch.uint8, device=DEV)
    wsc = torch.empty(G, N, K // 32, dtype=torch.uint8, device=DEV)
    gl.gl_group_quantize_mxfp8(w.to(DEV), wq, wsc)
    y = nan_tail(T + 11, N, T, out, DEV)
    bo = b.to(out).to(DEV)  # the bias comes in the output type (bf16 -> fp32 is exact)
    gl.gl_forward(xq, wq, y, ws, x_scale=xs, w_scale=wsc, bias=bo)
    y2 = torch.empty(T, N, dtype=out, device=DEV)
    gl.gl_forward(xq, [wq[g] for g in range(G)], y2, ws, x_scale=xs, w_scale=[wsc[g] for g in range(G)], bias=bo)
    torch.cuda.synchronize()
    oq, os_ = oracle.quantize_mxfp8(to64(x))
    assert np.array_equal(xq.cpu().numpy(), oq) and np.array_equal(xs.cpu().numpy(), os_)
    wqs = [oracle.quantize_mxfp8(to64(w[g])) for g in range(G)]
    assert np.array_equal(wq.cpu().numpy(), np.stack([a for a, _ in wqs]))
    ref = oracle.forward_mxfp8(oq, os_, [a for a, _ in wqs], [c for _, c in wqs], to64(b), m)
    assert_close(y[:T], ref, TOL_BF16 if out == torch.bfloat16 else TOL_F32, "MXFP8 forward")
    assert torch.isnan(y[T:]).all()
    assert_bits_equal(y[:T], y2, "MXFP8 stacked vs per-group weights")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
@pytest.mark.parametrize("per_group", [False, True])
def test_wgrad_accumulate_into_16bit(dtype, per_group):
    """accumulate=1 into a weight gradient of the input type (not an fp32 main_grad):
    the stored value is read, the fp32 sum added and the result rounded once; an
    empty group's gradient stays bit-identical."""
    G, K, N, m = 3, 136, 200, [0, 300, 77]
    say(f"wgrad accumulate into {dtype} per_group={per_group}")
    x, _, _, dy, mg = rand_case(31, G, K, N, m, dtype)
    mg16 = mg.to(dtype)
    ws = workspace_for(m, sum(m))
    dw = [t.to(DEV) for t in mg16] if per_group else mg16.to(DEV)
    gl.gl_wgrad(x.to(DEV), dy.to(DEV), dw, ws, accumulate=True)
    torch.cuda.synchronize()
    got = torch.stack(dw) if per_group else dw
    assert_close(got, oracle.wgrad(to64(x), to64(dy), m, main_grad=to64(mg16), accumulate=True),
                 TOL_BF16 if dtype == torch.bfloat16 else 2e-3, "16-bit accumulate")
    assert_bits_equal(got[0], mg16[0].to(DEV), "empty group untouched")


def test_mxfp8_wgrad_accumulate_into_bf16():
    """The MXFP8 wgrad's accumulate mode into a bf16 weight gradient."""
    G, K, N, m = 3, 128, 256, [100, 0, 333]
    T = sum(m)
    say("MXFP8 wgrad accumulate into bf16")
    x, _, _, dy, mg = rand_case(32, G, K, N, m, torch.bfloat16)
    mg16 = mg.to(torch.bfloat16)
    ws = workspace_for(m, T)
    ld = gl.gl_colwise_ld(G, T)
    u8 = dict(dtype=torch.uint8, device=DEV)
    xq, xs = torch.zeros(K, ld, **u8), torch.zeros(K, ld // 32, **u8)
    dq, ds = torch.zeros(N, ld, **u8), torch.zeros(N, ld // 32, **u8)
    gl.gl_group_quantize_mxfp8_colwise(x.to(DEV), xq, xs, ws, G)
    gl.gl_group_quantize_mxfp8_colwise(dy.to(DEV), dq, ds, ws, G)
    dw = mg16.to(DEV)
    gl.gl_wgrad_mxfp8(dq, ds, xq, xs, dw, ws, T, accumulate=True)
    torch.cuda.synchronize()
    cxq, cxs, poff = oracle.quantize_mxfp8_colwise(to64(x), m, ld=ld)
    cdq, cds, _ = oracle.quantize_mxfp8_colwise(to64(dy), m, ld=ld)
    end = int(poff[-1])
    ref = oracle.wgrad_mxfp8(cdq[:, :end], cds[:, : end // 32], cxq[:, :end], cxs[:, : end // 32], m,
                             main_grad=to64(mg16), accumulate=True)
    assert_close(dw, ref, TOL_BF16, "MXFP8 accumulate into bf16")
    assert_bits_equal(dw[1], mg16[1].to(DEV), "empty group untouched")
