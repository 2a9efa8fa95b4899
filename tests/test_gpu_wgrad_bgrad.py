"""GPU parity of gl_wgrad_bgrad: the weight gradient and the bias gradient of the
same dy in one call (for 16-bit inputs the bias gradient is summed from the dy
stages the wgrad tiles of the first column already hold in LDS).

The weight gradient must equal gl_wgrad's bit for bit (the added sums do not touch
the GEMM); the bias gradient is checked against the oracle (tolerance), exactly on
integer inputs, and for empty groups in both store and accumulate mode.
"""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
import synth
from gl_testutil import TOL_BF16, TOL_F32, assert_bits_equal, assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"

SHAPES = [
    # (G, K, N, m): ragged rows, partial k and n tiles, empty groups (first, last, adjacent)
    (5, 200, 264, [0, 300, 1, 0, 513]),
    (3, 256, 512, [256, 257, 255]),
    (1, 64, 8, [37]),
    (8, 136, 72, [3, 0, 0, 70, 260, 1, 0, 90]),
    (4, 520, 776, [700, 0, 64, 1100]),
]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def workspace_for(m):
    ws = gl.new_workspace(len(m))
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), int(sum(m)), ws)
    return ws


def case(seed, G, K, N, m, dtype, integer=False):
    g = torch.Generator().manual_seed(seed)
    T = int(sum(m))
    if integer:
        r = lambda *s: torch.randint(-3, 4, s, generator=g).to(dtype)
        return r(T, K), r(T, N), torch.randint(-3, 4, (G, N, K), generator=g).float()
    return (torch.randn(T, K, generator=g).to(dtype), torch.randn(T, N, generator=g).to(dtype),
            torch.randn(G, N, K, generator=g))


@pytest.mark.parametrize("G,K,N,m", SHAPES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32])
def test_wgrad_bgrad_matches_oracle_and_wgrad(G, K, N, m, dtype):
    say(f"wgrad+bgrad {dtype} G={G} K={K} N={N} m={m}")
    x, dy, mg = case(21, G, K, N, m, dtype)
    ws = workspace_for(m)
    xd, dyd = x.to(DEV), dy.to(DEV)
    dw = torch.full((G, N, K), float("nan"), dtype=dtype, device=DEV)
    db = torch.full((G, N), float("nan"), dtype=dtype, device=DEV)
    gl.gl_wgrad_bgrad(xd, dyd, dw, db, ws)
    dw_ref = torch.full((G, N, K), float("nan"), dtype=dtype, device=DEV)
    gl.gl_wgrad(xd, dyd, dw_ref, ws)
    # fp32 bias grad into per-group buffers, with accumulate into main_grad
    mgd = mg.to(DEV)
    db32 = [torch.full((N,), float("nan"), device=DEV) for _ in range(G)]
    gl.gl_wgrad_bgrad(xd, dyd, mgd, db32, ws, accumulate=True)
    torch.cuda.synchronize()
    assert_bits_equal(dw, dw_ref, "dW equals gl_wgrad's")
    DY = to64(dy)
    tol = TOL_F32 if dtype == torch.float32 else 2e-3 if dtype == torch.float16 else TOL_BF16
    ref_db = oracle.bgrad(DY, m)
    assert_close(db, ref_db, tol, "db")
    assert_close(torch.stack(db32), ref_db, TOL_F32 if dtype == torch.float32 else 1e-4, "db fp32")
    X, MG = to64(x), to64(mg)
    assert_close(mgd, oracle.wgrad(X, DY, m, main_grad=MG, accumulate=True), TOL_F32, "main_grad")
    for g in range(G):
        if m[g] == 0:
            assert not db[g].float().abs().sum().item() and not db32[g].abs().sum().item()
            assert_bits_equal(mgd[g], mg[g].to(DEV), f"empty group {g} main_grad untouched")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_wgrad_bgrad_integer_exact(dtype):
    G, K, N, m = 4, 264, 520, [130, 0, 257, 64]
    x, dy, _ = case(22, G, K, N, m, dtype, integer=True)
    ws = workspace_for(m)
    dw = torch.empty(G, N, K, dtype=torch.float32, device=DEV)
    db = torch.empty(G, N, dtype=torch.float32, device=DEV)
    gl.gl_wgrad_bgrad(x.to(DEV), dy.to(DEV), dw, db, ws)
    torch.cuda.synchronize()
    assert np.array_equal(db.cpu().numpy(), oracle.bgrad(to64(dy), m)), "db not exact on integers"
    assert np.array_equal(dw.cpu().numpy(), oracle.wgrad(to64(x), to64(dy), m)), "dW not exact on integers"


def test_wgrad_bgrad_long_group_fp32_db():
    # fp32 bias grad of bf16 inputs over a 20000-row group (its tiles split into parts by
    # the contraction plan), held to the fp32 bound: each lane's column sum takes about
    # 1250 rows, two at a time
    G, K, N, m = 2, 64, 264, [20000, 37]
    say(f"wgrad+bgrad long group, fp32 db G={G} K={K} N={N} m={m}")
    x, dy, _ = case(24, G, K, N, m, torch.bfloat16)
    ws = workspace_for(m)
    dw = torch.empty(G, N, K, dtype=torch.bfloat16, device=DEV)
    db = torch.full((G, N), float("nan"), device=DEV)
    gl.gl_wgrad_bgrad(x.to(DEV), dy.to(DEV), dw, db, ws)
    torch.cuda.synchronize()
    assert_close(db, oracle.bgrad(to64(dy), m), TOL_F32, "db fp32, 20000-row group")


def test_wgrad_bgrad_deterministic():
    G, K, N, m = 3, 512, 1024, [1000, 17, 600]
    x, dy, _ = case(23, G, K, N, m, torch.bfloat16)
    ws = workspace_for(m)
    outs = []
    for _ in range(2):
        dw = torch.empty(G, N, K, dtype=torch.bfloat16, device=DEV)
        db = torch.empty(G, N, dtype=torch.bfloat16, device=DEV)
        gl.gl_wgrad_bgrad(x.to(DEV), dy.to(DEV), dw, db, ws)
        outs.append((dw, db))
    torch.cuda.synchronize()
    assert_bits_equal(outs[0][0], outs[1][0], "dW")
    assert_bits_equal(outs[0][1], outs[1][1], "db")


def test_wgrad_bgrad_8_group_workload():
    wl = synth.WORKLOADS["bf16_train_g8_k4096_n14336"]
    say(f"workload {wl.name}: generating")
    m = synth.split_sizes(wl)
    x, dy = synth.x(wl), synth.dy(wl)
    ws = workspace_for(m.tolist())
    dw = torch.empty(wl.G, wl.N, wl.K, dtype=torch.bfloat16, device=DEV)
    db = torch.empty(wl.G, wl.N, dtype=torch.bfloat16, device=DEV)
    say("  launching wgrad+bgrad")
    gl.gl_wgrad_bgrad(x.to(DEV), dy.to(DEV), dw, db, ws)
    db_sep = torch.empty_like(db)
    gl.gl_bgrad(dy.to(DEV), db_sep, ws)
    torch.cuda.synchronize()
    say("  checking against the oracle")
    DY = dy.float().numpy()
    assert_close(db, oracle.bgrad(DY, m), TOL_BF16, "db")
    assert_close(db, to64(db_sep), TOL_BF16, "db vs the separate kernel")
    groups, nsel = [0, 5], np.array([0, 255, 256, 9000, wl.N - 1])
    ref = oracle.wgrad(x.float().numpy(), DY, m, groups=groups, out_rows=nsel)
    assert_close(dw[groups][:, torch.from_numpy(nsel).to(DEV)], ref, TOL_BF16, "dW rows")
