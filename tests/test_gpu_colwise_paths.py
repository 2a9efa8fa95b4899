"""GPU parity of the group-mode columnwise MXFP8 quantizer on each of its paths, bit
for bit against the oracle: the 128-row x 64-column tile kernel with its one-round
group lookup (fewer than 64 groups) and its two-round lookup (64 groups or more), and
the per-thread kernel it falls back to when the column count is not a multiple of 8
or the scale matrix is not 4-byte aligned (page "transformer_engine/pytorch/ops/
basic/grouped_linear.py", the quantized backward's columnwise usage; OCP MX rule)."""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
from gl_testutil import to64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_case(m, cols, seed, scale_offset=0):
    m = [int(v) for v in m]
    G, T = len(m), sum(m)
    g = torch.Generator().manual_seed(seed)
    x = (torch.randn(T, cols, generator=g) * 3).to(torch.bfloat16)
    if T > 40:
        x[7, 1] = float("-inf")  # a non-finite block
        x[33:40, 0] = 0.0
    ws = gl.new_workspace(G)
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), T, ws)
    ld = gl.gl_colwise_ld(G, T)
    q = torch.full((cols, ld), 0xAB, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((cols * (ld // 32) + 8,), 0xAB, dtype=torch.uint8, device=DEV)
    s = sbuf[scale_offset:scale_offset + cols * (ld // 32)].view(cols, ld // 32)
    assert s.data_ptr() % 4 == scale_offset % 4
    gl.gl_group_quantize_mxfp8_colwise(x.to(DEV), q, s, ws, G)
    torch.cuda.synchronize()
    rq, rs, poff = oracle.quantize_mxfp8_colwise(to64(x), m, ld=ld)
    end = int(poff[-1])
    assert np.array_equal(q[:, :end].cpu().numpy(), rq[:, :end]), "codes"
    assert np.array_equal(s[:, : end // 32].cpu().numpy(), rs[:, : end // 32]), "scales"
    assert (q[:, end:] == 0xAB).all() and (s[:, end // 32:] == 0xAB).all(), "columns past the padding"
    assert (sbuf[:scale_offset] == 0xAB).all() and (sbuf[scale_offset + s.numel():] == 0xAB).all()


def test_tile_path_two_round_lookup_many_groups():
    rng = np.random.default_rng(61)
    m = rng.integers(0, 200, 70) * (rng.random(70) < 0.7)
    m[[0, 35, 69]] = [0, 300, 0]
    say(f"colwise, 70 groups, T={int(m.sum())}, 72 columns")
    run_case(m, 72, 62)


def test_tile_path_one_round_lookup_63_groups():
    rng = np.random.default_rng(63)
    m = rng.integers(0, 150, 63)
    run_case(m, 136, 64)


@pytest.mark.parametrize("cols", [100, 36])
def test_fallback_columns_not_multiple_of_8(cols):
    run_case([50, 0, 257, 3], cols, 65)


@pytest.mark.parametrize("offset", [1, 2])
def test_fallback_misaligned_scales(offset):
    run_case([129, 0, 64, 300], 64, 66, scale_offset=offset)


@pytest.mark.parametrize("G,cols,scale_offset", [(5, 96, 0), (70, 64, 0), (4, 160, 1)])
def test_rowwise_and_colwise_in_one_pass(G, cols, scale_offset):
    """Both usages of one tensor from one call: bit-equal to the two separate
    quantizations and to the oracle (a misaligned columnwise scale matrix takes the
    two-launch path)."""
    rng = np.random.default_rng(67 + G)
    m = (rng.integers(0, 300, G) * (rng.random(G) < 0.8)).tolist()
    m[0] = 0
    T = int(sum(m))
    g = torch.Generator().manual_seed(68)
    x = (torch.randn(T, cols, generator=g) * 2).to(torch.bfloat16)
    ws = gl.new_workspace(G)
    gl.gl_offsets(torch.tensor(m, dtype=torch.int64, device=DEV), T, ws)
    ld = gl.gl_colwise_ld(G, T)
    u8 = dict(dtype=torch.uint8, device=DEV)
    dq, ds = torch.empty(T, cols, **u8), torch.empty(T, cols // 32, **u8)
    tq = torch.full((cols, ld), 0xAB, **u8)
    sbuf = torch.full((cols * (ld // 32) + 8,), 0xAB, **u8)
    ts = sbuf[scale_offset:scale_offset + cols * (ld // 32)].view(cols, ld // 32)
    xd = x.to(DEV)
    gl.gl_group_quantize_mxfp8_rowwise_colwise(xd, dq, ds, tq, ts, ws, G)
    rq, rs = torch.empty_like(dq), torch.empty_like(ds)
    gl.gl_group_quantize_mxfp8(xd, rq, rs)
    ctq, cts = torch.full((cols, ld), 0xAB, **u8), torch.full((cols, ld // 32), 0xAB, **u8)
    gl.gl_group_quantize_mxfp8_colwise(xd, ctq, cts, ws, G)
    torch.cuda.synchronize()
    assert torch.equal(dq, rq) and torch.equal(ds, rs), "rowwise differs from gl_group_quantize_mxfp8"
    assert torch.equal(tq, ctq) and torch.equal(ts, cts), "columnwise differs from gl_group_quantize_mxfp8_colwise"
    oq, osc = oracle.quantize_mxfp8(to64(x))
    assert np.array_equal(dq.cpu().numpy(), oq) and np.array_equal(ds.cpu().numpy(), osc)
    cq, cs, poff = oracle.quantize_mxfp8_colwise(to64(x), m, ld=ld)
    end = int(poff[-1])
    assert np.array_equal(tq[:, :end].cpu().numpy(), cq[:, :end])
    assert np.array_equal(ts[:, : end // 32].cpu().numpy(), cs[:, : end // 32])
