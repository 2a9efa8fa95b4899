"""GPU parity of launches whose last round of tiles is split over the contraction.

When a launch's tiles leave at least half the CUs idle in their last round, those
tail tiles are cut into contraction ranges; each range's fp32 partial goes to the
workspace and the last range to finish adds them in range order and stores the
tile.  These cases are sized from the device's CU count so that the split happens,
and check the split tiles against the oracle, the untouched tail of a caller
buffer, and that repeated launches (which reuse the workspace's arrival counters)
give bit-identical results.
"""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
from gl_testutil import TOL_BF16, assert_bits_equal, assert_close, nan_tail, to64

pytestmark = pytest.mark.gpu
DEV = "cuda"
TILE, STAGE, MIN_STAGES, SLOTS = 256, 64, 4, 256


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def parts_per_tile(tiles, max_items, nk):
    """How many contraction ranges the launch cuts each tail tile into (1: none);
    mirrors the grid sizing (one workgroup per CU, a multiple of 8) and the rule."""
    grid = min(cus(), max_items)
    grid = grid & ~7 if grid >= 8 else grid
    rem = tiles % grid
    if rem == 0:
        return 1
    s = grid // rem
    if s * rem > SLOTS:
        s = SLOTS // rem
    s = min(s, nk // MIN_STAGES)
    return s if s >= 2 else 1


def splits_for(row_tiles):
    """Five groups (one empty, two ragged) covering exactly `row_tiles` 256-row tiles."""
    a = row_tiles // 4
    c = row_tiles // 4 - 1
    d = row_tiles - 2 * a - (c + 1)
    m = np.array([TILE * a - 17, 0, TILE * a, TILE * c + 5, TILE * d - 100], dtype=np.int64)
    assert int(np.ceil(m / TILE).sum()) == row_tiles and (m >= 0).all()
    return m


def sample_rows(m, tail_tiles, seed=0):
    """Rows at every group's edges, random rows, and rows of the last tail_tiles row
    tiles (the split ones when each row tile is one tile)."""
    off = np.concatenate([[0], np.cumsum(m)])
    T = int(off[-1])
    rng = np.random.default_rng(seed)
    rows = set()
    for g in range(len(m)):
        if m[g]:
            rows.update(int(r) for r in (off[g], off[g] + 1, off[g + 1] - 2, off[g + 1] - 1) if off[g] <= r < off[g + 1])
    rows.update(int(r) for r in rng.integers(0, T, 24))
    # the last tail_tiles row tiles, counted per group from the end
    tiles = [(g, t) for g in range(len(m)) for t in range(int(np.ceil(m[g] / TILE)))]
    for g, t in tiles[-tail_tiles:]:
        lo = int(off[g]) + t * TILE
        hi = min(lo + TILE, int(off[g + 1]))
        rows.update((lo, hi - 1, int(rng.integers(lo, hi))))
    return np.array(sorted(rows), dtype=np.int64)


def make_workspace(m):
    ws = gl.new_workspace(len(m))
    gl.gl_offsets(torch.from_numpy(m).to(DEV), int(m.sum()), ws)
    assert gl.gl_read_status(ws) == 0
    return ws


def bf16(shape, std, gen):
    return (torch.randn(*shape, generator=gen) * std).to(torch.bfloat16)


def test_forward_split_tail_bias_caller_buffer_repeatable():
    K, N = 1024, 256                       # one tile column, 16 contraction stages
    row_tiles = cus() + cus() // 8
    m = splits_for(row_tiles)
    T, G = int(m.sum()), len(m)
    S = parts_per_tile(row_tiles, (int(np.ceil(T / TILE)) + G), K // STAGE)
    assert S >= 2, "the case must split its last round"
    say(f"forward split tail: T={T} tiles={row_tiles} parts={S}")
    gen = torch.Generator().manual_seed(11)
    x, w, b = bf16((T, K), 1.0, gen), bf16((G, N, K), 0.02, gen), bf16((G, N), 0.1, gen)
    xd, wd, bd = x.to(DEV), w.to(DEV), b.to(DEV)
    ws = make_workspace(m)
    y = nan_tail(T + 50, N, T, torch.bfloat16, DEV)
    tail = y[T:].clone()
    gl.gl_forward(xd, wd, y, ws, bias=bd)
    y2 = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    gl.gl_forward(xd, wd, y2, ws, bias=bd)
    torch.cuda.synchronize()
    assert_bits_equal(y[T:], tail, "caller buffer tail")
    assert_bits_equal(y[:T], y2, "second launch")
    rows = sample_rows(m, row_tiles % cus() or row_tiles)
    ref = oracle.forward(x.float().numpy(), to64(w), to64(b), m, rows=rows)
    assert_close(y[torch.from_numpy(rows).to(DEV)], ref, TOL_BF16, "y rows")


def test_dgrad_split_tail_caller_buffer_repeatable():
    K, N = 256, 1024                       # one tile column, 16 contraction stages
    row_tiles = cus() + cus() // 8
    m = splits_for(row_tiles)
    T, G = int(m.sum()), len(m)
    S = parts_per_tile(row_tiles, (int(np.ceil(T / TILE)) + G), N // STAGE)
    assert S >= 2, "the case must split its last round"
    say(f"dgrad split tail: T={T} tiles={row_tiles} parts={S}")
    gen = torch.Generator().manual_seed(12)
    dy, w = bf16((T, N), 1.0, gen), bf16((G, N, K), 0.02, gen)
    dyd, wd = dy.to(DEV), w.to(DEV)
    ws = make_workspace(m)
    dx = nan_tail(T + 9, K, T, torch.bfloat16, DEV)
    tail = dx[T:].clone()
    gl.gl_dgrad(dyd, wd, dx, ws)
    # a forward in between reuses the workspace's split counters
    gl.gl_forward(torch.zeros(T, N, dtype=torch.bfloat16, device=DEV),
                  torch.zeros(G, K, N, dtype=torch.bfloat16, device=DEV),
                  torch.empty(T, K, dtype=torch.bfloat16, device=DEV), ws)
    dx2 = torch.empty(T, K, dtype=torch.bfloat16, device=DEV)
    gl.gl_dgrad(dyd, wd, dx2, ws)
    torch.cuda.synchronize()
    assert_bits_equal(dx[T:], tail, "caller buffer tail")
    assert_bits_equal(dx[:T], dx2, "second launch")
    rows = sample_rows(m, row_tiles % cus() or row_tiles)
    ref = oracle.dgrad(dy.float().numpy(), to64(w), m, rows=rows)
    assert_close(dx[torch.from_numpy(rows).to(DEV)], ref, TOL_BF16, "dx rows")


def test_small_problem_split_every_tile():
    """Fewer tiles than half the CUs: every tile is split (forward and dgrad)."""
    m = np.array([100, 0, 1, 255, 200], dtype=np.int64)
    T, G, K, N = int(m.sum()), len(m), 2048, 2048
    row_tiles = int(np.ceil(m / TILE).sum())
    gen = torch.Generator().manual_seed(13)
    x, w, dy = bf16((T, K), 1.0, gen), bf16((G, N, K), 0.02, gen), bf16((T, N), 1.0, gen)
    tiles_j = N // TILE
    S = parts_per_tile(row_tiles * tiles_j, (int(np.ceil(T / TILE)) + G) * tiles_j, K // STAGE)
    assert S >= 2, "the case must split its tiles"
    say(f"small problem: tiles={row_tiles * tiles_j} parts={S}")
    xd, wd, dyd = x.to(DEV), w.to(DEV), dy.to(DEV)
    ws = make_workspace(m)
    y = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
    dx = torch.empty(T, K, dtype=torch.bfloat16, device=DEV)
    gl.gl_forward(xd, wd, y, ws)
    gl.gl_dgrad(dyd, wd, dx, ws)
    torch.cuda.synchronize()
    W = to64(w)
    assert_close(y, oracle.forward(x.float().numpy(), W, None, m), TOL_BF16, "y")
    assert_close(dx, oracle.dgrad(dy.float().numpy(), W, m), TOL_BF16, "dx")
