"""GPU tests of the fused split-offset scan + activation quantize launch and of the
cached MXFP8 weight workspace with its device no-op flag (page "Improve
device-init grouped linear module with single grouped weight support": in-place
group_quantize into a cached output, skipped through a noop_flag when a captured
graph is replayed).

Codes and scales are compared bit for bit with the separate entry points and with
the oracle's quantizer; the graph test replays a captured weight refresh + MXFP8
forward several times, with eager work and synchronisation between replays, and
checks every replay against the eager result.
"""
import sys

import numpy as np
import pytest
import torch

import grouped_gemm_gl_amd as gl
import oracle
from gl_testutil import assert_bits_equal

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16(shape, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * std).to(torch.bfloat16)


def table_bytes(G):
    """Header, offsets and the four row-tile prefix tables of a workspace."""
    return 32 + 8 * (G + 1) + 4 * 4 * (G + 1)


# the last case has more groups than the fused launch's scan workgroup has threads
MANY = np.random.default_rng(7).integers(0, 40, 600) * (np.arange(600) % 7 != 3)


@pytest.mark.parametrize("m", [[5, 0, 300, 17, 1], [0, 0, 64], [2048, 1, 0, 511, 1000, 3], MANY.tolist()])
def test_fused_offsets_quantize_matches_separate_calls(m):
    m = np.array(m, dtype=np.int64)
    G, T, K = len(m), int(m.sum()), 256
    say(f"fused offsets+quantize: m={m.tolist()}")
    x = bf16((T, K), 3.0, 1).to(DEV)
    md = torch.from_numpy(m).to(DEV)
    ws_a, ws_b = gl.new_workspace(G), gl.new_workspace(G)
    ws_a.fill_(0x5a)
    ws_b.fill_(0x5a)
    qa = torch.empty(T, K, dtype=torch.uint8, device=DEV)
    sa = torch.empty(T, K // 32, dtype=torch.uint8, device=DEV)
    qb, sb = torch.empty_like(qa), torch.empty_like(sa)
    gl.gl_offsets_quantize_mxfp8(md, x, ws_a, qa, sa)
    gl.gl_offsets(md, T, ws_b)
    gl.gl_group_quantize_mxfp8(x, qb, sb)
    torch.cuda.synchronize()
    nb = table_bytes(G)
    assert_bits_equal(ws_a[:nb], ws_b[:nb], "workspace tables")
    assert gl.gl_read_status(ws_a) == 0
    assert_bits_equal(qa, qb, "codes")
    assert_bits_equal(sa, sb, "scales")
    ref_q, ref_s = oracle.quantize_mxfp8(x.cpu().double().numpy())
    assert np.array_equal(qa.cpu().numpy(), ref_q) and np.array_equal(sa.cpu().numpy(), ref_s)


def test_fused_offsets_quantize_invalid_splits_sets_status():
    m = np.array([10, -3, 25], dtype=np.int64)
    T, K = 32, 64
    x = bf16((T, K), 1.0, 2).to(DEV)
    ws = gl.new_workspace(3)
    q = torch.zeros(T, K, dtype=torch.uint8, device=DEV)
    s = torch.zeros(T, K // 32, dtype=torch.uint8, device=DEV)
    gl.gl_offsets_quantize_mxfp8(torch.from_numpy(m).to(DEV), x, ws, q, s)
    assert gl.gl_read_status(ws) & gl.GL_STATUS_NEGATIVE_SPLIT
    # rowwise blocks do not depend on the splits: the codes are still written
    ref_q, ref_s = oracle.quantize_mxfp8(x.cpu().double().numpy())
    assert np.array_equal(q.cpu().numpy(), ref_q) and np.array_equal(s.cpu().numpy(), ref_s)


def test_fused_offsets_quantize_zero_rows():
    m = torch.zeros(4, dtype=torch.int64, device=DEV)
    ws = gl.new_workspace(4)
    x = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    gl.gl_offsets_quantize_mxfp8(m, x, ws, torch.empty(0, 64, dtype=torch.uint8, device=DEV),
                                 torch.empty(0, 2, dtype=torch.uint8, device=DEV))
    assert gl.gl_read_status(ws) == 0
    assert gl.workspace_offsets(ws, 4).cpu().tolist() == [0] * 5


def both_buffers(T, K, G, scale_offset=0):
    ld = gl.gl_colwise_ld(G, T)
    u8 = dict(dtype=torch.uint8, device=DEV)
    sbuf = torch.full((K * (ld // 32) + 8,), 0xAB, **u8)
    return (torch.empty(T, K, **u8), torch.empty(T, K // 32, **u8), torch.full((K, ld), 0xAB, **u8),
            sbuf[scale_offset:scale_offset + K * (ld // 32)].view(K, ld // 32))


@pytest.mark.parametrize("m,scale_offset", [([5, 0, 300, 17, 1], 0), ([2048, 1, 0, 511, 1000, 3], 0),
                                            (MANY.tolist(), 0), ([129, 0, 64], 1)])
def test_offsets_and_both_usages_in_one_pass(m, scale_offset):
    """The scan plus rowwise and columnwise codes of x: the workspace tables and both
    codes bit-equal to gl_offsets + gl_group_quantize_mxfp8 + the columnwise call (one
    launch below 64 groups with an aligned scale matrix, two launches otherwise)."""
    m = np.array(m, dtype=np.int64)
    G, T, K = len(m), int(m.sum()), 192
    say(f"offsets + both usages: G={G} T={T} scale_offset={scale_offset}")
    x = bf16((T, K), 2.0, 3).to(DEV)
    md = torch.from_numpy(m).to(DEV)
    ws_a, ws_b = gl.new_workspace(G), gl.new_workspace(G)
    ws_a.fill_(0x5a)
    ws_b.fill_(0x5a)
    qa, sa, ta, tsa = both_buffers(T, K, G, scale_offset)
    qb, sb, tb, tsb = both_buffers(T, K, G)
    gl.gl_offsets_quantize_mxfp8_rowwise_colwise(md, x, ws_a, qa, sa, ta, tsa)
    gl.gl_offsets(md, T, ws_b)
    gl.gl_group_quantize_mxfp8(x, qb, sb)
    gl.gl_group_quantize_mxfp8_colwise(x, tb, tsb, ws_b, G)
    torch.cuda.synchronize()
    nb = table_bytes(G)
    assert_bits_equal(ws_a[:nb], ws_b[:nb], "workspace tables")
    assert gl.gl_read_status(ws_a) == 0
    assert_bits_equal(qa, qb, "rowwise codes")
    assert_bits_equal(sa, sb, "rowwise scales")
    assert_bits_equal(ta, tb, "columnwise codes")
    assert_bits_equal(tsa, tsb, "columnwise scales")


def test_offsets_and_both_usages_invalid_and_empty():
    for m, bit in (([10, -3, 25], gl.GL_STATUS_NEGATIVE_SPLIT), ([0, 0, 0, 0], 0)):
        md = torch.tensor(m, dtype=torch.int64, device=DEV)
        T = 32 if bit else 0
        x = bf16((T, 64), 1.0, 4).to(DEV)
        ws = gl.new_workspace(len(m))
        gl.gl_offsets_quantize_mxfp8_rowwise_colwise(md, x, ws, *both_buffers(T, 64, len(m)))
        st = gl.gl_read_status(ws)
        assert (st & bit) if bit else st == 0
    assert gl.workspace_offsets(ws, 4).cpu().tolist() == [0] * 5


def weight_buffers(G, N, K):
    u8 = dict(dtype=torch.uint8, device=DEV)
    return (torch.empty(G, N, K, **u8), torch.empty(G, N, K // 32, **u8), torch.empty(G, K, N, **u8),
            torch.empty(G, K, N // 32, **u8))


def test_weight_workspace_matches_separate_quantizers_and_noop_skips():
    G, N, K = 3, 96, 160
    w = bf16((G, N, K), 0.05, 3).to(DEV)
    d, s, dt, st = weight_buffers(G, N, K)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    gl.gl_quantize_mxfp8_weights(w, d, s, dt, st, noop_flag=flag)
    rd, rs, rdt, rst = weight_buffers(G, N, K)
    gl.gl_group_quantize_mxfp8(w, rd, rs)
    gl.gl_quantize_mxfp8_colwise_weights(w, rdt, rst)
    torch.cuda.synchronize()
    for a, b, what in ((d, rd, "rowwise codes"), (s, rs, "rowwise scales"), (dt, rdt, "columnwise codes"),
                       (st, rst, "columnwise scales")):
        assert_bits_equal(a, b, what)
    # the oracle's rowwise quantizer on one group
    q1, s1 = oracle.quantize_mxfp8(w[1].cpu().double().numpy())
    assert np.array_equal(d[1].cpu().numpy(), q1) and np.array_equal(s[1].cpu().numpy(), s1)
    # flag set: new weights leave the workspace as it was; cleared: refreshed
    before = [t.clone() for t in (d, s, dt, st)]
    w.mul_(-2.0)
    flag.fill_(1)
    gl.gl_quantize_mxfp8_weights(w, d, s, dt, st, noop_flag=flag)
    torch.cuda.synchronize()
    for a, b in zip((d, s, dt, st), before):
        assert_bits_equal(a, b, "workspace under a set noop flag")
    flag.fill_(0)
    gl.gl_quantize_mxfp8_weights(w, d, s, dt, st, noop_flag=flag)
    gl.gl_group_quantize_mxfp8(w, rd, rs)
    torch.cuda.synchronize()
    assert_bits_equal(d, rd, "refreshed rowwise codes")
    assert_bits_equal(s, rs, "refreshed rowwise scales")
    # rowwise only (no columnwise buffers)
    d2, s2, _, _ = weight_buffers(G, N, K)
    gl.gl_quantize_mxfp8_weights(w, d2, s2)
    torch.cuda.synchronize()
    assert_bits_equal(d2, rd, "rowwise-only codes")


def test_graph_replay_of_weight_refresh_and_mxfp8_forward():
    G, N, K = 4, 256, 512
    m = torch.tensor([100, 0, 300, 57], dtype=torch.int64, device=DEV)
    T = int(m.sum())
    x = bf16((T, K), 1.0, 4).to(DEV)
    w1 = bf16((G, N, K), 0.02, 5).to(DEV)
    w2 = bf16((G, N, K), 0.02, 6).to(DEV)
    w = w1.clone()
    ws = gl.new_workspace(G)
    xq = torch.empty(T, K, dtype=torch.uint8, device=DEV)
    xs = torch.empty(T, K // 32, dtype=torch.uint8, device=DEV)
    gl.gl_offsets_quantize_mxfp8(m, x, ws, xq, xs)
    d, s, _, _ = weight_buffers(G, N, K)
    flag = torch.zeros(1, dtype=torch.int32, device=DEV)
    y = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)

    def eager(wsrc):
        dd, ss, _, _ = weight_buffers(G, N, K)
        gl.gl_quantize_mxfp8_weights(wsrc, dd, ss)
        out = torch.empty(T, N, dtype=torch.bfloat16, device=DEV)
        gl.gl_forward(xq, dd, out, ws, x_scale=xs, w_scale=ss)
        torch.cuda.synchronize()
        return out

    ref1, ref2 = eager(w1), eager(w2)
    assert not torch.equal(ref1, ref2)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        # one eager pass on the capture stream first (warm-up, as graph capture expects)
        gl.gl_quantize_mxfp8_weights(w, d, s, noop_flag=flag)
        gl.gl_forward(xq, d, y, ws, x_scale=xs, w_scale=s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        gl.gl_quantize_mxfp8_weights(w, d, s, noop_flag=flag)
        gl.gl_forward(xq, d, y, ws, x_scale=xs, w_scale=s)
    steps = [(w1, 0, ref1), (w2, 1, ref1), (w2, 1, ref1), (w2, 0, ref2), (w1, 1, ref2), (w1, 0, ref1)]
    for i, (wsrc, f, ref) in enumerate(steps):
        say(f"replay {i}: noop={f}")
        w.copy_(wsrc)
        flag.fill_(f)
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_bits_equal(y, ref, f"replay {i} (noop flag {f})")
