"""The deferred-wgrad queue on the host (no GPU: a put checks its arguments and
records the call without launching or reading device memory; only empty queues are
run here).  The queue follows the layer's delayed weight-gradient store (page
"transformer_engine/pytorch/ops/basic/grouped_linear.py", delay_wgrad_compute and
backward_dw: the backward stores its wgrad call, a later call runs the oldest)."""
import ctypes
import os

import pytest
import torch

import grouped_gemm_gl_amd as gl

pytestmark = pytest.mark.skipif(not os.path.exists(gl.library_path), reason="library not built")

FAKE = 0x100000  # aligned, never dereferenced
FAKE2 = 0x200000


def new_queue():
    q = ctypes.c_void_p()
    assert gl.load().gl_wgrad_queue_create(ctypes.byref(q)) == 0 and q.value
    return q


def put(q, G=4, K=64, N=32, T=100, ind=gl.GL_BF16, outd=gl.GL_BF16, dbd=gl.GL_BF16, x=FAKE, dy=FAKE2, dw=FAKE,
        dwp=None, acc=0, db=None, dbp=None, ws=FAKE):
    return gl.load().gl_wgrad_queue_put(q, G, K, N, T, ind, outd, dbd, x, dy, dw, dwp, acc, db, dbp, ws)


def put_mx(q, G=2, K=64, N=64, T=100, outd=gl.GL_BF16, ld=None, dw=FAKE, ws=FAKE):
    lib = gl.load()
    ld = lib.gl_colwise_ld(G, T) if ld is None else ld
    return lib.gl_wgrad_queue_put_mxfp8(q, G, K, N, T, outd, FAKE, FAKE2, FAKE, FAKE2, ld, dw, None, 0, ws)


def test_put_counts_and_clear():
    lib = gl.load()
    q = new_queue()
    try:
        assert lib.gl_wgrad_queue_size(q) == 0
        assert put(q) == 0
        assert put(q, db=FAKE) == 0
        assert put(q, ind=gl.GL_F32, outd=gl.GL_F32, acc=1) == 0
        assert put_mx(q) == 0
        assert lib.gl_wgrad_queue_size(q) == 4
        assert lib.gl_wgrad_queue_clear(q) == 0
        assert lib.gl_wgrad_queue_size(q) == 0
        # running an empty queue launches nothing and succeeds
        assert lib.gl_wgrad_queue_run_next(q, None) == 0
        assert lib.gl_wgrad_queue_flush(q, None) == 0
    finally:
        assert lib.gl_wgrad_queue_destroy(q) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(G=0), -1), (dict(T=-1), -1), (dict(K=60), -3),
    (dict(dw=None), -1), (dict(dwp=FAKE), -1),            # neither / both dW forms
    (dict(x=None), -1), (dict(x=FAKE + 4), -1),
    (dict(acc=2), -1), (dict(ws=None), -1),
    (dict(outd=gl.GL_F16), -2),                          # bf16 in, fp16 out
    (dict(db=FAKE, dbd=gl.GL_F16), -2),                  # bias grad fp32 or the input type
    (dict(db=FAKE, dbp=FAKE), -1),
])
def test_put_rejects_and_queues_nothing(kw, code):
    lib = gl.load()
    q = new_queue()
    try:
        assert put(q) == 0
        assert put(q, **kw) == code
        assert lib.gl_last_error()
        assert lib.gl_wgrad_queue_size(q) == 1
    finally:
        lib.gl_wgrad_queue_destroy(q)


@pytest.mark.parametrize("kw,code", [(dict(K=60), -3), (dict(ld=96), -3), (dict(outd=gl.GL_F16), -2),
                                     (dict(dw=None), -1), (dict(ws=None), -1)])
def test_put_mxfp8_rejects(kw, code):
    lib = gl.load()
    q = new_queue()
    try:
        assert put_mx(q, **kw) == code
        assert lib.gl_wgrad_queue_size(q) == 0
    finally:
        lib.gl_wgrad_queue_destroy(q)


def test_null_queue():
    lib = gl.load()
    assert lib.gl_wgrad_queue_create(None) == -1
    assert lib.gl_wgrad_queue_size(None) == -1
    assert lib.gl_wgrad_queue_run_next(None, None) == -1
    assert lib.gl_wgrad_queue_flush(None, None) == -1
    assert lib.gl_wgrad_queue_clear(None) == -1
    assert put(None) == -1
    assert lib.gl_wgrad_queue_destroy(None) == 0


def test_python_queue_marshalling():
    """The binding's queue records what it puts and drops it on clear (host tensors
    stand in for device ones: nothing runs)."""
    q = gl.WgradQueue()
    G, K, N, T = 3, 64, 32, 10
    x, dy = torch.zeros(T, K, dtype=torch.bfloat16), torch.zeros(T, N, dtype=torch.bfloat16)
    dw, db = torch.zeros(G, N, K, dtype=torch.bfloat16), torch.zeros(G, N, dtype=torch.float32)
    ws = torch.zeros(4096, dtype=torch.uint8)
    q.put(x, dy, dw, ws)
    q.put(x, dy, dw, ws, db=db)
    assert len(q) == 2
    with pytest.raises(gl.GLError):
        q.put(x, dy, dw, torch.zeros(0, dtype=torch.uint8))  # no workspace
    with pytest.raises(ValueError):
        q.put(x, dy[:5], dw, ws)
    assert len(q) == 2
    q.clear()
    assert len(q) == 0
    q.close()
