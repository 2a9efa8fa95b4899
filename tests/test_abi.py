"""The C ABI: the built library loads, exports every entry point the header
declares, and rejects bad arguments on the host (no GPU needed: each call below
fails validation before anything is enqueued, so no pointer is dereferenced)."""
import ctypes
import os
import re

import pytest

import grouped_gemm_gl_amd as gl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grouped_linear.h")

pytestmark = pytest.mark.skipif(not os.path.exists(gl.library_path), reason="library not built")

FAKE = 0x100000  # aligned, never dereferenced: validation fails first
FAKE2 = 0x200000


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gl_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_symbols()
    for n in ["gl_offsets", "gl_forward", "gl_dgrad", "gl_wgrad", "gl_bgrad", "gl_group_quantize_mxfp8",
              "gl_workspace_size", "gl_last_error", "gl_read_status"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gl.library_path)
    missing = [n for n in declared_symbols() if not hasattr(lib, n)]
    assert not missing


def test_binding_covers_every_declared_entry_point():
    """Every C entry point has a Python function of the same name (the deferred-wgrad
    queue's calls are the methods of WgradQueue; the error and workspace-pointer
    helpers are used inside the binding)."""
    internal = {"gl_last_error", "gl_workspace_offsets"}
    names = [n for n in declared_symbols() if not n.startswith("gl_wgrad_queue_") and n not in internal]
    assert not [n for n in names if n not in gl.__all__ or not callable(getattr(gl, n, None))]
    for m in ["put", "put_mxfp8", "run_next", "flush", "clear", "close", "__len__"]:
        assert callable(getattr(gl.WgradQueue, m))
    lib = gl.load()
    assert not [n for n in declared_symbols() if getattr(lib, n).argtypes is None], "entry point without a signature"


def test_version_and_workspace_size():
    lib = gl.load()
    assert b"gfx950" in lib.gl_version()
    assert gl.gl_workspace_size(0) == 0
    for G in (1, 4, 256, 1000):
        sz = gl.gl_workspace_size(G)
        assert sz % 256 == 0
        assert sz >= 32 + 8 * (G + 1) + 4 * 4 * (G + 1)


def fwd(G=4, K=64, N=32, T=32, ind=gl.GL_BF16, outd=gl.GL_BF16, x=FAKE, xs=None, w=FAKE, wp=None, ws_=None,
        wsp=None, b=None, bp=None, y=FAKE2, y_rows=None, ws=FAKE):
    lib = gl.load()
    return lib.gl_forward(G, K, N, T, ind, outd, x, xs, w, wp, ws_, wsp, b, bp, y, T if y_rows is None else y_rows,
                          ws, None)


@pytest.mark.parametrize("kw,code", [
    (dict(G=0), -1), (dict(K=0), -1), (dict(N=-3), -1), (dict(T=-1), -1),
    (dict(y_rows=31), -3),                          # caller buffer too small
    (dict(w=None), -1), (dict(wp=FAKE), -1),        # neither / both weight forms
    (dict(b=FAKE, bp=FAKE), -1),
    (dict(x=FAKE + 8), -1),                         # misaligned
    (dict(ind=gl.GL_F16, outd=gl.GL_BF16), -2),     # fp16 in, bf16 out
    (dict(ind=gl.GL_BF16, outd=gl.GL_F32), -2),
    (dict(ind=7, outd=7), -2),
    (dict(K=60), -3), (dict(N=36), -3),             # bf16 rows must be 16-byte multiples
    (dict(K=(1 << 22) + 8), -3), (dict(N=(1 << 22) + 8), -3),  # bf16 rows above 2^22 elements
    (dict(ind=gl.GL_E4M3, outd=gl.GL_BF16, K=96), -3),
    (dict(ind=gl.GL_E4M3, outd=gl.GL_BF16, K=128, xs=None), -1),
    (dict(ind=gl.GL_E4M3, outd=gl.GL_E4M3, K=128, xs=FAKE), -2),
    (dict(ind=gl.GL_E4M3, outd=gl.GL_BF16, K=(1 << 22) + 128, xs=FAKE), -3),  # MXFP8 rows above 2^22 codes
    (dict(ws=None), -1),
])
def test_forward_rejects(kw, code):
    assert fwd(**kw) == code
    assert gl.load().gl_last_error()


def test_other_entry_points_reject():
    lib = gl.load()
    assert lib.gl_offsets(None, 4, 32, FAKE, None) == -1
    assert lib.gl_offsets(FAKE, 0, 32, FAKE, None) == -1
    assert lib.gl_offsets(FAKE, 4, -1, FAKE, None) == -1
    assert lib.gl_offsets(FAKE, 4, 32, FAKE + 4, None) == -1
    assert lib.gl_dgrad(4, 64, 32, 32, gl.GL_BF16, FAKE, FAKE, None, FAKE2, 16, FAKE, None) == -3
    assert lib.gl_dgrad(4, 64, 32, 32, 7, FAKE, FAKE, None, FAKE2, 32, FAKE, None) == -2
    assert lib.gl_wgrad(4, 64, 32, 32, gl.GL_F16, gl.GL_BF16, FAKE, FAKE, FAKE2, None, 0, FAKE, None) == -2
    assert lib.gl_wgrad(4, 64, 32, 32, gl.GL_F32, gl.GL_BF16, FAKE, FAKE, FAKE2, None, 0, FAKE, None) == -2
    assert lib.gl_wgrad(4, 64, 32, 32, gl.GL_BF16, gl.GL_F32, FAKE, FAKE, None, None, 0, FAKE, None) == -1
    assert lib.gl_wgrad(4, 64, 32, 32, gl.GL_BF16, gl.GL_F32, FAKE, FAKE, FAKE2, None, 2, FAKE, None) == -1
    assert lib.gl_bgrad(4, 36, 32, gl.GL_BF16, FAKE, FAKE2, None, FAKE, None) == -3
    assert lib.gl_bgrad(4, 32, 32, gl.GL_BF16, FAKE, FAKE2, FAKE2, FAKE, None) == -1
    assert lib.gl_group_quantize_mxfp8(FAKE, 4, 48, FAKE2, FAKE2, None) == -3
    assert lib.gl_group_quantize_mxfp8(FAKE, -1, 64, FAKE2, FAKE2, None) == -1
    assert lib.gl_group_quantize_mxfp8(FAKE + 2, 4, 64, FAKE2, FAKE2, None) == -1
    assert lib.gl_read_status(None, None, None) == -1
    # MXFP8 backward: layout and shape rules
    ld = lib.gl_colwise_ld(4, 1000)
    assert ld == 1536 and lib.gl_colwise_ld(0, 10) == -1
    assert lib.gl_group_quantize_mxfp8_colwise(FAKE, 64, 4, 1000, FAKE, FAKE2, FAKE2, ld - 128, None) == -3
    assert lib.gl_group_quantize_mxfp8_colwise(FAKE, 64, 4, 1000, FAKE, FAKE2, FAKE2, ld + 64, None) == -3
    assert lib.gl_group_quantize_mxfp8_colwise(FAKE, 64, 4, 1000, None, FAKE2, FAKE2, ld, None) == -1
    assert lib.gl_quantize_mxfp8_colwise_weights(FAKE, 2, 48, 64, FAKE2, FAKE2, None) == -3
    rc = lib.gl_group_quantize_mxfp8_rowwise_colwise
    assert rc(FAKE, 48, 4, 1000, FAKE, FAKE2, FAKE2, FAKE2, FAKE2, ld, None) == -3       # cols % 32
    assert rc(FAKE, 64, 4, 1000, FAKE, FAKE2, FAKE2, FAKE2, FAKE2, ld - 128, None) == -3  # ld too short
    assert rc(FAKE, 64, 4, 1000, FAKE, None, FAKE2, FAKE2, FAKE2, ld, None) == -1         # a buffer missing
    assert rc(FAKE + 8, 64, 4, 1000, FAKE, FAKE2, FAKE2, FAKE2, FAKE2, ld, None) == -1    # misaligned src
    assert lib.gl_dgrad_mxfp8(4, 64, 192, 32, gl.GL_BF16, FAKE, FAKE, FAKE, FAKE, FAKE2, 32, FAKE, None) == -3
    assert lib.gl_dgrad_mxfp8(4, 64, 256, 32, gl.GL_E4M3, FAKE, FAKE, FAKE, FAKE, FAKE2, 32, FAKE, None) == -2
    assert lib.gl_dgrad_mxfp8(4, 64, 256, 32, gl.GL_BF16, FAKE, FAKE, FAKE, FAKE, FAKE2, 16, FAKE, None) == -3
    assert lib.gl_dgrad_mxfp8(4, 64, (1 << 22) + 128, 32, gl.GL_BF16, FAKE, FAKE, FAKE, FAKE, FAKE2, 32, FAKE,
                              None) == -3
    assert lib.gl_wgrad_mxfp8(4, 64, 32, 1000, gl.GL_F32, FAKE, FAKE, FAKE, FAKE, ld - 128, FAKE2, None, 1, FAKE,
                              None) == -3
    assert lib.gl_wgrad_mxfp8(4, 64, 32, 1000, gl.GL_F32, FAKE, FAKE, FAKE, FAKE, ld, FAKE2, FAKE2, 1, FAKE,
                              None) == -1
    # wgrad + bias grad in one call
    assert lib.gl_wgrad_bgrad(4, 64, 32, 32, gl.GL_BF16, gl.GL_BF16, gl.GL_F16, FAKE, FAKE, FAKE2, None, 0,
                              FAKE2, None, FAKE, None) == -2
    assert lib.gl_wgrad_bgrad(4, 64, 32, 32, gl.GL_BF16, gl.GL_BF16, gl.GL_BF16, FAKE, FAKE, FAKE2, None, 0,
                              None, None, FAKE, None) == -1
    assert lib.gl_wgrad_bgrad(4, 64, 32, 32, gl.GL_BF16, gl.GL_BF16, gl.GL_F32, FAKE, FAKE, FAKE2, None, 0,
                              FAKE2, FAKE2, FAKE, None) == -1
    assert lib.gl_wgrad_bgrad(4, 64, 30, 32, gl.GL_F32, gl.GL_F32, gl.GL_F32, FAKE, FAKE, FAKE2, None, 0,
                              FAKE2, None, FAKE, None) == -3
    # SwiGLU and the grouped MLP
    assert lib.gl_swiglu_forward(32, 12, gl.GL_BF16, FAKE, FAKE2, None) == -3
    assert lib.gl_swiglu_forward(32, 16, 7, FAKE, FAKE2, None) == -2
    assert lib.gl_swiglu_backward(32, 16, gl.GL_BF16, FAKE, None, FAKE2, None) == -1
    assert lib.gl_swiglu_backward(32, 16, gl.GL_BF16, FAKE, FAKE + 8, FAKE2, None) == -1
    mlp_f = lambda **k: lib.gl_grouped_mlp_forward(
        4, 64, k.get("F", 32), 48, 32, gl.GL_BF16, FAKE, FAKE, k.get("w1p"), None, None, FAKE, None, None, None,
        FAKE2, FAKE2, FAKE2, k.get("y_rows", 32), FAKE, None)
    assert mlp_f(F=36) == -3                         # F % 8
    assert mlp_f(w1p=FAKE) == -1                     # both weight forms for FC1
    assert mlp_f(y_rows=31) == -3                    # output buffer too small
    mlp_b = lambda **k: lib.gl_grouped_mlp_backward(
        4, 64, 32, 48, 32, gl.GL_BF16, k.get("wd", gl.GL_F32), FAKE, FAKE, None, FAKE, None, FAKE, FAKE, FAKE,
        FAKE2, FAKE2, FAKE2, k.get("dx_rows", 32), FAKE2, None, None, None, FAKE2, None, k.get("db2"), k.get("db2p"),
        0, FAKE, None)
    assert mlp_b(wd=gl.GL_F16) == -2                  # wgrad dtype neither fp32 nor the input's
    assert mlp_b(dx_rows=16) == -3
    assert mlp_b(db2=FAKE2, db2p=FAKE2) == -1         # both bias-grad forms
    # fused offsets + activation quantize
    assert lib.gl_offsets_quantize_mxfp8(FAKE, 0, 32, FAKE, FAKE, 64, FAKE2, FAKE2, None) == -1
    assert lib.gl_offsets_quantize_mxfp8(FAKE, 4, 32, FAKE, FAKE, 48, FAKE2, FAKE2, None) == -3
    assert lib.gl_offsets_quantize_mxfp8(FAKE + 4, 4, 32, FAKE, FAKE, 64, FAKE2, FAKE2, None) == -1
    assert lib.gl_offsets_quantize_mxfp8(FAKE, 4, 32, FAKE, None, 64, FAKE2, FAKE2, None) == -1
    assert lib.gl_offsets_quantize_mxfp8(FAKE, 4, 32, FAKE, FAKE + 8, 64, FAKE2, FAKE2, None) == -1
    # cached weight workspace
    assert lib.gl_quantize_mxfp8_weights(FAKE, 2, 64, 48, FAKE2, FAKE2, None, None, None, None) == -3
    assert lib.gl_quantize_mxfp8_weights(FAKE, 2, 64, 64, FAKE2, FAKE2, FAKE2, None, None, None) == -1
    assert lib.gl_quantize_mxfp8_weights(FAKE, 2, 48, 64, FAKE2, FAKE2, FAKE2, FAKE2, None, None) == -3
    assert lib.gl_quantize_mxfp8_weights(FAKE, 2, 64, 64, FAKE2, FAKE2, None, None, FAKE + 2, None) == -1
    assert lib.gl_quantize_mxfp8_weights(FAKE, 0, 64, 64, FAKE2, FAKE2, None, None, None, None) == -1


def test_zero_rows_is_a_no_op_without_device_work():
    # nothing to compute and nothing to write: returns OK without touching pointers
    assert fwd(T=0, x=None, y=None) == 0
    assert gl.load().gl_group_quantize_mxfp8(None, 0, 64, None, None, None) == 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(gl, "_lib", None)
    monkeypatch.setattr(gl, "library_path", "/nonexistent/libgrouped_linear.so")
    with pytest.raises(RuntimeError, match="not built"):
        gl.load()


def test_forward_noalloc_rejects_before_any_device_work():
    """The allocation-free forward checks everything gl_forward checks, plus its own
    group bound and the split-size pointer, before it looks up its device array."""
    lib = gl.load()
    args = lambda G=4, K=64, N=32, T=16, m=FAKE, x=FAKE2, y=FAKE2, yr=16: (
        G, K, N, T, gl.GL_BF16, gl.GL_BF16, m, x, None, FAKE, None, None, None, None, None, y, yr, None)
    assert lib.gl_forward_noalloc(*args(G=gl.NOALLOC_MAX_GROUPS + 1)) == -3
    assert b"maximum" in lib.gl_last_error()
    assert lib.gl_forward_noalloc(*args(G=0)) == -1
    assert lib.gl_forward_noalloc(*args(m=None)) == -1
    assert lib.gl_forward_noalloc(*args(m=FAKE + 4)) == -1
    assert lib.gl_forward_noalloc(*args(K=0)) == -1
    assert lib.gl_forward_noalloc(*args(yr=15)) == -3          # output capacity below T
    assert lib.gl_forward_noalloc(*args(K=60)) == -3           # bf16 rows of 16-byte multiples
    assert lib.gl_forward_noalloc(*args(T=0, x=None, y=None)) == 0  # nothing to do
    assert lib.gl_forward_noalloc(*args(G=gl.NOALLOC_MAX_GROUPS, T=0, x=None, y=None)) == 0
