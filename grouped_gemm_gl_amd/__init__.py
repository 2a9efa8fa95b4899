"""Python binding of the gfx950 grouped-linear library ``libgrouped_linear.so``.

Argument marshalling only: each function takes torch tensors (device memory),
checks that their shapes, dtypes and devices agree with one another, and passes
their addresses plus the current HIP stream to the C entry point of the same name
(declared in ``include/grouped_linear.h``).  Every step of the computation runs in
the library's HIP kernels; nothing here computes, and there is no fallback: if the
library is not built, importing works but the first call raises.

Weights, biases and weight gradients are accepted stacked (one tensor with a
leading group dimension) or per group (a list of tensors); for a list, a device
array of their addresses is built and handed over.
"""
from __future__ import annotations

import collections
import ctypes
import os
from typing import Optional, Sequence, Union

import torch

__all__ = [
    "GL_F32", "GL_BF16", "GL_F16", "GL_E4M3", "GLError", "library_path", "load", "gl_version",
    "gl_workspace_size", "new_workspace", "workspace_offsets", "gl_offsets", "gl_read_status",
    "gl_forward", "gl_dgrad", "gl_wgrad", "gl_wgrad_bgrad", "gl_bgrad",
    "gl_group_quantize_mxfp8", "gl_colwise_ld", "gl_group_quantize_mxfp8_colwise",
    "gl_group_quantize_mxfp8_rowwise_colwise", "gl_quantize_mxfp8_colwise_weights",
    "gl_offsets_quantize_mxfp8", "gl_offsets_quantize_mxfp8_rowwise_colwise", "gl_quantize_mxfp8_weights",
    "gl_dgrad_mxfp8", "gl_wgrad_mxfp8", "gl_swiglu_forward", "gl_swiglu_backward",
    "gl_grouped_mlp_forward", "gl_grouped_mlp_backward", "WgradQueue", "gl_forward_noalloc",
    "NOALLOC_MAX_GROUPS",
]

GL_F32, GL_BF16, GL_F16, GL_E4M3 = 0, 1, 2, 3
NOALLOC_MAX_GROUPS = 16384  # GL_NOALLOC_MAX_GROUPS
GL_STATUS_NEGATIVE_SPLIT, GL_STATUS_SUM_MISMATCH, GL_STATUS_WORKSPACE = 1, 2, 4

_HERE = os.path.dirname(os.path.abspath(__file__))
# GL_LIBRARY_PATH selects another build of the same library (e.g. the host-sanitized one)
library_path = os.environ.get("GL_LIBRARY_PATH") or os.path.join(_HERE, "libgrouped_linear.so")
_lib = None

Tensor = torch.Tensor
Grouped = Union[Tensor, Sequence[Tensor]]


class GLError(RuntimeError):
    """A non-zero return code of the C library, with its message."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def load():
    """Load the shared library (once); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise RuntimeError(f"{library_path} is not built; run `python -m grouped_gemm_gl_amd.build`")
    lib = ctypes.CDLL(library_path)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    sig = {
        "gl_workspace_size": (ctypes.c_size_t, [I]),
        "gl_workspace_offsets": (P, [P]),
        "gl_offsets": (I, [P, I, I64, P, P]),
        "gl_read_status": (I, [P, ctypes.POINTER(ctypes.c_int), P]),
        "gl_forward": (I, [I, I64, I64, I64, I, I, P, P, P, P, P, P, P, P, P, I64, P, P]),
        "gl_dgrad": (I, [I, I64, I64, I64, I, P, P, P, P, I64, P, P]),
        "gl_wgrad": (I, [I, I64, I64, I64, I, I, P, P, P, P, I, P, P]),
        "gl_wgrad_bgrad": (I, [I, I64, I64, I64, I, I, I, P, P, P, P, I, P, P, P, P]),
        "gl_bgrad": (I, [I, I64, I64, I, P, P, P, P, P]),
        "gl_group_quantize_mxfp8": (I, [P, I64, I64, P, P, P]),
        "gl_colwise_ld": (I64, [I, I64]),
        "gl_group_quantize_mxfp8_colwise": (I, [P, I64, I, I64, P, P, P, I64, P]),
        "gl_quantize_mxfp8_colwise_weights": (I, [P, I, I64, I64, P, P, P]),
        "gl_group_quantize_mxfp8_rowwise_colwise": (I, [P, I64, I, I64, P, P, P, P, P, I64, P]),
        "gl_offsets_quantize_mxfp8": (I, [P, I, I64, P, P, I64, P, P, P]),
        "gl_offsets_quantize_mxfp8_rowwise_colwise": (I, [P, I, I64, P, P, I64, P, P, P, P, I64, P]),
        "gl_swiglu_forward": (I, [I64, I64, I, P, P, P]),
        "gl_swiglu_backward": (I, [I64, I64, I, P, P, P, P]),
        "gl_grouped_mlp_forward": (I, [I, I64, I64, I64, I64, I] + [P] * 12 + [I64, P, P]),
        "gl_grouped_mlp_backward": (I, [I, I64, I64, I64, I64, I, I] + [P] * 11 + [I64] + [P] * 8 + [I, P, P]),
        "gl_quantize_mxfp8_weights": (I, [P, I, I64, I64, P, P, P, P, P, P]),
        "gl_dgrad_mxfp8": (I, [I, I64, I64, I64, I, P, P, P, P, P, I64, P, P]),
        "gl_wgrad_mxfp8": (I, [I, I64, I64, I64, I, P, P, P, P, I64, P, P, I, P, P]),
        "gl_wgrad_queue_create": (I, [ctypes.POINTER(P)]),
        "gl_wgrad_queue_destroy": (I, [P]),
        "gl_wgrad_queue_put": (I, [P, I, I64, I64, I64, I, I, I, P, P, P, P, I, P, P, P]),
        "gl_wgrad_queue_put_mxfp8": (I, [P, I, I64, I64, I64, I, P, P, P, P, I64, P, P, I, P]),
        "gl_wgrad_queue_size": (I, [P]),
        "gl_wgrad_queue_run_next": (I, [P, P]),
        "gl_wgrad_queue_flush": (I, [P, P]),
        "gl_wgrad_queue_clear": (I, [P]),
        "gl_forward_noalloc": (I, [I, I64, I64, I64, I, I] + [P] * 10 + [I64, P]),
        "gl_last_error": (ctypes.c_char_p, []),
        "gl_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype, fn.argtypes = res, args
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise GLError(rc, load().gl_last_error().decode())


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t: Optional[Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr() if t.numel() else None


_DT = {torch.float32: GL_F32, torch.bfloat16: GL_BF16, torch.float16: GL_F16, torch.uint8: GL_E4M3}


def _dtype(t: Tensor) -> int:
    if t.dtype not in _DT:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _record(tensors, stream):
    """Ties tensors' memory to a caller-given stream: torch's caching allocator
    then waits for the work queued on that stream before it reuses the memory
    (without it, a pointer array freed right after an enqueue on another stream
    could be handed out again before the kernel has read it)."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(_stream(stream))
    for t in tensors:
        if isinstance(t, Tensor) and t.is_cuda:
            t.record_stream(s)


def _grouped(g: Optional[Grouped], device, stream=None):
    """(stacked pointer, pointer-array pointer, keep-alive) for a stacked tensor or a
    list; the device pointer array of a list is tied to ``stream`` (see _record)."""
    if g is None:
        return None, None, None
    if isinstance(g, Tensor):
        return _ptr(g), None, None
    ptrs = torch.tensor([_ptr(t) or 0 for t in g], dtype=torch.int64, device=device)
    _record([ptrs], stream)
    return None, ptrs.data_ptr(), (ptrs, list(g))


def _first(g: Grouped) -> Tensor:
    return g[0] if not isinstance(g, Tensor) or g.dim() == 3 else g


def gl_version() -> str:
    return load().gl_version().decode()


def gl_workspace_size(num_groups: int) -> int:
    return int(load().gl_workspace_size(num_groups))


def new_workspace(num_groups: int, device="cuda") -> Tensor:
    """Device buffer sized for a call sequence over ``num_groups`` groups."""
    return torch.empty(gl_workspace_size(num_groups), dtype=torch.uint8, device=device)


def gl_offsets(m_splits: Tensor, total_rows: int, workspace: Tensor, stream=None) -> None:
    """Split-offset scan of the device int64 split sizes into ``workspace``."""
    if m_splits.dtype != torch.int64:
        raise ValueError("m_splits must be int64")
    _check(load().gl_offsets(_ptr(m_splits), m_splits.numel(), int(total_rows), _ptr(workspace), _stream(stream)))


def workspace_offsets(workspace: Tensor, num_groups: int) -> Tensor:
    """The int64[G+1] offsets inside a workspace, as a view (no device work); the
    library names where they sit (gl_workspace_offsets)."""
    start = int(load().gl_workspace_offsets(_ptr(workspace))) - workspace.data_ptr()
    return workspace[start: start + 8 * (num_groups + 1)].view(torch.int64)


def gl_read_status(workspace: Tensor, stream=None) -> int:
    """Synchronise the stream and return the workspace status word (0 = valid splits)."""
    st = ctypes.c_int(0)
    _check(load().gl_read_status(_ptr(workspace), ctypes.byref(st), _stream(stream)))
    return st.value


def gl_forward(x: Tensor, w: Grouped, y: Tensor, workspace: Tensor, *, bias: Optional[Grouped] = None,
               x_scale: Optional[Tensor] = None, w_scale: Optional[Grouped] = None, stream=None) -> Tensor:
    """y[:T] = grouped x W_g^T (+ b_g); T = x.shape[0]; rows of y past T are left untouched.

    x: [T, K] float32 / bfloat16, or uint8 E4M3 codes with ``x_scale`` [T, K/32];
    w: [G, N, K] or G tensors [N, K] (uint8 with ``w_scale`` for MXFP8);
    y: [>= T, N] (float32 / bfloat16; for MXFP8 its dtype picks the output type).
    """
    G = w.shape[0] if isinstance(w, Tensor) else len(w)
    w0 = _first(w)
    N, K = w0.shape[-2], w0.shape[-1]
    T = x.shape[0]
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [T, {K}], got {tuple(x.shape)}")
    if y.dim() != 2 or y.shape[1] != N:
        raise ValueError(f"y must be [rows >= {T}, {N}], got {tuple(y.shape)}")
    if w0.dtype != x.dtype:
        raise ValueError("x and w must have the same dtype")
    if bias is not None and _first(bias).dtype != y.dtype:
        raise ValueError("bias dtype must equal the output dtype")
    dev = x.device
    wp, wpp, keep_w = _grouped(w, dev, stream)
    bp, bpp, keep_b = _grouped(bias, dev, stream)
    sp, spp, keep_s = _grouped(w_scale, dev, stream)
    _check(load().gl_forward(G, K, N, T, _dtype(x), _dtype(y), _ptr(x), _ptr(x_scale), wp, wpp, sp, spp, bp, bpp,
                             _ptr(y), y.shape[0], _ptr(workspace), _stream(stream)))
    del keep_w, keep_b, keep_s
    return y


def gl_forward_noalloc(m_splits: Tensor, x: Tensor, w: Grouped, y: Tensor, *, bias: Optional[Grouped] = None,
                       x_scale: Optional[Tensor] = None, w_scale: Optional[Grouped] = None, stream=None) -> Tensor:
    """gl_offsets + gl_forward with the library's own fixed device scratch in place of a
    workspace (the C call allocates nothing; the per-group pointer form of ``w`` builds
    its pointer array here, so callers that must not allocate pass stacked tensors).
    At most NOALLOC_MAX_GROUPS groups; calls that overlap on one device race."""
    G = w.shape[0] if isinstance(w, Tensor) else len(w)
    w0 = _first(w)
    N, K = w0.shape[-2], w0.shape[-1]
    T = x.shape[0]
    if m_splits.dtype != torch.int64 or m_splits.numel() != G:
        raise ValueError(f"m_splits must be int64 with {G} entries")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError(f"x must be [T, {K}], got {tuple(x.shape)}")
    if y.dim() != 2 or y.shape[1] != N:
        raise ValueError(f"y must be [rows >= {T}, {N}], got {tuple(y.shape)}")
    if w0.dtype != x.dtype:
        raise ValueError("x and w must have the same dtype")
    if bias is not None and _first(bias).dtype != y.dtype:
        raise ValueError("bias dtype must equal the output dtype")
    dev = x.device
    wp, wpp, keep_w = _grouped(w, dev, stream)
    bp, bpp, keep_b = _grouped(bias, dev, stream)
    sp, spp, keep_s = _grouped(w_scale, dev, stream)
    _check(load().gl_forward_noalloc(G, K, N, T, _dtype(x), _dtype(y), _ptr(m_splits), _ptr(x), _ptr(x_scale), wp,
                                     wpp, sp, spp, bp, bpp, _ptr(y), y.shape[0], _stream(stream)))
    del keep_w, keep_b, keep_s
    return y


def gl_dgrad(dy: Tensor, w: Grouped, dx: Tensor, workspace: Tensor, stream=None) -> Tensor:
    """dx[:T] = grouped dy W_g; T = dy.shape[0]; rows of dx past T are left untouched."""
    G = w.shape[0] if isinstance(w, Tensor) else len(w)
    w0 = _first(w)
    N, K = w0.shape[-2], w0.shape[-1]
    T = dy.shape[0]
    if dy.dim() != 2 or dy.shape[1] != N:
        raise ValueError(f"dy must be [T, {N}], got {tuple(dy.shape)}")
    if dx.dim() != 2 or dx.shape[1] != K or dx.dtype != dy.dtype or w0.dtype != dy.dtype:
        raise ValueError("dx must be [rows >= T, K] and dy, w, dx must share one dtype")
    wp, wpp, keep = _grouped(w, dy.device, stream)
    _check(load().gl_dgrad(G, K, N, T, _dtype(dy), _ptr(dy), wp, wpp, _ptr(dx), dx.shape[0], _ptr(workspace),
                           _stream(stream)))
    del keep
    return dx


def gl_wgrad(x: Tensor, dy: Tensor, dw: Grouped, workspace: Tensor, *, accumulate: bool = False,
             stream=None) -> Grouped:
    """dW_g (+)= dy_g^T x_g over each group's rows; dw is [G, N, K] or G tensors [N, K]."""
    G = dw.shape[0] if isinstance(dw, Tensor) else len(dw)
    d0 = _first(dw)
    N, K = d0.shape[-2], d0.shape[-1]
    T = x.shape[0]
    if x.shape != (T, K) or dy.shape != (T, N) or x.dtype != dy.dtype:
        raise ValueError("x must be [T, K] and dy [T, N] with one dtype")
    dp, dpp, keep = _grouped(dw, x.device, stream)
    _check(load().gl_wgrad(G, K, N, T, _dtype(x), _dtype(d0), _ptr(x), _ptr(dy), dp, dpp, int(bool(accumulate)),
                           _ptr(workspace), _stream(stream)))
    del keep
    return dw


def gl_wgrad_bgrad(x: Tensor, dy: Tensor, dw: Grouped, db: Grouped, workspace: Tensor, *, accumulate: bool = False,
                   stream=None):
    """gl_wgrad and the bias gradient of the same dy in one call: db is [G, N] or G
    tensors [N], of dy's dtype or fp32."""
    G = dw.shape[0] if isinstance(dw, Tensor) else len(dw)
    d0 = _first(dw)
    b0 = _first(db)
    N, K = d0.shape[-2], d0.shape[-1]
    T = x.shape[0]
    if x.shape != (T, K) or dy.shape != (T, N) or x.dtype != dy.dtype:
        raise ValueError("x must be [T, K] and dy [T, N] with one dtype")
    if b0.shape[-1] != N or (isinstance(db, Tensor) and db.shape != (G, N)):
        raise ValueError("db must be [G, N] or G tensors [N]")
    dp, dpp, keep = _grouped(dw, x.device, stream)
    bp, bpp, keep_b = _grouped(db, x.device, stream)
    _check(load().gl_wgrad_bgrad(G, K, N, T, _dtype(x), _dtype(d0), _dtype(b0), _ptr(x), _ptr(dy), dp, dpp,
                                 int(bool(accumulate)), bp, bpp, _ptr(workspace), _stream(stream)))
    del keep, keep_b
    return dw, db


def gl_bgrad(dy: Tensor, db: Grouped, workspace: Tensor, stream=None) -> Grouped:
    """db_g = column sums of dy over each group's rows; db is [G, N] or G tensors [N]."""
    G = db.shape[0] if isinstance(db, Tensor) else len(db)
    N = dy.shape[1]
    d0 = db[0] if not isinstance(db, Tensor) else db
    if d0.shape[-1] != N or d0.dtype != dy.dtype:
        raise ValueError("db must have dy's column count and dtype")
    dp, dpp, keep = _grouped(db, dy.device, stream)
    _check(load().gl_bgrad(G, N, dy.shape[0], _dtype(dy), _ptr(dy), dp, dpp, _ptr(workspace), _stream(stream)))
    del keep
    return db


def gl_group_quantize_mxfp8(src: Tensor, data: Tensor, scale: Tensor, stream=None):
    """Rowwise MXFP8 of a bf16 [rows, cols] tensor into uint8 data [rows, cols] and
    uint8 scale [rows, cols/32] (leading dimensions are flattened into rows)."""
    if src.dtype != torch.bfloat16:
        raise ValueError("src must be bfloat16")
    cols = src.shape[-1]
    rows = src.numel() // cols if cols else 0
    if data.numel() != src.numel() or data.dtype != torch.uint8:
        raise ValueError("data must be uint8 with src's element count")
    if scale.numel() != rows * (cols // 32) or scale.dtype != torch.uint8:
        raise ValueError("scale must be uint8 with rows * cols/32 elements")
    _check(load().gl_group_quantize_mxfp8(_ptr(src), rows, cols, _ptr(data), _ptr(scale), _stream(stream)))
    return data, scale


# ------------------------------------------------------------------ MXFP8 backward


def gl_colwise_ld(num_groups: int, total_rows: int) -> int:
    """Row length of the transposed columnwise activation layout that fits any split."""
    return int(load().gl_colwise_ld(int(num_groups), int(total_rows)))


def gl_group_quantize_mxfp8_colwise(src: Tensor, data_t: Tensor, scale_t: Tensor, workspace: Tensor,
                                    num_groups: int, stream=None):
    """Columnwise MXFP8 of bf16 [T, C] per group into data_t [C, ld] / scale_t [C, ld/32]."""
    T, C = src.shape
    ld = data_t.shape[1]
    if src.dtype != torch.bfloat16 or data_t.shape != (C, ld) or scale_t.shape != (C, ld // 32):
        raise ValueError("src must be bf16 [T, C], data_t [C, ld] and scale_t [C, ld/32]")
    _check(load().gl_group_quantize_mxfp8_colwise(_ptr(src), C, int(num_groups), T, _ptr(workspace), _ptr(data_t),
                                                  _ptr(scale_t), ld, _stream(stream)))
    return data_t, scale_t


def gl_group_quantize_mxfp8_rowwise_colwise(src: Tensor, data: Tensor, scale: Tensor, data_t: Tensor,
                                            scale_t: Tensor, workspace: Tensor, num_groups: int, stream=None):
    """Rowwise codes data [T, C] / scale [T, C/32] and per-group columnwise codes
    data_t [C, ld] / scale_t [C, ld/32] of one bf16 tensor [T, C], read once."""
    T, C = src.shape
    ld = data_t.shape[1]
    if src.dtype != torch.bfloat16 or data.shape != (T, C) or scale.shape != (T, C // 32):
        raise ValueError("src must be bf16 [T, C], data [T, C] and scale [T, C/32]")
    if data_t.shape != (C, ld) or scale_t.shape != (C, ld // 32):
        raise ValueError("data_t must be [C, ld] and scale_t [C, ld/32]")
    _check(load().gl_group_quantize_mxfp8_rowwise_colwise(_ptr(src), C, int(num_groups), T, _ptr(workspace),
                                                          _ptr(data), _ptr(scale), _ptr(data_t), _ptr(scale_t), ld,
                                                          _stream(stream)))
    return data, scale, data_t, scale_t


def gl_quantize_mxfp8_colwise_weights(w: Tensor, data_t: Tensor, scale_t: Tensor, stream=None):
    """Columnwise MXFP8 of bf16 weights [G, N, K] into data_t [G, K, N] / scale_t [G, K, N/32]."""
    G, N, K = w.shape
    if w.dtype != torch.bfloat16 or data_t.shape != (G, K, N) or scale_t.shape != (G, K, N // 32):
        raise ValueError("w must be bf16 [G, N, K], data_t [G, K, N] and scale_t [G, K, N/32]")
    _check(load().gl_quantize_mxfp8_colwise_weights(_ptr(w), G, N, K, _ptr(data_t), _ptr(scale_t), _stream(stream)))
    return data_t, scale_t


def gl_offsets_quantize_mxfp8(m_splits: Tensor, x: Tensor, workspace: Tensor, data: Tensor, scale: Tensor,
                              stream=None):
    """One launch: the split-offset scan into ``workspace`` and rowwise MXFP8 of the
    bf16 activations x [T, K] into data [T, K] / scale [T, K/32]."""
    if m_splits.dtype != torch.int64:
        raise ValueError("m_splits must be int64")
    T, K = x.shape
    if x.dtype != torch.bfloat16 or data.shape != (T, K) or scale.shape != (T, K // 32):
        raise ValueError("x must be bf16 [T, K], data [T, K] and scale [T, K/32]")
    _check(load().gl_offsets_quantize_mxfp8(_ptr(m_splits), m_splits.numel(), T, _ptr(workspace), _ptr(x), K,
                                            _ptr(data), _ptr(scale), _stream(stream)))
    return data, scale


def gl_offsets_quantize_mxfp8_rowwise_colwise(m_splits: Tensor, x: Tensor, workspace: Tensor, data: Tensor,
                                              scale: Tensor, data_t: Tensor, scale_t: Tensor, stream=None):
    """The split-offset scan into ``workspace`` and both MXFP8 usages of the bf16
    activations x [T, K]: rowwise data [T, K] / scale [T, K/32] and per-group
    columnwise data_t [K, ld] / scale_t [K, ld/32], x read once."""
    if m_splits.dtype != torch.int64:
        raise ValueError("m_splits must be int64")
    T, K = x.shape
    ld = data_t.shape[1]
    if x.dtype != torch.bfloat16 or data.shape != (T, K) or scale.shape != (T, K // 32):
        raise ValueError("x must be bf16 [T, K], data [T, K] and scale [T, K/32]")
    if data_t.shape != (K, ld) or scale_t.shape != (K, ld // 32):
        raise ValueError("data_t must be [K, ld] and scale_t [K, ld/32]")
    _check(load().gl_offsets_quantize_mxfp8_rowwise_colwise(_ptr(m_splits), m_splits.numel(), T, _ptr(workspace),
                                                            _ptr(x), K, _ptr(data), _ptr(scale), _ptr(data_t),
                                                            _ptr(scale_t), ld, _stream(stream)))
    return data, scale, data_t, scale_t


def gl_quantize_mxfp8_weights(w: Tensor, data: Tensor, scale: Tensor, data_t: Tensor = None, scale_t: Tensor = None,
                              noop_flag: Tensor = None, stream=None):
    """The weights' MXFP8 workspace in one launch: rowwise data [G, N, K] / scale
    [G, N, K/32] and, if given, columnwise data_t [G, K, N] / scale_t [G, K, N/32].
    ``noop_flag`` (device int32, one element): nonzero at run time skips the work."""
    G, N, K = w.shape
    if w.dtype != torch.bfloat16 or data.shape != (G, N, K) or scale.shape != (G, N, K // 32):
        raise ValueError("w must be bf16 [G, N, K], data [G, N, K] and scale [G, N, K/32]")
    if (data_t is None) != (scale_t is None):
        raise ValueError("give both data_t and scale_t, or neither")
    if data_t is not None and (data_t.shape != (G, K, N) or scale_t.shape != (G, K, N // 32)):
        raise ValueError("data_t must be [G, K, N] and scale_t [G, K, N/32]")
    if noop_flag is not None and (noop_flag.dtype != torch.int32 or noop_flag.numel() != 1):
        raise ValueError("noop_flag must be a one-element int32 tensor")
    _check(load().gl_quantize_mxfp8_weights(_ptr(w), G, N, K, _ptr(data), _ptr(scale),
                                            _ptr(data_t) if data_t is not None else None,
                                            _ptr(scale_t) if scale_t is not None else None,
                                            _ptr(noop_flag) if noop_flag is not None else None, _stream(stream)))
    return data, scale


def gl_swiglu_forward(h: Tensor, a: Tensor, stream=None) -> Tensor:
    """a [T, F] = silu(h[:, :F]) * h[:, F:] for h [T, 2F]."""
    T, F2 = h.shape
    if a.shape != (T, F2 // 2) or a.dtype != h.dtype or F2 % 2:
        raise ValueError("h must be [T, 2F] and a [T, F] of h's dtype")
    _check(load().gl_swiglu_forward(T, F2 // 2, _dtype(h), _ptr(h), _ptr(a), _stream(stream)))
    return a


def gl_swiglu_backward(h: Tensor, da: Tensor, dh: Tensor, stream=None) -> Tensor:
    """dh [T, 2F]: the gradient of gl_swiglu_forward at h for the upstream gradient da [T, F]."""
    T, F2 = h.shape
    if da.shape != (T, F2 // 2) or dh.shape != h.shape or not (da.dtype == dh.dtype == h.dtype):
        raise ValueError("h and dh must be [T, 2F] and da [T, F], one dtype")
    _check(load().gl_swiglu_backward(T, F2 // 2, _dtype(h), _ptr(h), _ptr(da), _ptr(dh), _stream(stream)))
    return dh


def gl_grouped_mlp_forward(x: Tensor, w1: Grouped, w2: Grouped, h: Tensor, a: Tensor, y: Tensor, workspace: Tensor,
                           b1: Grouped = None, b2: Grouped = None, stream=None) -> Tensor:
    """y[:T] = FC2(SwiGLU(FC1(x))) per group; h [T, 2F] and a [T, F] receive the
    intermediates (kept for the backward); y may have more rows than T."""
    G = w1.shape[0] if isinstance(w1, Tensor) else len(w1)
    F2, K = _first(w1).shape[-2:]
    N = _first(w2).shape[-2]
    T = x.shape[0]
    if x.shape != (T, K) or h.shape != (T, F2) or a.shape != (T, F2 // 2) or y.dim() != 2 or y.shape[1] != N:
        raise ValueError("shapes: x [T, K], w1 [G, 2F, K], w2 [G, N, F], h [T, 2F], a [T, F], y [rows >= T, N]")
    p1, pp1, k1 = _grouped(w1, x.device, stream)
    p2, pp2, k2 = _grouped(w2, x.device, stream)
    q1, qq1, k3 = _grouped(b1, x.device, stream)
    q2, qq2, k4 = _grouped(b2, x.device, stream)
    _check(load().gl_grouped_mlp_forward(G, K, F2 // 2, N, T, _dtype(x), _ptr(x), p1, pp1, q1, qq1, p2, pp2, q2, qq2,
                                         _ptr(h), _ptr(a), _ptr(y), y.shape[0], _ptr(workspace), _stream(stream)))
    del k1, k2, k3, k4
    return y


def gl_grouped_mlp_backward(x: Tensor, w1: Grouped, w2: Grouped, h: Tensor, a: Tensor, dy: Tensor, da: Tensor,
                            dh: Tensor, dx: Tensor, dw1: Grouped, dw2: Grouped, workspace: Tensor,
                            db1: Grouped = None, db2: Grouped = None, *, accumulate: bool = False, stream=None):
    """Backward of gl_grouped_mlp_forward: dx[:T], dW1, dW2 (of dw1's dtype: the
    input's or fp32, added into them with ``accumulate``), optional db1, db2; da
    [T, F] and dh [T, 2F] are scratch."""
    G = w1.shape[0] if isinstance(w1, Tensor) else len(w1)
    F2, K = _first(w1).shape[-2:]
    N = _first(w2).shape[-2]
    T = x.shape[0]
    if dy.shape != (T, N) or da.shape != (T, F2 // 2) or dh.shape != (T, F2) or dx.dim() != 2 or dx.shape[1] != K:
        raise ValueError("shapes: dy [T, N], da [T, F], dh [T, 2F], dx [rows >= T, K]")
    keep = []
    ptr = {}
    for name, g in (("w1", w1), ("w2", w2), ("dw1", dw1), ("dw2", dw2), ("db1", db1), ("db2", db2)):
        p, pp, k = _grouped(g, x.device, stream)
        ptr[name] = (p, pp)
        keep.append(k)
    _check(load().gl_grouped_mlp_backward(G, K, F2 // 2, N, T, _dtype(x), _dtype(_first(dw1)), _ptr(x), *ptr["w1"],
                                          *ptr["w2"], _ptr(h), _ptr(a), _ptr(dy), _ptr(da), _ptr(dh), _ptr(dx),
                                          dx.shape[0], *ptr["dw1"], *ptr["db1"], *ptr["dw2"], *ptr["db2"],
                                          int(bool(accumulate)), _ptr(workspace), _stream(stream)))
    del keep
    return dx


def gl_dgrad_mxfp8(dy: Tensor, dy_scale: Tensor, w_t: Tensor, w_t_scale: Tensor, dx: Tensor, workspace: Tensor,
                   stream=None) -> Tensor:
    """dx[:T] = grouped deq(dy) deq(W_g) from rowwise dy codes and columnwise weight codes [G, K, N]."""
    G, K, N = w_t.shape
    T = dy.shape[0]
    if dy.shape != (T, N) or dx.dim() != 2 or dx.shape[1] != K:
        raise ValueError("dy must be [T, N] codes and dx [rows >= T, K]")
    _check(load().gl_dgrad_mxfp8(G, K, N, T, _dtype(dx), _ptr(dy), _ptr(dy_scale), _ptr(w_t), _ptr(w_t_scale),
                                 _ptr(dx), dx.shape[0], _ptr(workspace), _stream(stream)))
    return dx


def gl_wgrad_mxfp8(dy_t: Tensor, dy_t_scale: Tensor, x_t: Tensor, x_t_scale: Tensor, dw: Grouped,
                   workspace: Tensor, total_rows: int, *, accumulate: bool = False, stream=None) -> Grouped:
    """dW_g (+)= deq(dy_g)^T deq(x_g) from columnwise codes dy_t [N, ld] and x_t [K, ld]."""
    G = dw.shape[0] if isinstance(dw, Tensor) else len(dw)
    d0 = _first(dw)
    N, ld = dy_t.shape
    K = x_t.shape[0]
    if x_t.shape != (K, ld) or tuple(d0.shape[-2:]) != (N, K):
        raise ValueError("x_t must be [K, ld] and dw [G, N, K] or G tensors [N, K]")
    dp, dpp, keep = _grouped(dw, dy_t.device, stream)
    _check(load().gl_wgrad_mxfp8(G, K, N, int(total_rows), _dtype(d0), _ptr(dy_t), _ptr(dy_t_scale), _ptr(x_t),
                                 _ptr(x_t_scale), ld, dp, dpp, int(bool(accumulate)), _ptr(workspace),
                                 _stream(stream)))
    del keep
    return dw


def _tensors(obj):
    """Every tensor inside nested tuples / lists."""
    if isinstance(obj, Tensor):
        yield obj
    elif isinstance(obj, (tuple, list)):
        for o in obj:
            yield from _tensors(o)


class WgradQueue:
    """Deferred grouped weight gradients (the ``gl_wgrad_queue_*`` entry points).

    ``put`` / ``put_mxfp8`` take the arguments of ``gl_wgrad_bgrad`` (``db=None``:
    plain ``gl_wgrad``) / ``gl_wgrad_mxfp8``, check them in full and record the
    call without running it; ``run_next`` launches the oldest recorded call and
    ``flush`` all of them, in put order.  The queue holds a reference to every
    tensor of a recorded call until it has been launched, and ties their memory
    to the stream it runs on; the workspace must still hold the same splits' offsets.
    """

    def __init__(self):
        self._q = ctypes.c_void_p()
        _check(load().gl_wgrad_queue_create(ctypes.byref(self._q)))
        self._held = collections.deque()

    def __len__(self) -> int:
        n = load().gl_wgrad_queue_size(self._q)
        if n < 0:
            _check(n)
        return n

    def put(self, x: Tensor, dy: Tensor, dw: Grouped, workspace: Tensor, *, db: Optional[Grouped] = None,
            accumulate: bool = False) -> None:
        G = dw.shape[0] if isinstance(dw, Tensor) else len(dw)
        d0 = _first(dw)
        N, K = d0.shape[-2], d0.shape[-1]
        T = x.shape[0]
        if x.shape != (T, K) or dy.shape != (T, N) or x.dtype != dy.dtype:
            raise ValueError("x must be [T, K] and dy [T, N] with one dtype")
        db_dtype = GL_F32
        if db is not None:
            b0 = _first(db)
            if b0.shape[-1] != N or (isinstance(db, Tensor) and db.shape != (G, N)):
                raise ValueError("db must be [G, N] or G tensors [N]")
            db_dtype = _dtype(b0)
        dp, dpp, keep = _grouped(dw, x.device)
        bp, bpp, keep_b = _grouped(db, x.device)
        _check(load().gl_wgrad_queue_put(self._q, G, K, N, T, _dtype(x), _dtype(d0), db_dtype, _ptr(x), _ptr(dy), dp,
                                         dpp, int(bool(accumulate)), bp, bpp, _ptr(workspace)))
        self._held.append((x, dy, dw, db, workspace, keep, keep_b))

    def put_mxfp8(self, dy_t: Tensor, dy_t_scale: Tensor, x_t: Tensor, x_t_scale: Tensor, dw: Grouped,
                  workspace: Tensor, total_rows: int, *, accumulate: bool = False) -> None:
        G = dw.shape[0] if isinstance(dw, Tensor) else len(dw)
        d0 = _first(dw)
        N, ld = dy_t.shape
        K = x_t.shape[0]
        if x_t.shape != (K, ld) or tuple(d0.shape[-2:]) != (N, K):
            raise ValueError("x_t must be [K, ld] and dw [G, N, K] or G tensors [N, K]")
        dp, dpp, keep = _grouped(dw, dy_t.device)
        _check(load().gl_wgrad_queue_put_mxfp8(self._q, G, K, N, int(total_rows), _dtype(d0), _ptr(dy_t),
                                               _ptr(dy_t_scale), _ptr(x_t), _ptr(x_t_scale), ld, dp, dpp,
                                               int(bool(accumulate)), _ptr(workspace)))
        self._held.append((dy_t, dy_t_scale, x_t, x_t_scale, dw, workspace, keep))

    def _launching(self, held, stream):
        _record(list(_tensors(held)), torch.cuda.current_stream() if stream is None else stream)

    def run_next(self, stream=None) -> None:
        """Launch the oldest recorded call on ``stream`` (torch's current one by default)."""
        if not self._held:
            return
        self._launching(self._held.popleft(), stream)
        _check(load().gl_wgrad_queue_run_next(self._q, _stream(stream)))

    def flush(self, stream=None) -> None:
        """Launch every recorded call, in put order."""
        held, self._held = list(self._held), collections.deque()
        for h in held:
            self._launching(h, stream)
        _check(load().gl_wgrad_queue_flush(self._q, _stream(stream)))

    def clear(self) -> None:
        """Drop the recorded calls without running them."""
        _check(load().gl_wgrad_queue_clear(self._q))
        self._held.clear()

    def close(self) -> None:
        if self._q:
            load().gl_wgrad_queue_destroy(self._q)
            self._q = ctypes.c_void_p()
        self._held.clear()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
