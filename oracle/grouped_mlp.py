"""Float64 CPU oracle of the grouped MLP built from two grouped linear layers --
test infrastructure only.

What is computed (page "[PyTorch] Add optional caller-provided output/grad-input
buffers to GroupedLinear and fused grouped MLP": a fused op of FC1, an
activation and FC2 over the same split sizes, whose FC2 output and FC1 grad-input
may be caller-provided buffers, written on the valid rows alone).  The pages
do not name the activation; it is taken here as SwiGLU over the two halves of
FC1's output: act(h) = silu(h[:, :F]) * h[:, F:], silu(v) = v / (1 + exp(-v)).

Storage points: FC1's output h and the activation a are stored in the layer's
dtype (bf16 / fp16 / fp32) before the next step reads them, as the layers' own
outputs are; ``store`` rounds a float64 array to that dtype (identity for fp32)
so the oracle follows the same definition.  All arithmetic is float64; the
grouped GEMMs are those of ``grouped_linear``.
"""
from __future__ import annotations

import numpy as np
import torch

from . import grouped_linear as gl

_TORCH = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32, "f64": torch.float64}


def store(v, dtype: str) -> np.ndarray:
    """Round float64 values to the storage dtype (round to nearest even) and back;
    "f64" keeps them as they are."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float64))
    return t.to(_TORCH[dtype]).to(torch.float64).numpy()


def silu(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return v / (1.0 + np.exp(-v))


def swiglu(h) -> np.ndarray:
    """act(h) for h [T, 2F]: silu of the first half times the second half -> [T, F]."""
    h = np.asarray(h, dtype=np.float64)
    F = h.shape[1] // 2
    return silu(h[:, :F]) * h[:, F:]


def swiglu_backward(h, da) -> np.ndarray:
    """d act / d h for h [T, 2F] and upstream da [T, F] -> dh [T, 2F].

    With s = sigmoid(g): d silu(g)/dg = s + g s (1 - s); so
    dh[:, :F] = da * u * (s + g s (1 - s)),  dh[:, F:] = da * silu(g).
    """
    h = np.asarray(h, dtype=np.float64)
    da = np.asarray(da, dtype=np.float64)
    F = h.shape[1] // 2
    g, u = h[:, :F], h[:, F:]
    s = 1.0 / (1.0 + np.exp(-g))
    return np.concatenate([da * u * (s + g * s * (1.0 - s)), da * g * s], axis=1)


def mlp_forward(x, w1, b1, w2, b2, m_splits, dtype: str = "bf16"):
    """FC1 -> SwiGLU -> FC2 per group.  w1: [G, 2F, K] (or G arrays), w2: [G, N, F];
    b1 [G, 2F] / b2 [G, N] or None.  Returns (h, a, y): h and a as stored in
    ``dtype``, y in float64 (the caller compares it against its rounded output)."""
    h = store(gl.forward(x, w1, b1, m_splits), dtype)
    a = store(swiglu(h), dtype)
    y = gl.forward(a, w2, b2, m_splits)
    return h, a, y


def mlp_backward(x, w1, w2, h, a, dy, m_splits, dtype: str = "bf16"):
    """Backward of ``mlp_forward`` given its stored h and a: returns
    (dx, dw1, db1, dw2, db2, da, dh) in float64, with da and dh as stored in
    ``dtype`` (they are the layers' intermediate gradients)."""
    dw2 = gl.wgrad(a, dy, m_splits)
    db2 = gl.bgrad(dy, m_splits)
    da = store(gl.dgrad(dy, w2, m_splits), dtype)
    dh = store(swiglu_backward(h, da), dtype)
    dw1 = gl.wgrad(x, dh, m_splits)
    db1 = gl.bgrad(dh, m_splits)
    dx = gl.dgrad(dh, w1, m_splits)
    return dx, dw1, db1, dw2, db2, da, dh
