"""Helpers shared by the GPU parity tests: tolerance checks against the oracle and
bit-level comparisons.  No arithmetic of the method lives here."""
from __future__ import annotations

import numpy as np
import torch

# Tolerances of the parity bar: fp32 results 1e-4 * (|ref| + 1); bf16 and MXFP8
# GEMM outputs 2e-2 * (|ref| + 1), both against the oracle on the same rounded inputs.
TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def to64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def assert_close(got: torch.Tensor, ref: np.ndarray, rel: float, what: str = ""):
    g = to64(got)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    err = np.abs(g - ref)
    lim = rel * (np.abs(ref) + 1.0)
    bad = ~(err <= lim)
    if bad.any():
        idx = np.unravel_index(np.argmax(np.where(bad, err / lim, 0)), bad.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements outside {rel}*(|ref|+1); "
                             f"worst at {idx}: got {g[idx]!r}, ref {ref[idx]!r}")


def bits(t: torch.Tensor) -> torch.Tensor:
    """Raw bit pattern (so NaN payloads compare equal to themselves)."""
    t = t.detach().contiguous()
    view = {torch.float32: torch.int32, torch.bfloat16: torch.int16, torch.float16: torch.int16,
            torch.uint8: torch.uint8, torch.int64: torch.int64}[t.dtype]
    return t.view(view)


def assert_bits_equal(a: torch.Tensor, b: torch.Tensor, what: str = ""):
    ba, bb = bits(a).cpu(), bits(b).cpu()
    if not torch.equal(ba, bb):
        n = int((ba != bb).sum())
        raise AssertionError(f"{what}: {n} of {ba.numel()} elements differ bitwise")


def nan_tail(rows: int, cols: int, valid: int, dtype, device) -> torch.Tensor:
    """Output buffer whose rows >= valid hold a NaN sentinel, the rest garbage."""
    y = torch.full((rows, cols), float("nan"), dtype=dtype, device=device)
    y[:valid] = 12345.0
    return y
