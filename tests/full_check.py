"""Whole-output comparisons against the oracle at full workload sizes.

The oracle is run one group (or one block of rows) at a time, so host memory stays
bounded, and every element of the GPU output is compared.  Each comparison prints
one summary line: elements compared, elements outside the bound, the worst
err / limit ratio and, for fp32 outputs, the share within the fp32 bound.
No arithmetic of the method lives here: the reference values all come from
``oracle``.
"""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

from gl_testutil import TOL_F32, to64


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def pool_map(fn, items):
    """fn over items on host threads (numpy's elementwise work releases the GIL)."""
    items = list(items)
    with ThreadPoolExecutor(threads()) as ex:
        return list(ex.map(fn, items))


class Tally:
    """Running comparison of chunks of one output against the oracle:
    |got - ref| <= rel * (|ref| + 1) element by element."""

    def __init__(self, what: str, rel: float):
        self.what, self.rel = what, rel
        self.n = self.bad = 0
        self.worst = 0.0
        self.worst_at = None
        self.within_f32 = 0
        self.worst_f32 = 0.0

    def add(self, label, got, ref):
        g = to64(got) if isinstance(got, torch.Tensor) else np.asarray(got, dtype=np.float64)
        ref = np.asarray(ref, dtype=np.float64)
        assert g.shape == ref.shape, f"{self.what} {label}: shape {g.shape} vs {ref.shape}"
        err = np.abs(g - ref)
        scale = np.abs(ref) + 1.0
        ratio = np.where(np.isnan(err), np.inf, err / (self.rel * scale))
        nbad = int((ratio > 1.0).sum())
        self.n += ratio.size
        self.bad += nbad
        if ratio.size:
            i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
            if ratio[i] > self.worst or self.worst_at is None:
                self.worst = float(ratio[i])
                self.worst_at = (label, tuple(int(v) for v in i), float(g[i]), float(ref[i]))
            r32 = np.where(np.isnan(err), np.inf, err / (TOL_F32 * scale))
            self.within_f32 += int((r32 <= 1.0).sum())
            self.worst_f32 = max(self.worst_f32, float(r32.max()))

    def finish(self, f32_floor=None):
        """Asserts the bound on every element; with ``f32_floor`` also that at least
        that share of the elements is within the fp32 bound (a regression guard for
        outputs whose fp32 summation order alone misses it on a few elements)."""
        frac32 = self.within_f32 / self.n if self.n else 1.0
        say(f"  {self.what}: {self.n} elements, {self.bad} outside {self.rel}*(|ref|+1), "
            f"worst err/limit {self.worst:.3g} at {self.worst_at}; "
            f"within {TOL_F32}*(|ref|+1): {frac32:.6%} (worst err/limit {self.worst_f32:.3g})")
        assert self.n > 0, f"{self.what}: nothing compared"
        assert self.bad == 0, (f"{self.what}: {self.bad} of {self.n} elements outside {self.rel}*(|ref|+1); "
                               f"worst {self.worst:.3g} at {self.worst_at}")
        if f32_floor is not None:
            assert frac32 >= f32_floor, (f"{self.what}: only {frac32:.6%} of the elements within "
                                         f"{TOL_F32}*(|ref|+1), below {f32_floor:.4%}")
        return frac32


def check_chunks(what, rel, chunks, f32_floor=None):
    """chunks: iterable of (label, got, ref); every element of every chunk is compared."""
    t = Tally(what, rel)
    for label, got, ref in chunks:
        t.add(label, got, ref)
    return t.finish(f32_floor)


def group_bounds(m):
    off = np.concatenate([[0], np.cumsum(np.asarray(m, dtype=np.int64))])
    return [(g, int(off[g]), int(off[g + 1])) for g in range(len(m))]


def assert_codes_equal(what, got: np.ndarray, ref: np.ndarray):
    if not np.array_equal(got, ref):
        bad = np.argwhere(got != ref)
        raise AssertionError(f"{what}: {len(bad)} of {got.size} bytes differ, first at {tuple(bad[0])}: "
                             f"got {got[tuple(bad[0])]:#04x}, oracle {ref[tuple(bad[0])]:#04x}")
