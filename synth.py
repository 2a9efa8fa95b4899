"""Seeded synthetic inputs for the grouped-linear workloads.

This module only draws random numbers and lays them out; it holds none of the
grouped-linear arithmetic. Both the HIP library's tests/benchmark and the CPU
oracle consume what it produces, so it must stay free of either side's code.

Recipe (every workload, seed 0 unless a caller overrides it):
  * numpy ``SeedSequence(seed).spawn(7)`` gives one child per role, in order:
    split sizes, group permutation, x, W, bias, dy, main_grad.
  * x and dy are drawn in blocks of ``ROW_BLOCK`` rows; block ``i`` comes from
    child ``i`` of that role's sequence.  W is drawn one group at a time from
    child ``g`` of the W sequence, so any single group can be regenerated alone.
  * Samples are float32 (``Generator.standard_normal`` / ``uniform``) and, for
    bf16 workloads, rounded to bfloat16 by round-to-nearest-even.
  * Split sizes: a fixed list, a uniform multinomial, or a Zipf-weighted
    multinomial over a seeded permutation of the groups, after which the
    ``zipf_zeros`` lowest-probability groups are emptied into the most
    probable group (a multinomial with these weights essentially never yields
    an empty group by itself).
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np
import torch

ROW_BLOCK = 1024

_ROLE = {"m": 0, "perm": 1, "x": 2, "w": 3, "b": 4, "dy": 5, "main_grad": 6}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    G: int                     # number of groups
    K: int                     # in_features
    N: int                     # out_features
    T: int                     # total valid rows (sum of split sizes)
    dtype: str                 # "f32" or "bf16" (storage type of x, W, b, y, dy)
    m_law: str                 # "fixed" | "uniform" | "zipf"
    m_fixed: tuple = ()
    zipf_s: float = 1.2
    zipf_zeros: int = 0
    bias: bool = False
    w_law: str = "normal"      # "normal" (std w_std) | "uniform" (+-w_bound)
    w_std: float = 0.02
    w_bound: float = 0.125
    b_std: float = 0.1
    passes: tuple = ("fwd",)   # which passes the workload exercises
    accumulate: bool = False   # wgrad accumulates into an fp32 main_grad
    out_rows: int = 0          # caller output buffer rows (0: exactly T)
    per_group_weights: bool = False
    mxfp8: bool = False
    seed: int = 0

    def scaled(self, **kw) -> "Workload":
        """Same structure at other sizes (used for oracle-sized parity cases)."""
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("fwd_f32_g4_k64_n32", G=4, K=64, N=32, T=32, dtype="f32", m_law="fixed",
                 m_fixed=(5, 0, 17, 10), bias=True, w_law="uniform", w_bound=0.125,
                 passes=("fwd",)),
        Workload("bf16_train_g8_k4096_n14336", G=8, K=4096, N=14336, T=16384, dtype="bf16",
                 m_law="uniform", bias=True, passes=("fwd", "dgrad", "wgrad", "bgrad")),
        Workload("bf16_zipf_g64_k2048_n1536", G=64, K=2048, N=1536, T=65536, dtype="bf16",
                 m_law="zipf", zipf_s=1.2, zipf_zeros=4, bias=False,
                 passes=("fwd", "dgrad", "wgrad"), accumulate=True),
        Workload("bf16_fwd_g256_k7168_n2048_outbuf", G=256, K=7168, N=2048, T=32768,
                 dtype="bf16", m_law="uniform", bias=False, passes=("fwd",), out_rows=34000,
                 per_group_weights=True),
        Workload("mxfp8_fwd_g32_k4096_n4096", G=32, K=4096, N=4096, T=32768, dtype="bf16",
                 m_law="uniform", bias=False, w_std=0.02, passes=("fwd",), mxfp8=True),
    ]
}


def _children(wl: Workload, role: str, n: int):
    root = np.random.SeedSequence(wl.seed).spawn(len(_ROLE))[_ROLE[role]]
    return root.spawn(n)


def _rng(seq) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seq))


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def split_sizes(wl: Workload) -> np.ndarray:
    """int64[G] row counts per group; they sum to wl.T."""
    if wl.m_law == "fixed":
        m = np.array(wl.m_fixed, dtype=np.int64)
    elif wl.m_law == "uniform":
        (c,) = _children(wl, "m", 1)
        m = _rng(c).multinomial(wl.T, [1.0 / wl.G] * wl.G).astype(np.int64)
    elif wl.m_law == "zipf":
        (c,) = _children(wl, "m", 1)
        (cp,) = _children(wl, "perm", 1)
        perm = _rng(cp).permutation(wl.G)
        p = np.empty(wl.G, dtype=np.float64)
        ranks = np.arange(1, wl.G + 1, dtype=np.float64)
        p[perm] = ranks ** (-wl.zipf_s)
        p /= p.sum()
        m = _rng(c).multinomial(wl.T, p).astype(np.int64)
        if wl.zipf_zeros:
            order = np.argsort(p, kind="stable")
            lowest = order[: wl.zipf_zeros]
            top = order[-1]
            m[top] += m[lowest].sum()
            m[lowest] = 0
    else:
        raise ValueError(wl.m_law)
    assert m.shape == (wl.G,) and int(m.sum()) == wl.T and (m >= 0).all()
    return m


def _storage_dtype(wl: Workload):
    return torch.float32 if wl.dtype == "f32" else torch.bfloat16


def _to_storage(a: np.ndarray, wl: Workload) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t if wl.dtype == "f32" else t.to(torch.bfloat16)


def _rows_normal(wl: Workload, role: str, rows: int, cols: int, std: float = 1.0,
                 dtype=None) -> torch.Tensor:
    nblk = (rows + ROW_BLOCK - 1) // ROW_BLOCK
    kids = _children(wl, role, max(nblk, 1))
    out = torch.empty((rows, cols), dtype=dtype or _storage_dtype(wl))

    def fill(i):
        lo, hi = i * ROW_BLOCK, min(rows, (i + 1) * ROW_BLOCK)
        a = _rng(kids[i]).standard_normal((hi - lo, cols), dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        t = torch.from_numpy(a)
        out[lo:hi] = t if out.dtype == torch.float32 else t.to(out.dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nblk)))
    return out


def x(wl: Workload) -> torch.Tensor:
    """Input activations [T, K], N(0, 1)."""
    return _rows_normal(wl, "x", wl.T, wl.K)


def dy(wl: Workload) -> torch.Tensor:
    """Output gradient [T, N], N(0, 1)."""
    return _rows_normal(wl, "dy", wl.T, wl.N)


def weight_group(wl: Workload, g: int) -> torch.Tensor:
    """Weight of one group [N, K] (regenerable on its own)."""
    kid = _children(wl, "w", wl.G)[g]
    r = _rng(kid)
    if wl.w_law == "uniform":
        a = r.uniform(-wl.w_bound, wl.w_bound, size=(wl.N, wl.K)).astype(np.float32)
    else:
        a = r.standard_normal((wl.N, wl.K), dtype=np.float32)
        a *= np.float32(wl.w_std)
    return _to_storage(a, wl)


def weight(wl: Workload, groups=None) -> torch.Tensor:
    """Stacked weights [G, N, K] (or only the listed groups, stacked in that order)."""
    groups = list(range(wl.G)) if groups is None else list(groups)
    out = torch.empty((len(groups), wl.N, wl.K), dtype=_storage_dtype(wl))

    def fill(i):
        out[i] = weight_group(wl, groups[i])

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(groups))))
    return out


def bias(wl: Workload) -> torch.Tensor:
    """Per-group biases [G, N], N(0, b_std)."""
    (kid,) = _children(wl, "b", 1)
    a = _rng(kid).standard_normal((wl.G, wl.N), dtype=np.float32) * np.float32(wl.b_std)
    return _to_storage(a, wl)


def main_grad(wl: Workload) -> torch.Tensor:
    """Preset fp32 main_grad [G, N, K], N(0, 1)."""
    kids = _children(wl, "main_grad", wl.G)
    out = torch.empty((wl.G, wl.N, wl.K), dtype=torch.float32)

    def fill(g):
        out[g] = torch.from_numpy(_rng(kids[g]).standard_normal((wl.N, wl.K), dtype=np.float32))

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(wl.G)))
    return out


def checksum(t) -> str:
    """First 16 hex digits of the SHA-256 of a tensor's or array's raw bytes (row-major),
    recorded beside results so that a run's inputs can be matched to this recipe."""
    import hashlib
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous()
        t = t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t
        a = t.numpy()
    else:
        a = np.ascontiguousarray(t)
    return hashlib.sha256(a.tobytes()).hexdigest()[:16]


def special_bf16_block_values() -> torch.Tensor:
    """Every finite bfloat16 bit pattern, as a bf16 tensor (for exhaustive quantizer cases)."""
    bits = torch.arange(0, 1 << 16, dtype=torch.int32).to(torch.int16)
    v = bits.view(torch.bfloat16)
    return v[torch.isfinite(v.float())]
