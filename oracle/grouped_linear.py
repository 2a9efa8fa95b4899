"""Float64 CPU oracle of the grouped linear layer -- test infrastructure only.

What is computed (page "transformer_engine/pytorch/ops/basic/grouped_linear.py",
the GroupedLinear fusible op):

* class docstring: y_i = x_i W_i^T + b_i, which is the same as splitting the
  token matrix along its first dimension by the split sizes, applying one
  ``torch.nn.Linear`` per split and concatenating the results;
* ``fuser_backward``: dgrad dx_i = dy_i W_i (the "NN" grouped GEMM), wgrad
  dW_i = dy_i^T x_i (the "NT" grouped GEMM, optionally added into
  ``main_grad``), bias grad = column sums of each split of dy.

Inputs are the already-rounded storage values (bf16 or fp32); converting them
to float64 is exact, and all arithmetic here is float64.  Groups are handled
one at a time with a library matmul per group; nothing is blocked, fused or
reordered beyond that.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def offsets(m_splits, num_groups: int, total_rows: int) -> np.ndarray:
    """Split offsets: int64[G+1], off[0] = 0 and off[g+1] = off[g] + m[g].

    The exclusive prefix sum with a leading zero is what the offsets kernel of
    page "Single parameter for GroupedLinear module" computes (Greptile summary:
    one cumsum-with-leading-zero kernel replacing cumsum followed by cat).
    Rejections: a split count different from the number of groups (fuser_forward,
    "Extract split sizes from extra input"), a negative split, and splits that do
    not add up to the number of rows (torch.split's contract in fuser_forward).
    """
    m = [int(v) for v in np.asarray(m_splits).reshape(-1).tolist()]
    if len(m) != num_groups:
        raise ValueError(f"Expected {num_groups} splits, but got {len(m)}.")
    if any(v < 0 for v in m):
        raise ValueError("split sizes must be non-negative")
    off = [0]
    for v in m:
        off.append(off[-1] + v)
    if off[-1] != total_rows:
        raise ValueError(f"split sizes add up to {off[-1]}, but the input has {total_rows} rows")
    return np.array(off, dtype=np.int64)


def group_of_rows(off: np.ndarray, rows) -> np.ndarray:
    """Group index of each token row: the g with off[g] <= r < off[g+1]."""
    rows = np.asarray(rows, dtype=np.int64)
    return np.searchsorted(off, rows, side="right") - 1


def _group(mats, g: int) -> np.ndarray:
    """Group g of a stacked [G, ...] array or of a sequence of per-group arrays."""
    return _f64(mats[g])


def forward(x, w, b, m_splits, rows=None) -> np.ndarray:
    """Grouped forward y[r, :] = x[r, :] W_g^T + b_g for r in group g.

    x: [T, K]; w: stacked [G, N, K] or G arrays [N, K]; b: [G, N], G arrays [N]
    or None.  Rows of empty groups do not exist.  With ``rows`` given, only those
    output rows are computed (same definition, row by row) and returned as
    [len(rows), N]; otherwise the full [T, N].
    """
    x = np.asarray(x)
    G = len(m_splits)
    off = offsets(m_splits, G, x.shape[0])
    N = np.asarray(w[0]).shape[0]
    if rows is None:
        y = np.zeros((x.shape[0], N), dtype=np.float64)
        for g in range(G):
            lo, hi = int(off[g]), int(off[g + 1])
            if hi == lo:
                continue
            y[lo:hi] = _f64(x[lo:hi]) @ _group(w, g).T
            if b is not None:
                y[lo:hi] += _group(b, g)
        return y
    rows = np.asarray(rows, dtype=np.int64)
    gs = group_of_rows(off, rows)
    y = np.zeros((rows.size, N), dtype=np.float64)
    for g in np.unique(gs):
        sel = np.nonzero(gs == g)[0]
        y[sel] = _f64(x[rows[sel]]) @ _group(w, int(g)).T
        if b is not None:
            y[sel] += _group(b, int(g))
    return y


def dgrad(dy, w, m_splits, rows=None) -> np.ndarray:
    """Grouped dgrad dx[r, :] = dy[r, :] W_g for r in group g ("NN" layout in
    fuser_backward, "Perform dgrad GEMMs").  Shapes: dy [T, N] -> dx [T, K]."""
    dy = np.asarray(dy)
    G = len(m_splits)
    off = offsets(m_splits, G, dy.shape[0])
    K = np.asarray(w[0]).shape[1]
    if rows is None:
        dx = np.zeros((dy.shape[0], K), dtype=np.float64)
        for g in range(G):
            lo, hi = int(off[g]), int(off[g + 1])
            if hi == lo:
                continue
            dx[lo:hi] = _f64(dy[lo:hi]) @ _group(w, g)
        return dx
    rows = np.asarray(rows, dtype=np.int64)
    gs = group_of_rows(off, rows)
    dx = np.zeros((rows.size, K), dtype=np.float64)
    for g in np.unique(gs):
        sel = np.nonzero(gs == g)[0]
        dx[sel] = _f64(dy[rows[sel]]) @ _group(w, int(g))
    return dx


def wgrad(x, dy, m_splits, main_grad=None, accumulate: bool = False, groups=None,
          out_rows=None) -> np.ndarray:
    """Grouped wgrad dW_g = dy_g^T x_g, contracted over the group's own rows
    ("NT" layout in fuser_backward, "Perform wgrad GEMMs"); with ``accumulate``
    the sum is added to ``main_grad[g]`` (the Megatron-LM main_grad fusion in
    "Initialize grad weight buffers"), otherwise it overwrites.

    An empty group contributes an empty sum: zeros when storing, main_grad[g]
    unchanged when accumulating.  ``groups`` selects groups (default all) and
    ``out_rows`` selects rows n of each dW_g; the result is
    [len(groups), len(out_rows) or N, K].
    """
    x = np.asarray(x)
    dy = np.asarray(dy)
    G = len(m_splits)
    off = offsets(m_splits, G, x.shape[0])
    if dy.shape[0] != x.shape[0]:
        raise ValueError("x and dy must have the same number of rows")
    groups = list(range(G)) if groups is None else [int(g) for g in groups]
    nsel = np.arange(dy.shape[1]) if out_rows is None else np.asarray(out_rows, dtype=np.int64)
    if accumulate and main_grad is None:
        raise ValueError("accumulate needs main_grad")
    out = np.zeros((len(groups), nsel.size, x.shape[1]), dtype=np.float64)
    for i, g in enumerate(groups):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            out[i] = _f64(dy[lo:hi][:, nsel]).T @ _f64(x[lo:hi])
        if accumulate:
            out[i] += _f64(main_grad[g])[nsel]
    return out


def bgrad(dy, m_splits, groups=None) -> np.ndarray:
    """Bias grad db_g = sum of dy over the rows of group g (fuser_backward,
    "Split grad output tensor": a column sum per split); an empty group gives
    zeros, as a sum over an empty dimension does.  Returns [len(groups), N]."""
    dy = np.asarray(dy)
    G = len(m_splits)
    off = offsets(m_splits, G, dy.shape[0])
    groups = list(range(G)) if groups is None else [int(g) for g in groups]
    db = np.zeros((len(groups), dy.shape[1]), dtype=np.float64)
    for i, g in enumerate(groups):
        lo, hi = int(off[g]), int(off[g + 1])
        if hi > lo:
            db[i] = _f64(dy[lo:hi]).sum(axis=0)
    return db
