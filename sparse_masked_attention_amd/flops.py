"""Exact count of unmasked (row, column) pairs from the four boundary vectors.

Effective throughput counts only the FLOPs of pairs the mask leaves open. For
column j the masked rows are the union of at most three intervals, each
clipped to [0, N): the causal part [0, j), the lower interval
[LTS_j, LTE_j) and, when not causal, the upper interval [UTS_j, UTE_j). The
count per column is N minus the size of that union, in O(N) total.

FLOPs per open pair: forward 2(d + dv) (Q K^T and P V); backward
2(3d + 2dv) (recomputed Q K^T, dO V^T, P^T dO, dS^T Q and dS K).
"""
from __future__ import annotations

import numpy as np

__all__ = ["nnz_columns", "nnz", "fwd_flops", "bwd_flops"]


def nnz_columns(n, causal, lts=None, lte=None, uts=None, ute=None, n_rows=None) -> np.ndarray:
    """Open pairs per column for one (batch, head); n key columns, vectors
    [n] or None, n_rows query rows (default n)."""
    nr = n if n_rows is None else int(n_rows)
    j = np.arange(n, dtype=np.int64)
    zero = np.zeros(n, np.int64)
    starts, ends = [], []
    if causal:
        starts.append(zero)
        ends.append(j)
    if lts is not None:
        e = np.full(n, nr, np.int64) if lte is None else np.asarray(lte, np.int64)
        starts.append(np.asarray(lts, np.int64))
        ends.append(e)
    if (not causal) and uts is not None and ute is not None:
        starts.append(np.asarray(uts, np.int64))
        ends.append(np.asarray(ute, np.int64))
    if not starts:
        return np.full(n, nr, np.int64)
    s = np.clip(np.stack(starts), 0, nr)
    e = np.clip(np.stack(ends), 0, nr)
    e = np.maximum(s, e)                       # empty interval -> zero length
    order = np.argsort(s, axis=0, kind="stable")
    s = np.take_along_axis(s, order, axis=0)
    e = np.take_along_axis(e, order, axis=0)
    covered = np.zeros(n, np.int64)
    reach = np.zeros(n, np.int64)               # end of the union so far
    for t in range(s.shape[0]):
        lo = np.maximum(s[t], reach)
        covered += np.maximum(0, e[t] - lo)
        reach = np.maximum(reach, e[t])
    return nr - covered


def nnz(B, H, n, causal, lts=None, lte=None, uts=None, ute=None, n_rows=None) -> int:
    """Open pairs summed over all (batch, head); vectors are [B, Hm, n] or None
    over n keys, n_rows query rows (default n)."""
    def row(v, b, h):
        if v is None:
            return None
        v = np.asarray(v)
        return v[b, h if v.shape[1] > 1 else 0]
    hm = np.asarray(lts).shape[1] if lts is not None else (
        np.asarray(uts).shape[1] if uts is not None else 1)
    total = 0
    for b in range(B):
        for h in range(hm):
            c = int(nnz_columns(n, causal, row(lts, b, h), row(lte, b, h),
                                row(uts, b, h), row(ute, b, h), n_rows=n_rows).sum())
            total += c * (H if hm == 1 else 1)
    return total


def fwd_flops(nnz_pairs: int, d: int, dv: int) -> int:
    return 2 * (d + dv) * nnz_pairs


def bwd_flops(nnz_pairs: int, d: int, dv: int) -> int:
    return 2 * (3 * d + 2 * dv) * nnz_pairs
