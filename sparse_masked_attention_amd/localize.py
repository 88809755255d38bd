"""Boundary vectors of one context-parallel rank's share of the query rows.

The FlashMask-3 abstract has each rank localise the column-wise mask without
communication ("clip-shift-max"): the rank holds some chunks of the global
query rows and all keys, and every row bound stored per key column is mapped
to the rank's local row numbering. With the rank's chunks [q0_c, q1_c)
(sorted, disjoint; local rows are the chunks' rows in order), a global row
bound t maps to

    local(t) = sum_c clip(t - q0_c, 0, q1_c - q0_c)

(shift by the chunk start, clip to the chunk, add up). The map is monotone,
so a global half-open interval [a, b) of rows becomes [local(a), local(b))
over exactly the local rows it contained. A causal mask's edge (global rows
i < j masked for key j) becomes the upper interval [0, local(j)), so the local
mask is always the non-causal four-vector form.

Host-side numpy (this module) and the library's `flashmask_localize` compute
the same integers.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

__all__ = ["check_chunks", "local_rows", "localize"]


def check_chunks(chunks: Sequence[Tuple[int, int]], n_rows: int) -> np.ndarray:
    """int64 [C, 2] chunk array; raises unless sorted, disjoint, non-empty and
    inside [0, n_rows]."""
    c = np.asarray(chunks, np.int64).reshape(-1, 2)
    if c.shape[0] == 0:
        raise ValueError("no chunks")
    if (c[:, 0] < 0).any() or (c[:, 1] > n_rows).any() or (c[:, 1] <= c[:, 0]).any():
        raise ValueError("chunks must be non-empty ranges inside [0, n_rows]")
    if (c[1:, 0] < c[:-1, 1]).any():
        raise ValueError("chunks must be sorted and disjoint")
    return c


def local_rows(chunks, n_rows: int) -> np.ndarray:
    """Global row index of every local row, in local order."""
    c = check_chunks(chunks, n_rows)
    return np.concatenate([np.arange(a, b) for a, b in c])


def _map(t: np.ndarray, c: np.ndarray) -> np.ndarray:
    t = np.asarray(t, np.int64)
    out = np.zeros(t.shape, np.int64)
    for a, b in c:
        out += np.clip(t - a, 0, b - a)
    return out


def localize(lts: Optional[np.ndarray], lte: Optional[np.ndarray], uts: Optional[np.ndarray],
             ute: Optional[np.ndarray], causal: bool, chunks, n_rows: int):
    """Local (lts, lte, uts, ute) int32 arrays (same shape as the inputs,
    [B, hm, Nk]) and the local causal flag (always False).

    Absent vectors follow the library's conventions (lts None: no lower
    interval; lte None: LTE = n_rows; non-causal uts/ute None: no upper
    interval); the outputs are always all four, with empty intervals
    ([Nq, Nq) and [0, 0)) where nothing is masked.
    """
    c = check_chunks(chunks, n_rows)
    nq = int((c[:, 1] - c[:, 0]).sum())
    ref = next(v for v in (lts, uts, ute, lte) if v is not None) if any(
        v is not None for v in (lts, uts, ute, lte)) else None
    if ref is None:
        raise ValueError("shape unknown: pass at least one vector")
    shape = np.asarray(ref).shape
    nk = shape[-1]
    if lts is None:
        l_lts = np.full(shape, nq, np.int64)
        l_lte = np.full(shape, nq, np.int64)
    else:
        l_lts = _map(lts, c)
        l_lte = _map(np.full(shape, n_rows, np.int64) if lte is None else lte, c)
    if causal:
        j = np.broadcast_to(np.arange(nk, dtype=np.int64), shape)
        l_uts = np.zeros(shape, np.int64)
        l_ute = _map(j, c)
    elif uts is not None and ute is not None:
        l_uts = _map(uts, c)
        l_ute = _map(ute, c)
    else:
        l_uts = np.zeros(shape, np.int64)
        l_ute = np.zeros(shape, np.int64)
    return (l_lts.astype(np.int32), l_lte.astype(np.int32), l_uts.astype(np.int32),
            l_ute.astype(np.int32), False)
