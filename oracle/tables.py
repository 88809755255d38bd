"""Oracle of the block tables and tile classes (test infrastructure only).

FlashMask uses its column-wise representation to skip work the mask makes
unnecessary (README "News" and "Overview"; FlashMask abstract). The skipping
rule used here: reduce each boundary vector to its min and max over a block
of key columns, then call a (query block, key block) tile

  * fully masked when the causal edge hides it (c0 > r1 - 1), or every column
    hides every row through the lower interval (max LTS <= r0 and
    min LTE >= r1), or, non-causal, through the upper interval
    (max UTS <= r0 and min UTE >= r1);
  * unmasked when neither causality (causal and c1 - 1 > r0), nor the lower
    interval (max LTE > r0 and min LTS < r1), nor, non-causal, the upper
    interval (max UTE > r0 and min UTS < r1) can reach any element;
  * partial otherwise,

with rows [r0, r1) and columns [c0, c1) clipped to N. Classes: 0 masked
(skip), 1 partial, 2 unmasked. The rule is conservative: it never calls a
tile masked or unmasked wrongly, but may call a tile partial that is not.

Missing vectors take their neutral values in the table: no lower interval ->
LTS = LTE = N; LTE missing -> LTE = N; no upper interval -> UTS = UTE = 0.
"""
from __future__ import annotations

import numpy as np

__all__ = ["kblock_minmax", "classify", "classify_counts", "nnz_dense"]


def _full(vec, B, hm, n, fill):
    if vec is None:
        return np.full((B, hm, n), fill, np.int64)
    return np.asarray(vec, np.int64)


def _neutral(lts, lte, uts, ute, B, hm, n, n_rows):
    """The four [B, Hm, n] vectors with neutral values where one is missing
    (the empty lower interval is [n_rows, n_rows), n_rows query rows)."""
    if lts is None:
        LTS = np.full((B, hm, n), n_rows, np.int64)
        LTE = np.full((B, hm, n), n_rows, np.int64)
    else:
        LTS = np.asarray(lts, np.int64)
        LTE = _full(lte, B, hm, n, n_rows)
    if uts is None or ute is None:
        UTS = np.zeros((B, hm, n), np.int64)
        UTE = np.zeros((B, hm, n), np.int64)
    else:
        UTS = np.asarray(uts, np.int64)
        UTE = np.asarray(ute, np.int64)
    return LTS, LTE, UTS, UTE


def kblock_minmax(B, hm, n, block, lts=None, lte=None, uts=None, ute=None, n_rows=None):
    """int32 [B, Hm, ceil(n/block), 8] table over n key columns.

    Entry order: LTS min, LTS max, LTE min, LTE max, UTS min, UTS max,
    UTE min, UTE max, each over columns [kb*block, min(n, (kb+1)*block)).
    Missing vectors take neutral values for n_rows query rows (default n).
    Plain loops over key blocks.
    """
    vecs = _neutral(lts, lte, uts, ute, B, hm, n, n if n_rows is None else int(n_rows))
    nkb = (n + block - 1) // block
    out = np.zeros((B, hm, nkb, 8), np.int64)
    for kb in range(nkb):
        c0, c1 = kb * block, min(n, (kb + 1) * block)
        for t, v in enumerate(vecs):
            seg = v[:, :, c0:c1]
            out[:, :, kb, 2 * t] = seg.min(axis=2)
            out[:, :, kb, 2 * t + 1] = seg.max(axis=2)
    return out.astype(np.int32)


def classify(table, n, block_q, block_k, causal, n_rows=None):
    """int8 [B, Hm, ceil(n_rows/block_q), ceil(n/block_k)] tile classes.

    ``table`` must be the kblock_minmax table at granularity block_k over n
    key columns; there are n_rows query rows (default n). The rule of the
    module docstring is evaluated for every (query block, key block) pair at
    once with numpy broadcasting: rows index query blocks, columns key blocks.
    """
    t = np.asarray(table, np.int64)
    B, hm, nkb, _ = t.shape
    nr = n if n_rows is None else int(n_rows)
    nqb = (nr + block_q - 1) // block_q
    r0 = (np.arange(nqb, dtype=np.int64) * block_q)[:, None]
    r1 = np.minimum(nr, r0 + block_q)
    c0 = (np.arange(nkb, dtype=np.int64) * block_k)[None, :]
    c1 = np.minimum(n, c0 + block_k)
    out = np.zeros((B, hm, nqb, nkb), np.int8)
    for b in range(B):
        for h in range(hm):
            lts_mn, lts_mx, lte_mn, lte_mx, uts_mn, uts_mx, ute_mn, ute_mx = \
                (t[b, h, :, e][None, :] for e in range(8))
            full = (lts_mx <= r0) & (lte_mn >= r1)
            if causal:
                full |= c0 > r1 - 1
            else:
                full |= (uts_mx <= r0) & (ute_mn >= r1)
            causal_free = (c1 - 1 <= r0) if causal else np.ones_like(full)
            lt_free = (lte_mx <= r0) | (lts_mn >= r1)
            ut_free = np.ones_like(full) if causal else ((ute_mx <= r0) | (uts_mn >= r1))
            none = causal_free & lt_free & ut_free
            out[b, h] = np.where(full, 0, np.where(none, 2, 1))
    return out


def classify_counts(classes) -> np.ndarray:
    """Histogram [masked, partial, unmasked] of a class map."""
    c = np.asarray(classes)
    return np.array([(c == 0).sum(), (c == 1).sum(), (c == 2).sum()], np.int64)


def nnz_dense(masked: np.ndarray) -> int:
    """Count of unmasked (i, j) pairs of a dense boolean mask."""
    return int(masked.size - np.count_nonzero(masked))
