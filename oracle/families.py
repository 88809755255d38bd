"""Mask families written as dense predicates, from their definitions (test infrastructure).

These are independent of the boundary-vector encoders that generate inputs:
each predicate says which (row i, column j) pairs may attend, straight from
the family's description in the FlashMask-3 abstract (document, prefix-LM,
share-question, sliding-window, block-sparse) plus causal and all-open. A
test decodes an encoder's vectors with the oracle and compares the result to
these predicates, so a mistake in either side shows up.

Each function returns ``allowed`` [N, N] (True = may attend).
"""
from __future__ import annotations

import numpy as np

__all__ = ["causal", "all_open", "causal_document", "share_question",
           "sliding_window", "prefix_lm_document", "block_sparse"]


def _ij(n):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return i, j


def _doc_ids(lengths):
    return np.repeat(np.arange(len(lengths)), lengths)


def causal(n):
    i, j = _ij(n)
    return j <= i


def all_open(n):
    return np.ones((n, n), bool)


def causal_document(lengths):
    """Causal attention restricted to the row's own document."""
    doc = _doc_ids(lengths)
    n = doc.shape[0]
    i, j = _ij(n)
    return (doc[:, None] == doc[None, :]) & (j <= i)


def share_question(q_len, answer_lengths):
    """Question tokens attend causally to the question; each answer token
    attends to the whole question and causally to its own answer."""
    n = q_len + sum(answer_lengths)
    seg = np.concatenate([np.zeros(q_len, int)] +
                         [np.full(L, a + 1) for a, L in enumerate(answer_lengths)])
    i, j = _ij(n)
    same = seg[:, None] == seg[None, :]
    col_in_question = (seg == 0)[None, :]
    return (j <= i) & (same | col_in_question)


def sliding_window(n, w):
    """Row i sees the w most recent keys including itself: i - w < j <= i."""
    i, j = _ij(n)
    return (j <= i) & (j > i - w)


def prefix_lm_document(lengths, prefixes):
    """Per document: the first p keys are seen by every row of the document,
    the rest causally; nothing crosses documents."""
    doc = _doc_ids(lengths)
    n = doc.shape[0]
    starts = np.cumsum([0] + list(lengths[:-1]))
    prefix_end = (starts + np.asarray(prefixes))[doc]   # s + p of the column's document
    i, j = _ij(n)
    same = doc[:, None] == doc[None, :]
    return same & ((j <= i) | (j < prefix_end[None, :]))


def block_sparse(n, block, keep):
    """Causal; a dropped key block is seen only by its own query block."""
    i, j = _ij(n)
    kb = np.arange(n) // block
    qb = np.arange(n) // block
    kept = np.asarray(keep)[kb][None, :]
    return (j <= i) & (kept | (qb[:, None] == kb[None, :]))
