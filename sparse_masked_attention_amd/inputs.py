"""Seeded synthetic inputs: Q/K/V/dO tensors and the four boundary vectors.

This module only *generates inputs*. It draws random numbers and writes mask
families into the column-wise sparse form; it holds none of the attention
arithmetic, so the fp64 oracle and the HIP path can both consume its output
without sharing any of the method.

Column-wise sparse mask (FlashMask README, "Overview"; FlashMask-3 abstract):
for every key column j there are four int32 query-row boundaries. Rows i with
LTS[j] <= i < LTE[j] are masked (lower-triangle interval) and, when the mask is
not causal, rows with UTS[j] <= i < UTE[j] are masked too (upper-triangle
interval). With ``causal`` every j > i is masked as well and UTS/UTE are unused.
Intervals are half-open and 0-based; an empty lower interval is written
[N, N) and an empty upper interval [0, 0).

Family recipes follow the five structured families the FlashMask-3 abstract
names (document, prefix-LM, share-question, sliding-window, block-sparse) plus
causal-only and all-open. Where a recipe needs a detail the pages do not give
(how lengths are split, the exact window edge) the plainest reading is taken;
each is documented on its function.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

__all__ = [
    "Mask", "bf16_round", "bf16_bits", "randn", "qkv_seed",
    "causal_only", "all_open", "causal_document", "prefix_lm_document",
    "prefix_lm_params", "prefix_lm_document_from", "share_question",
    "share_question_lengths", "share_question_from", "sliding_window",
    "block_sparse", "block_sparse_keep", "block_sparse_from",
    "doc_lengths_three", "doc_lengths_loguniform", "random_composition",
    "stack_masks", "CONFIGS", "make_mask", "config_masks", "zigzag_chunks",
    "chunk_rows",
]


@dataclasses.dataclass
class Mask:
    """Four boundary vectors for one batch element (length N each).

    ``uts``/``ute`` are None for causal masks (they would be ignored).
    """
    n: int
    causal: bool
    lts: np.ndarray
    lte: np.ndarray
    uts: Optional[np.ndarray] = None
    ute: Optional[np.ndarray] = None
    name: str = ""


# ---------------------------------------------------------------- tensors

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Float32 array whose values are exactly representable in bfloat16 (RNE)."""
    bits = bf16_bits(x).astype(np.uint32) << 16
    return bits.view(np.float32).reshape(np.shape(x))


def qkv_seed(config: int, tensor: int) -> int:
    """Seed for tensor t (0 Q, 1 K, 2 V, 3 dO) of workload ``config``."""
    return 1000 * config + tensor


def randn(shape, seed: int, bf16: bool = True) -> np.ndarray:
    """i.i.d. N(0, 1) float32 draws, optionally rounded to bf16 values."""
    x = np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)
    return bf16_round(x) if bf16 else x


# ---------------------------------------------------------------- helpers

def random_composition(n: int, parts: int, rng: np.random.Generator,
                       min_part: int = 1) -> List[int]:
    """Split n into ``parts`` positive lengths: distinct sorted cut points drawn
    uniformly from {1..n-1}. ``min_part`` > 1 redraws until every part is long enough."""
    if parts <= 1:
        return [n]
    while True:
        cuts = np.sort(rng.choice(np.arange(1, n), size=parts - 1, replace=False))
        lens = np.diff(np.concatenate([[0], cuts, [n]])).astype(int).tolist()
        if min(lens) >= min_part:
            return lens


def doc_lengths_three(n: int, rng: np.random.Generator) -> List[int]:
    """Three documents whose lengths sum to n: two distinct cut points from {1..n-1}."""
    return random_composition(n, 3, rng)


def doc_lengths_loguniform(n: int, rng: np.random.Generator,
                           lo: int = 128, hi: int = 4096) -> List[int]:
    """Document lengths log-uniform in [lo, hi], resampled until they sum to n.

    A draw L = floor(exp(U(ln lo, ln hi))) is kept if the remainder after it is
    either 0 or at least ``lo``; when the remainder itself is <= hi and a draw
    would leave less than ``lo``, the remainder is taken whole. All lengths lie
    in [lo, hi].
    """
    lens: List[int] = []
    rem = n
    while rem > 0:
        if rem < lo:  # only when n itself is below lo
            lens.append(rem)
            break
        L = int(math.floor(math.exp(rng.uniform(math.log(lo), math.log(hi)))))
        L = min(max(L, lo), hi)
        if L >= rem:
            if rem <= hi:
                lens.append(rem)
                rem = 0
            continue
        if rem - L < lo:
            if rem <= hi:
                lens.append(rem)
                rem = 0
            continue
        lens.append(L)
        rem -= L
    return lens


def _starts_ends(lengths):
    ends = np.cumsum(np.asarray(lengths, dtype=np.int64))
    starts = ends - np.asarray(lengths, dtype=np.int64)
    return starts, ends


def _per_column(n, lengths):
    """Document start and end for every column."""
    starts, ends = _starts_ends(lengths)
    doc = np.repeat(np.arange(len(lengths)), lengths)
    assert doc.shape[0] == n
    return starts[doc], ends[doc]


def _i32(x):
    return np.ascontiguousarray(x, dtype=np.int32)


# ---------------------------------------------------------------- families

def causal_only(n: int) -> Mask:
    """Plain causal mask: no interval, every j > i masked."""
    return Mask(n, True, _i32(np.full(n, n)), _i32(np.full(n, n)), name="causal")


def all_open(n: int) -> Mask:
    """No mask at all (non-causal, both intervals empty)."""
    return Mask(n, False, _i32(np.full(n, n)), _i32(np.full(n, n)),
                _i32(np.zeros(n)), _i32(np.zeros(n)), name="all_open")


def causal_document(n: int, lengths) -> Mask:
    """Causal attention inside each document (packed sequences).

    Column j of document [s, e) is hidden from every row at or after e, so
    LTS = e and LTE = n; causality hides rows before j.
    """
    _, e = _per_column(n, lengths)
    return Mask(n, True, _i32(e), _i32(np.full(n, n)), name="document")


def share_question_lengths(n: int, rng: np.random.Generator,
                           q_lo: int = 512, q_hi: int = 4096,
                           a_lo: int = 2, a_hi: int = 6):
    """Draw (question length, answer lengths) summing to n.

    Reading: question length q ~ U{q_lo..q_hi}, answer count k ~ U{a_lo..a_hi},
    answer lengths a random composition of n - q (the split of answer lengths
    is not given; a uniform composition is the plainest choice).
    """
    q = int(rng.integers(q_lo, q_hi + 1))
    q = min(q, n - a_hi) if n > 2 * a_hi else max(1, n // 2)
    k = int(rng.integers(a_lo, a_hi + 1))
    k = max(1, min(k, n - q))
    return q, random_composition(n - q, k, rng)


def share_question_from(q: int, answers) -> Mask:
    """Encode a share-question mask: each answer sees the question and itself.

    Causal. Question columns carry no interval; a column of answer [s, e) is
    hidden from every row at or after e: LTS = e, LTE = n.
    """
    n = q + int(sum(answers))
    lts = np.full(n, n, dtype=np.int64)
    s = q
    for L in answers:
        lts[s:s + L] = s + L
        s += L
    return Mask(n, True, _i32(lts), _i32(np.full(n, n)), name="share_question")


def share_question(n: int, rng: np.random.Generator) -> Mask:
    q, answers = share_question_lengths(n, rng)
    return share_question_from(q, answers)


def sliding_window(n: int, w: int) -> Mask:
    """Causal sliding window of w keys including the row itself.

    Reading: row i sees keys j with i - w < j <= i. So column j is hidden from
    rows >= j + w: LTS = min(j + w, n), LTE = n.
    """
    j = np.arange(n, dtype=np.int64)
    return Mask(n, True, _i32(np.minimum(j + w, n)), _i32(np.full(n, n)),
                name="sliding_window")


def prefix_lm_params(n: int, rng: np.random.Generator,
                     docs_lo: int = 4, docs_hi: int = 16,
                     frac_lo: float = 0.1, frac_hi: float = 0.5):
    """Draw (document lengths, prefix lengths) for a prefix-LM document mask.

    Reading: k ~ U{docs_lo..docs_hi} documents, lengths a random composition of
    n; per document the prefix is p = max(1, floor(f * L)), f ~ U[frac_lo, frac_hi].
    """
    k = min(int(rng.integers(docs_lo, docs_hi + 1)), n)
    lengths = random_composition(n, k, rng)
    prefixes = [max(1, int(math.floor(rng.uniform(frac_lo, frac_hi) * L)))
                for L in lengths]
    return lengths, prefixes


def prefix_lm_document_from(lengths, prefixes) -> Mask:
    """Encode packed documents with a bidirectional prefix, causal after it.

    Allowed(i, j) = same document and (j <= i or j in the document's prefix).
    Non-causal four-vector encoding, column j of document [s, e): LTS = e,
    LTE = n, UTS = 0, UTE = s for prefix columns and UTE = j otherwise.
    """
    n = int(sum(lengths))
    lts = np.empty(n, np.int64)
    ute = np.empty(n, np.int64)
    s = 0
    for L, p in zip(lengths, prefixes):
        e = s + L
        lts[s:e] = e
        ute[s:s + p] = s
        ute[s + p:e] = np.arange(s + p, e)
        s = e
    return Mask(n, False, _i32(lts), _i32(np.full(n, n)),
                _i32(np.zeros(n)), _i32(ute), name="prefix_lm_document")


def prefix_lm_document(n: int, rng: np.random.Generator) -> Mask:
    lengths, prefixes = prefix_lm_params(n, rng)
    return prefix_lm_document_from(lengths, prefixes)


def block_sparse_keep(n: int, rng: np.random.Generator, block: int = 128,
                      p_keep: float = 0.5) -> np.ndarray:
    """Bernoulli(p_keep) keep flag per key block of ``block`` columns."""
    return rng.random((n + block - 1) // block) < p_keep


def block_sparse_from(n: int, keep, block: int = 128) -> Mask:
    """Encode a causal block-sparse mask from per-key-block keep flags.

    Reading: Bernoulli per (query block, key block) tile cannot be written with
    one lower interval per column, so each *key block* is kept or dropped. A
    dropped key block stays visible only to its own diagonal query block:
    LTS = min(block * (kb + 1), n), LTE = n. Kept blocks are plain causal.
    """
    keep = np.asarray(keep, bool)
    j = np.arange(n, dtype=np.int64)
    kb = j // block
    lts = np.where(keep[kb], n, np.minimum(block * (kb + 1), n))
    return Mask(n, True, _i32(lts), _i32(np.full(n, n)), name="block_sparse")


def block_sparse(n: int, rng: np.random.Generator, block: int = 128,
                 p_keep: float = 0.5) -> Mask:
    return block_sparse_from(n, block_sparse_keep(n, rng, block, p_keep), block)


def stack_masks(masks: List[Mask]):
    """Stack per-batch masks into [B, 1, N] arrays (mask head count 1).

    Returns (lts, lte, uts, ute, causal) with uts/ute None for causal masks.
    """
    causal = masks[0].causal
    assert all(m.causal == causal for m in masks)
    lts = np.stack([m.lts for m in masks])[:, None, :]
    lte = np.stack([m.lte for m in masks])[:, None, :]
    if causal:
        return _i32(lts), _i32(lte), None, None, True
    uts = np.stack([m.uts for m in masks])[:, None, :]
    ute = np.stack([m.ute for m in masks])[:, None, :]
    return _i32(lts), _i32(lte), _i32(uts), _i32(ute), False


# ---------------------------------------------------------------- workloads

# The five synthetic workloads: shapes, dtypes and mask families.
CONFIGS = {
    1: dict(name="tiny_fp32_fwd", B=1, H=2, N=256, d=64, dtype="fp32",
            masks=["document3"], passes=["fwd"]),
    2: dict(name="fwd_8k", B=1, H=32, N=8192, d=128, dtype="bf16",
            masks=["document", "causal", "all_open"], passes=["fwd"]),
    3: dict(name="fwd_16k", B=2, H=32, N=16384, d=128, dtype="bf16",
            masks=["share_question", "sliding_window"], passes=["fwd"]),
    4: dict(name="fwd_128k", B=1, H=8, N=131072, d=128, dtype="bf16",
            masks=["prefix_lm_document", "block_sparse"], passes=["fwd"]),
    5: dict(name="bwd_8k", B=1, H=32, N=8192, d=128, dtype="bf16",
            masks=["causal", "document", "share_question", "sliding_window",
                   "block_sparse"], passes=["bwd"], d_values=[128, 256]),
}


def mask_seed(config: int, s: int, b: int) -> int:
    """Seed of the mask structure for batch element b, mask seed s."""
    return 100 * config + 10 * s + b


def make_mask(family: str, n: int, rng: np.random.Generator) -> Mask:
    """One batch element's mask of the named family at length n.

    Family parameters are those of the 8K-128K workloads (question 512-4096,
    window 1024, 128-column key blocks). Below N = 8192 the question range and
    the window shrink in proportion (n / 8192, at least 8 and 16) so that small
    parity cases keep the same structure instead of degenerating to causal.
    """
    small = n < 8192
    if family == "causal":
        return causal_only(n)
    if family == "all_open":
        return all_open(n)
    if family == "document3":
        return causal_document(n, doc_lengths_three(n, rng))
    if family.startswith("equal_document_"):
        # documents of one length L (the last one shorter when L does not
        # divide n): every key block then sees the same number of rows, which
        # separates a kernel's per-block cost from its per-tile cost
        length = int(family[len("equal_document_"):])
        if length < 1:
            raise ValueError(f"document length must be positive: {family!r}")
        return causal_document(n, [length] * (n // length) + ([n % length] if n % length else []))
    if family == "document":
        if small:
            return causal_document(n, doc_lengths_loguniform(
                n, rng, lo=max(8, n // 64), hi=max(16, n // 2)))
        return causal_document(n, doc_lengths_loguniform(n, rng))
    if family == "share_question":
        if small:
            q, ans = share_question_lengths(n, rng, q_lo=max(8, n // 16),
                                            q_hi=max(9, n // 2))
            return share_question_from(q, ans)
        return share_question(n, rng)
    if family == "sliding_window":
        return sliding_window(n, max(16, n // 8) if small else 1024)
    if family == "prefix_lm_document":
        return prefix_lm_document(n, rng)
    if family == "block_sparse":
        return block_sparse(n, rng)
    raise ValueError(f"unknown mask family {family!r}")


def config_masks(config: int, family: str, s: int = 0, n: Optional[int] = None,
                 batch: Optional[int] = None):
    """Stacked [B,1,N] vectors for workload ``config`` (optionally resized)."""
    c = CONFIGS[config]
    n = c["N"] if n is None else n
    B = c["B"] if batch is None else batch
    ms = [make_mask(family, n, np.random.default_rng(mask_seed(config, s, b)))
          for b in range(B)]
    return stack_masks(ms)


# ---------------------------------------------------------------- rank shares

def zigzag_chunks(n: int, ranks: int, r: int):
    """Query-row chunks of rank r of ``ranks`` in a zig-zag context-parallel
    split (a common way to balance causal work over ranks): the rows are cut
    into 2 * ranks equal pieces and rank r holds pieces r and 2 ranks - 1 - r,
    as sorted (q0, q1) pairs."""
    e = np.linspace(0, n, 2 * ranks + 1).astype(int)
    return sorted([(int(e[r]), int(e[r + 1])), (int(e[2 * ranks - 1 - r]), int(e[2 * ranks - r]))])


def chunk_rows(chunks) -> np.ndarray:
    """Global row of every row a rank holds: its chunks' rows in order (used to
    pick that rank's Q and dO rows)."""
    return np.concatenate([np.arange(int(a), int(b)) for a, b in chunks]).astype(np.int64)
