"""fp64 CPU oracle of column-wise sparse masked attention (test infrastructure).

Only tests, the smoke check and the CPU-baseline leg of the benchmark use this
module; the library never calls it. It shares no code with the HIP path.

What it computes is the plain definition from the FlashMask README
("Formulation"): O = softmax(Q K^T / sqrt(d) + M) V, where d is the last
dimension of Q, and M is the column-wise sparse mask of the README "Overview"
and the FlashMask-3 abstract: for each key column j, four query-row
boundaries (LTS, LTE, UTS, UTE). The mask is materialised densely here (the
O(N^2) form the FlashMask abstract says previous approaches needed), then
softmax attention and its analytic gradient are evaluated in float64.

Readings of points the pages leave open:
  * intervals are half-open [start, end) over 0-based query rows;
  * masked(i, j) = (causal and j > i) or LTS[j] <= i < LTE[j]
                   or (not causal and UTS[j] <= i < UTE[j]);
  * a masked score is -inf (zero probability);
  * a row with every key masked outputs 0, its logsumexp is -inf and it
    contributes no gradient;
  * the scale is 1/sqrt(d) with d the Q/K head dim (not the V head dim);
  * lts None -> no lower interval; lte None -> LTE = the number of query
    rows; uts/ute None (non-causal) -> no upper interval;
  * with Nq query rows and Nk keys (one context-parallel rank's share of the
    rows, FlashMask-3 abstract) the vectors have Nk entries and hold bounds
    on the Nq local rows; the causal test stays j > i in local indices;
  * sink bias (named in the README "News", not defined there): a per-head
    logit s_h joins every row's softmax as one more, always open, entry with
    a zero value vector, in the units of the scaled scores:
    LSE_i = log(exp(s_h) + sum_open exp(S_ij)), P_ij = exp(S_ij - LSE_i),
    O_i = sum_j P_ij V_j. A row with nothing open has O = 0 and LSE = s_h.
    dL/ds_h = -sum_i exp(s_h - LSE_i) * (dO_i . O_i).

Vectors are [B, Hm, N] with Hm in {1, H}; head h uses mask row h if Hm == H,
else row 0.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

__all__ = ["dense_mask", "mask_row", "forward", "forward_rows", "backward",
           "backward_sampled", "softmax_probs"]


def mask_row(vec: Optional[np.ndarray], b: int, h: int) -> Optional[np.ndarray]:
    """The [N] boundary vector that head h of batch b uses (None stays None)."""
    if vec is None:
        return None
    v = np.asarray(vec)
    hm = v.shape[1]
    return v[b, h if hm > 1 else 0].astype(np.int64)


def dense_mask(n: int, causal: bool, lts=None, lte=None, uts=None, ute=None,
               rows: Optional[np.ndarray] = None, n_rows: Optional[int] = None) -> np.ndarray:
    """Boolean masked[i, j] for rows i (default all) and all columns j.

    Arguments are the [n] vectors of one (batch, head): n keys (columns);
    there are n_rows query rows (default n). Follows the interval test stated
    in the module docstring, term by term.
    """
    nr = n if n_rows is None else int(n_rows)
    i = np.arange(nr, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    I = i[:, None]
    J = np.arange(n, dtype=np.int64)[None, :]
    m = np.zeros((I.shape[0], n), dtype=bool)
    if causal:
        m |= J > I
    if lts is not None:
        end = np.full(n, nr, np.int64) if lte is None else np.asarray(lte, np.int64)
        m |= (np.asarray(lts, np.int64)[None, :] <= I) & (I < end[None, :])
    if not causal and uts is not None and ute is not None:
        m |= (np.asarray(uts, np.int64)[None, :] <= I) & (I < np.asarray(ute, np.int64)[None, :])
    return m


def _scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def softmax_probs(q: np.ndarray, k: np.ndarray, masked: np.ndarray, scale: float,
                  sink: Optional[float] = None):
    """Row-wise masked softmax of scale * q k^T for one (batch, head).

    q [R, d], k [N, d] in float64, masked [R, N]. Returns (P [R, N], lse [R]);
    rows with every key masked get P = 0 and lse = -inf (lse = sink with a
    sink logit, which takes part in every row's normaliser).
    """
    s = (q @ k.T) * scale
    s = np.where(masked, -np.inf, s)
    if sink is not None:
        # the sink as one more column, always open, with a zero value vector
        s = np.concatenate([s, np.full((s.shape[0], 1), float(sink))], axis=1)
    empty = np.isneginf(s).all(axis=1)
    m = np.where(empty, 0.0, s.max(axis=1))
    p = np.exp(s - m[:, None])          # exp(-inf) = 0 on masked entries
    l = p.sum(axis=1)
    l_safe = np.where(empty, 1.0, l)
    P = p / l_safe[:, None]
    lse = np.where(empty, -np.inf, m + np.log(l_safe))
    if sink is not None:
        P = P[:, :-1]                   # the sink's probability multiplies a zero value
    return P, lse


def forward_rows(q, k, v, n, causal, lts=None, lte=None, uts=None, ute=None,
                 rows=None, scale=None, chunk: int = 1024, sink: Optional[float] = None):
    """Forward of one (batch, head) for the given query rows.

    q [Nq, d], k [n, d], v [n, dv] (any float dtype, widened exactly to fp64);
    n is the number of keys, the query rows number q.shape[0]. Returns
    (O [R, dv], lse [R]). Rows are processed in chunks so that long sequences
    never hold an Nq x n matrix.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    sc = _scale(q.shape[-1], scale)
    nq = q.shape[0]
    rows = np.arange(nq) if rows is None else np.asarray(rows, np.int64)
    o = np.zeros((rows.shape[0], v.shape[-1]))
    lse = np.zeros(rows.shape[0])
    for c0 in range(0, rows.shape[0], chunk):
        r = rows[c0:c0 + chunk]
        msk = dense_mask(n, causal, lts, lte, uts, ute, rows=r, n_rows=nq)
        P, l = softmax_probs(q[r], k, msk, sc, sink)
        o[c0:c0 + chunk] = P @ v
        lse[c0:c0 + chunk] = l
    return o, lse


def forward(q, k, v, causal, lts=None, lte=None, uts=None, ute=None,
            scale=None, heads=None, sink=None) -> Tuple[np.ndarray, np.ndarray]:
    """O [B,H,Nq,dv] and logsumexp [B,H,Nq] (natural log, scale included).

    q [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,dv], vectors [B,Hm,Nk], sink
    optional [H] logits. ``heads``: optional list of (b, h) pairs to
    evaluate; other entries stay 0.
    """
    B, H, Nq, _ = q.shape
    Nk = k.shape[2]
    dv = v.shape[-1]
    o = np.zeros((B, H, Nq, dv))
    lse = np.zeros((B, H, Nq))
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        o[b, h], lse[b, h] = forward_rows(
            q[b, h], k[b, h], v[b, h], Nk, causal,
            mask_row(lts, b, h), mask_row(lte, b, h),
            mask_row(uts, b, h), mask_row(ute, b, h), scale=scale,
            sink=None if sink is None else float(sink[h]))
    return o, lse


def backward(q, k, v, do, causal, lts=None, lte=None, uts=None, ute=None,
             scale=None, heads=None, sink=None):
    """Analytic gradients (dQ, dK, dV) of O = softmax(scale Q K^T + M) V given dO,
    and with ``sink`` ([H] logits) also dsink [H].

    With P the masked softmax and dP = dO V^T:
      dV = P^T dO,  dS = P * (dP - rowsum(P * dP)),  dQ = scale dS K,
      dK = scale dS^T Q,  dsink_h = -sum_i P_sink,i * rowsum(P * dP)_i,
    where P_sink,i = exp(s_h - LSE_i) is the sink's share of row i and
    rowsum(P * dP) = dO_i . O_i. Rows with every key masked have P = 0 and so
    contribute nothing.
    """
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dv_ = v.shape[-1]
    dq = np.zeros((B, H, Nq, d))
    dk = np.zeros((B, H, Nk, d))
    dvv = np.zeros((B, H, Nk, dv_))
    sc = _scale(d, scale)
    dsink = np.zeros(H)
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        Q = np.asarray(q[b, h], np.float64)
        K = np.asarray(k[b, h], np.float64)
        V = np.asarray(v[b, h], np.float64)
        dO = np.asarray(do[b, h], np.float64)
        msk = dense_mask(Nk, causal, mask_row(lts, b, h), mask_row(lte, b, h),
                         mask_row(uts, b, h), mask_row(ute, b, h), n_rows=Nq)
        s_h = None if sink is None else float(sink[h])
        P, lse = softmax_probs(Q, K, msk, sc, s_h)
        del msk
        dvv[b, h] = P.T @ dO
        dP = dO @ V.T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        del dP, P
        dq[b, h] = sc * (dS @ K)
        dk[b, h] = sc * (dS.T @ Q)
        if s_h is not None:
            dsink[h] -= float((np.exp(s_h - lse) * D).sum())
    if sink is not None:
        return dq, dk, dvv, dsink
    return dq, dk, dvv


def backward_sampled(q, k, v, do, causal, lts=None, lte=None, uts=None, ute=None,
                     rows=(), keys=(), scale=None, chunk: int = 1024):
    """dQ at the given query rows and dK, dV at the given key columns of one
    (batch, head), with the gradient formulas of ``backward``, for sequences
    too long for its dense Nq x Nk matrices.

    q [Nq, d], k [Nk, d], v [Nk, dv], do [Nq, dv]; vectors [Nk]. Every row
    contributes to dK and dV, so all rows are evaluated, ``chunk`` rows at a
    time (as in forward_rows). Within a chunk, a key column that is masked in
    every row of the chunk has probability exactly 0 in all of them and is
    left out of that chunk's softmax: the values are those over all columns.
    Returns (dq [len(rows), d], dk [len(keys), d], dv [len(keys), dv]).
    """
    Q = np.asarray(q, np.float64)
    K = np.asarray(k, np.float64)
    V = np.asarray(v, np.float64)
    dO = np.asarray(do, np.float64)
    nq, d = Q.shape
    n = K.shape[0]
    sc = _scale(d, scale)
    rows = np.asarray(rows, np.int64)
    keys = np.asarray(keys, np.int64)
    dq = np.zeros((rows.shape[0], d))
    dk = np.zeros((keys.shape[0], d))
    dvv = np.zeros((keys.shape[0], V.shape[1]))
    for c0 in range(0, nq, chunk):
        r = np.arange(c0, min(nq, c0 + chunk))
        msk = dense_mask(n, causal, lts, lte, uts, ute, rows=r, n_rows=nq)
        cols = np.nonzero(~msk.all(axis=0))[0]
        if cols.size == 0:
            continue                      # every row of the chunk sees nothing
        P, _ = softmax_probs(Q[r], K[cols], msk[:, cols], sc)
        dP = dO[r] @ V[cols].T
        D = (P * dP).sum(axis=1)
        dS = P * (dP - D[:, None])
        # the requested keys among this chunk's columns
        at = np.searchsorted(cols, keys)
        hit = (at < cols.size) & (cols[np.minimum(at, cols.size - 1)] == keys)
        if hit.any():
            dvv[hit] += P[:, at[hit]].T @ dO[r]
            dk[hit] += sc * (dS[:, at[hit]].T @ Q[r])
        # the requested rows within this chunk
        inside = (rows >= c0) & (rows < c0 + r.shape[0])
        if inside.any():
            dq[inside] = sc * (dS[rows[inside] - c0] @ K[cols])
    return dq, dk, dvv
