"""bf16 rounding replay of masked attention (test infrastructure only).

The oracle (attention.py) evaluates the definition exactly in float64. A bf16
implementation cannot: its matrix products take bf16 operands, so the
probabilities P and the score gradients dS are rounded to bf16 before they
are multiplied, and the outputs are stored in bf16. The pages fix no
precision (the FlashMask abstract only says the method is exact, i.e. it
computes the same function); the reading taken for bf16 inputs is that P and
dS are bf16 operands with float32 accumulation and bf16 outputs. This module
evaluates attention and its gradient in float64 except at exactly those
rounding points, to bound the error the bf16 method itself must make on a
given input: the parity tests use it on inputs where that error alone
approaches the absolute tolerance, and require the GPU's error to stay
within a few percent of it.

Rounding points (values are rounded to float32 first, then to bf16 with
round-to-nearest-even, since a bf16 kernel holds them in float32):
  forward:  p = exp(S - m) with m the row max, rounded to bf16; the row sum
            l adds the rounded values; O = bf16((sum_j p_j v_j) / l);
            LSE = m + log(l) (float32), sink logit included when given;
  backward: P = exp(S - LSE) with the replayed LSE; delta_i = dO_i . O_i with
            the replayed bf16 O; dS = P * (dO V^T - delta);
            dV = bf16(bf16(P)^T dO), dK = bf16(scale bf16(dS)^T Q),
            dQ = bf16(scale bf16(dS) K).
With ``rounding=False`` no value is rounded and the results equal the
oracle's (tests/test_oracle_replay.py pins this, the rounding function
against torch's bfloat16 conversion, and an error bound of the forward).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from .attention import dense_mask, mask_row

__all__ = ["round_bf16", "forward", "backward"]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 values rounded to float32, then to bfloat16 (nearest, ties to
    even), returned as float64. Finite inputs only."""
    f = np.ascontiguousarray(np.asarray(x, np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    # keep the high 16 bits: add half an ulp of the kept part, plus one more
    # when the kept part is odd (ties go to the even neighbour)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def _id(x):
    return np.asarray(x, np.float64)


def _head_forward(Q, K, V, masked, scale, sink, rnd):
    s = (Q @ K.T) * scale
    s = np.where(masked, -np.inf, s)
    nq = s.shape[0]
    o = np.zeros((nq, V.shape[1]))
    lse = np.full(nq, -np.inf if sink is None else float(sink))
    for i in range(nq):
        open_ = ~masked[i]
        if not open_.any():
            continue
        m = s[i, open_].max()
        p = rnd(np.exp(s[i, open_] - m))
        l = float(p.sum())
        lse0 = m + math.log(l)
        acc = p @ V[open_]
        if sink is None:
            lse[i] = lse0
            o[i] = acc / l
        else:
            hi = max(lse0, float(sink))
            lse[i] = hi + math.log1p(math.exp(-abs(lse0 - float(sink))))
            o[i] = acc / l * math.exp(lse0 - lse[i])
    return rnd(o), lse.astype(np.float32).astype(np.float64)


def forward(q, k, v, causal, lts=None, lte=None, uts=None, ute=None, scale=None,
            sink=None, rounding: bool = True):
    """(O [B,H,Nq,dv], LSE [B,H,Nq]) with the forward's bf16 rounding points."""
    rnd = round_bf16 if rounding else _id
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = np.zeros((B, H, Nq, v.shape[-1]))
    lse = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            msk = dense_mask(Nk, causal, mask_row(lts, b, h), mask_row(lte, b, h),
                             mask_row(uts, b, h), mask_row(ute, b, h), n_rows=Nq)
            o[b, h], lse[b, h] = _head_forward(
                np.asarray(q[b, h], np.float64), np.asarray(k[b, h], np.float64),
                np.asarray(v[b, h], np.float64), msk, sc,
                None if sink is None else float(sink[h]), rnd)
    return o, lse


def backward(q, k, v, do, causal, lts=None, lte=None, uts=None, ute=None, scale=None,
             sink=None, rounding: bool = True):
    """(dQ, dK, dV) with the bf16 rounding points, from the replayed forward's
    O and LSE (as a user passes the forward's outputs to the backward)."""
    rnd = round_bf16 if rounding else _id
    o, lse = forward(q, k, v, causal, lts, lte, uts, ute, scale, sink, rounding)
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = np.zeros((B, H, Nq, d))
    dk = np.zeros((B, H, Nk, d))
    dv = np.zeros((B, H, Nk, v.shape[-1]))
    for b in range(B):
        for h in range(H):
            Q, K, V, dO = (np.asarray(x[b, h], np.float64) for x in (q, k, v, do))
            msk = dense_mask(Nk, causal, mask_row(lts, b, h), mask_row(lte, b, h),
                             mask_row(uts, b, h), mask_row(ute, b, h), n_rows=Nq)
            s = np.where(msk, -np.inf, (Q @ K.T) * sc)
            L = lse[b, h][:, None]
            P = np.where(np.isneginf(L) | msk, 0.0, np.exp(s - np.where(np.isneginf(L), 0.0, L)))
            delta = (dO * o[b, h]).sum(axis=1)
            dS = P * ((dO @ V.T) - delta[:, None])
            Pr, dSr = rnd(P), rnd(dS)
            dv[b, h] = rnd(Pr.T @ dO)
            dk[b, h] = rnd(sc * (dSr.T @ Q))
            dq[b, h] = rnd(sc * (dSr @ K))
    return dq, dk, dv
