"""Parity at the full sizes of the workloads, in the launch configuration the
benchmark times (one call over all heads).

Every output tensor is scanned whole for NaN/Inf on the GPU. Values are
checked against the fp64 oracle:
  * B=1 H=32 N=8192 forward (document, causal, all-open) and backward
    (d = 128: causal, document, share-question, sliding window,
    block-sparse): every row of 4 heads, spread over the XCD groups the
    kernels map heads to (head h runs on XCD h mod 8);
  * backward at d = 256: every row of 2 heads;
  * B=2 H=32 N=16384 and B=1 H=8 N=131072 forward: 1024 stratified rows per
    head on 2 heads of every batch element: the rows where some key column's
    masked interval starts or ends (document, question, answer and prefix
    boundaries, the edges of dropped key blocks), the rows where the vectors
    change along the key axis (the diagonal there), and uniform rows.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm
from gpu_util import BF16_ATOL, check_bf16, check_lse, mask_from, replays, say, to_dev, to_np
from _lib_fixture import ensure_built

pytestmark = pytest.mark.gpu

HEADS_8K = [0, 11, 22, 31]      # XCD groups 0, 3, 6 and 7


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def all_finite(*ts):
    for t in ts:
        assert bool(torch.isfinite(t).all()), "non-finite value in an output tensor"


def stratified_rows(vec, b, n, rng, count=1024):
    """Row indices of batch element b, ``count`` in all: first the rows on
    both sides of every structural edge of the mask, i.e. of every row bound
    shared by many key columns (document, answer and prefix ends, the edges
    of dropped key blocks) and of every key position where a vector's
    pattern breaks (a nonzero second difference: document, question, answer
    and prefix starts, on the diagonal); edges are subsampled to half the
    rows when there are more; then uniform rows."""
    edges = {0, 1, n - 2, n - 1}
    for x in vec[:4]:
        if x is None:
            continue
        col = np.clip(np.asarray(x)[b, 0].astype(np.int64), 0, n)
        vals, cnt = np.unique(col, return_counts=True)
        for t in vals[cnt >= 8]:                       # bounds shared by many columns
            edges.update((int(t) - 1, int(t)))
        brk = np.nonzero(np.diff(col, 2))[0] + 1       # pattern breaks along the keys
        for j in brk:
            edges.update((int(j) - 1, int(j), int(j) + 1))
    e = np.array(sorted(r for r in edges if 0 <= r < n), np.int64)
    if e.size > count // 2:
        e = np.sort(rng.choice(e, count // 2, replace=False))
    rest = np.setdiff1d(np.arange(n), e)
    extra = rng.choice(rest, count - e.size, replace=False)
    return np.sort(np.concatenate([e, extra]))


def fwd_full(cfg, family, d=128):
    c = I.CONFIGS[cfg]
    B, H, N = c["B"], c["H"], c["N"]
    q, k, v = (I.randn((B, H, N, d), I.qkv_seed(cfg, t)) for t in range(3))
    vec = I.config_masks(cfg, family)
    m = mask_from(vec)
    qd, kd, vd = (to_dev(x, torch.bfloat16) for x in (q, k, v))
    o, lse = fm.fwd(qd, kd, vd, m)
    torch.cuda.synchronize()
    all_finite(o)
    assert bool((torch.isfinite(lse) | torch.isneginf(lse)).all())
    return q, k, v, vec, o, lse


def check_rows(q, k, v, vec, o, lse, b, h, rows):
    lts, lte, uts, ute, causal = vec
    ro, rl = oracle.forward_rows(q[b, h], k[b, h], v[b, h], q.shape[2], causal,
                                 oracle.mask_row(lts, b, h), oracle.mask_row(lte, b, h),
                                 oracle.mask_row(uts, b, h), oracle.mask_row(ute, b, h), rows=rows)
    check_bf16(f"O[b{b},h{h}] {len(rows)} rows", to_np(o[b, h])[rows], ro)
    check_lse(to_np(lse[b, h])[rows], rl, BF16_ATOL)


@pytest.mark.parametrize("family", ["document", "causal", "all_open"])
def test_fwd_8k_all_rows_of_four_heads(family):
    say(f"full fwd B1 H32 N8192 family={family}")
    q, k, v, vec, o, lse = fwd_full(2, family)
    rows = np.arange(q.shape[2])
    for h in HEADS_8K:
        check_rows(q, k, v, vec, o, lse, 0, h, rows)


@pytest.mark.parametrize("family", ["share_question", "sliding_window"])
def test_fwd_16k_stratified(family):
    say(f"full fwd B2 H32 N16384 family={family}")
    q, k, v, vec, o, lse = fwd_full(3, family)
    rng = np.random.default_rng(31)
    N = q.shape[2]
    for b in range(q.shape[0]):
        rows = stratified_rows(vec, b, N, rng)
        for h in (5, 26):
            check_rows(q, k, v, vec, o, lse, b, h, rows)


@pytest.mark.parametrize("family", ["prefix_lm_document", "block_sparse"])
def test_fwd_128k_stratified(family):
    say(f"full fwd B1 H8 N131072 family={family}")
    q, k, v, vec, o, lse = fwd_full(4, family)
    rng = np.random.default_rng(41)
    rows = stratified_rows(vec, 0, q.shape[2], rng)
    for h in (2, 7):
        check_rows(q, k, v, vec, o, lse, 0, h, rows)


def bwd_full(family, d, heads):
    c = I.CONFIGS[5]
    B, H, N = c["B"], c["H"], c["N"]
    q, k, v, do = (I.randn((B, H, N, d), I.qkv_seed(5, t)) for t in range(4))
    vec = I.config_masks(5, family)
    m = mask_from(vec)
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    o, lse = fm.fwd(qd, kd, vd, m)
    dq, dk, dv = fm.bwd(qd, kd, vd, o, lse, dod, m)
    torch.cuda.synchronize()
    all_finite(o, dq, dk, dv)
    lts, lte, uts, ute, causal = vec
    for h in heads:
        rq, rk, rv = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute, heads=[(0, h)])
        _, rb = replays(q, k, v, do, vec, heads=[(0, h)])
        one = lambda i: (lambda: rb[i]()[0])
        check_bf16(f"dQ[h{h}]", to_np(dq[0, h]), rq[0, h], replay=one(0))
        check_bf16(f"dK[h{h}]", to_np(dk[0, h]), rk[0, h], replay=one(1))
        check_bf16(f"dV[h{h}]", to_np(dv[0, h]), rv[0, h], replay=one(2))


@pytest.mark.parametrize("family", ["causal", "document", "share_question", "sliding_window",
                                    "block_sparse"])
def test_bwd_8k_d128_all_rows_of_four_heads(family):
    say(f"full bwd B1 H32 N8192 d=128 family={family}")
    bwd_full(family, 128, HEADS_8K)


@pytest.mark.parametrize("family", ["causal", "document", "share_question", "sliding_window",
                                    "block_sparse"])
def test_bwd_8k_d256_all_rows_of_two_heads(family):
    say(f"full bwd B1 H32 N8192 d=256 family={family}")
    bwd_full(family, 256, [1, 30])
