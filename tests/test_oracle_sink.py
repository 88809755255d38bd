"""Pins of the oracle's sink bias.

The README ("News") names sink bias as a FlashMask feature without defining
it. The reading here (stated in oracle/attention.py): a per-head logit s_h is
one more, always open, entry of every row's softmax with a zero value vector.
Pinned three independent ways: torch SDPA on an augmented problem where one
extra key scores exactly s_h for every row, the closed form relating it to
the no-sink result, and central finite differences for d/ds.
"""
import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle
from sparse_masked_attention_amd import inputs as I


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _problem(n, d, dv, family, seed, H=2):
    vec = I.stack_masks([I.make_mask(family, n, np.random.default_rng(seed))])
    q, k, v, do = (_rand((1, H, n, x), seed + t) for t, x in enumerate((d, d, dv, dv)))
    sink = np.random.default_rng(seed + 9).standard_normal(H) * 2.0
    return q, k, v, do, vec, sink


@pytest.mark.parametrize("family", ["causal", "document", "prefix_lm_document", "all_open"])
def test_sink_equals_sdpa_with_an_extra_key(family):
    """Q' = [Q, 1], K' = [K, 0] plus one key [0, s / scale], V' = [V; 0]:
    every row's extra score is exactly s. SDPA (fp64) on that problem gives
    O, dQ, dK, dV and, through the extra key's last coordinate, d/ds."""
    n, d, dv = 48, 16, 8
    q, k, v, do, vec, sink = _problem(n, d, dv, family, 3)
    lts, lte, uts, ute, causal = vec
    o, lse = oracle.forward(q, k, v, causal, lts, lte, uts, ute, sink=sink)
    dq, dk, dvv, ds = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute, sink=sink)
    sc = 1.0 / np.sqrt(d)
    allowed = ~oracle.dense_mask(n, causal, lts[0, 0], lte[0, 0],
                                 None if uts is None else uts[0, 0], None if ute is None else ute[0, 0])
    for h in range(2):
        tq = torch.tensor(np.c_[q[0, h], np.ones(n)], requires_grad=True)
        kx = np.r_[np.c_[k[0, h], np.zeros(n)], [np.r_[np.zeros(d), sink[h] / sc]]]
        tk = torch.tensor(kx, requires_grad=True)
        tv = torch.tensor(np.r_[v[0, h], np.zeros((1, dv))], requires_grad=True)
        am = torch.from_numpy(np.c_[allowed, np.ones(n, bool)])
        out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None],
                                                               attn_mask=am[None], scale=sc)[0]
        out.backward(torch.from_numpy(do[0, h]))
        np.testing.assert_allclose(o[0, h], out.detach().numpy(), atol=1e-12)
        np.testing.assert_allclose(dq[0, h], tq.grad.numpy()[:, :d], atol=1e-11)
        np.testing.assert_allclose(dk[0, h], tk.grad.numpy()[:n, :d], atol=1e-11)
        np.testing.assert_allclose(dvv[0, h], tv.grad.numpy()[:n], atol=1e-11)
        # s enters as sc * k_extra[-1] * 1, so d/ds = grad(k_extra[-1]) / sc
        np.testing.assert_allclose(ds[h], tk.grad.numpy()[n, d] / sc, atol=1e-10)


@pytest.mark.parametrize("family", ["document", "sliding_window", "share_question"])
def test_sink_closed_form(family):
    """LSE_s = logaddexp(LSE, s) and O_s = O * exp(LSE - LSE_s); rows with
    nothing open: O = 0, LSE = s."""
    n, d, dv = 64, 8, 8
    q, k, v, do, vec, sink = _problem(n, d, dv, family, 5)
    lts, lte, uts, ute, causal = vec
    lte = lte.copy()
    lts = lts.copy()
    lts[0, 0, :] = np.minimum(lts[0, 0, :], 10)       # rows 10 .. 11 see no key
    lte[0, 0, :] = np.maximum(lte[0, 0, :], 12)
    o0, l0 = oracle.forward(q, k, v, causal, lts, lte, uts, ute)
    o1, l1 = oracle.forward(q, k, v, causal, lts, lte, uts, ute, sink=sink)
    for h in range(2):
        want = np.logaddexp(l0[0, h], sink[h])
        np.testing.assert_allclose(l1[0, h], want, atol=1e-12)
        fac = np.exp(np.where(np.isneginf(l0[0, h]), -np.inf, l0[0, h] - want))
        np.testing.assert_allclose(o1[0, h], o0[0, h] * fac[:, None], atol=1e-12)
        assert np.isneginf(l0[0, h, 10:12]).all()
        np.testing.assert_array_equal(o1[0, h, 10:12], 0.0)
        np.testing.assert_allclose(l1[0, h, 10:12], sink[h], atol=0)


def test_sink_gradient_finite_differences():
    n, d, dv = 14, 4, 3
    q, k, v, do, vec, sink = _problem(n, d, dv, "document", 7)
    lts, lte, uts, ute, causal = vec
    loss = lambda s: float((oracle.forward(q, k, v, causal, lts, lte, uts, ute, sink=s)[0] * do).sum())
    _, _, _, ds = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute, sink=sink)
    h = 1e-6
    for t in range(2):
        e = np.zeros(2)
        e[t] = h
        fd = (loss(sink + e) - loss(sink - e)) / (2 * h)
        np.testing.assert_allclose(ds[t], fd, rtol=1e-6, atol=1e-9)


def test_very_negative_sink_is_no_sink():
    n, d, dv = 40, 8, 8
    q, k, v, do, vec, _ = _problem(n, d, dv, "causal", 11)
    lts, lte, uts, ute, causal = vec
    o0, l0 = oracle.forward(q, k, v, causal, lts, lte, uts, ute)
    o1, l1 = oracle.forward(q, k, v, causal, lts, lte, uts, ute, sink=np.full(2, -1e4))
    np.testing.assert_allclose(o1, o0, atol=1e-15)
    np.testing.assert_allclose(l1, l0, atol=1e-12)
    # and the logsumexp is scipy's over the open scores plus the sink
    s = np.full(2, 0.7)
    _, l2 = oracle.forward(q, k, v, causal, lts, lte, uts, ute, sink=s)
    sc = 1 / np.sqrt(d)
    for h in range(2):
        scores = q[0, h] @ k[0, h].T * sc
        allowed = ~oracle.dense_mask(n, causal, lts[0, 0], lte[0, 0])
        for i in range(n):
            np.testing.assert_allclose(l2[0, h, i], logsumexp(np.r_[scores[i][allowed[i]], s[h]]), atol=1e-12)
