"""Pins of the oracle with Nq query rows against Nk keys, and of the row
localisation of one context-parallel rank's share (FlashMask-3 abstract:
each rank localises the column-wise mask without communication).

The square oracle is pinned elsewhere (SDPA, finite differences, closed
forms). These tests tie the rectangular case to it: a rank's local mask must
equal the rows it holds of the global mask, its forward the global forward on
those rows, and the sum of all ranks' dK/dV the global dK/dV. torch's SDPA
with a rectangular boolean mask is an independent second check.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I

pytestmark = pytest.mark.filterwarnings("ignore")

FAMILIES = ["causal", "document", "share_question", "sliding_window", "block_sparse",
            "prefix_lm_document", "all_open"]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _vec1(vec):
    lts, lte, uts, ute, causal = vec
    f = lambda x: None if x is None else np.asarray(x)[0, 0]
    return f(lts), f(lte), f(uts), f(ute), causal


def _chunkings(rng, n):
    """A few ways to cut [0, n) into ranks: contiguous, zig-zag pairs, random."""
    out = []
    r = 4
    edges = np.linspace(0, n, r + 1).astype(int)
    out.append([[(edges[i], edges[i + 1])] for i in range(r)])
    pieces = np.linspace(0, n, 2 * r + 1).astype(int)
    out.append([[(pieces[i], pieces[i + 1]), (pieces[2 * r - 1 - i], pieces[2 * r - i])]
                for i in range(r)])
    cuts = np.sort(rng.choice(np.arange(1, n), size=5, replace=False))
    segs = list(zip(np.r_[0, cuts], np.r_[cuts, n]))
    out.append([[segs[i] for i in range(len(segs)) if i % 2 == k] for k in range(2)])
    return [[sorted((int(a), int(b)) for a, b in ch) for ch in part] for part in out]


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("seed", range(3))
def test_local_mask_is_the_rows_it_holds(family, seed):
    n = 96
    rng = np.random.default_rng(seed)
    vec = I.stack_masks([I.make_mask(family, n, rng)])
    lts, lte, uts, ute, causal = _vec1(vec)
    glob = oracle.dense_mask(n, causal, lts, lte, uts, ute)
    for part in _chunkings(rng, n):
        for ch in part:
            l4 = oracle.localize(*vec[:4], causal, ch, n)
            rows = oracle.rank_rows(ch, n)
            loc = oracle.dense_mask(n, False, *[x[0, 0] for x in l4[:4]], n_rows=len(rows))
            np.testing.assert_array_equal(loc, glob[rows])


@pytest.mark.parametrize("seed", range(4))
def test_local_bound_counts_the_rows_before(seed):
    """local(t) is the number of the rank's rows that lie before global row t
    (brute force over every t, also outside [0, n])."""
    rng = np.random.default_rng(400 + seed)
    n = int(rng.integers(2, 90))
    for part in _chunkings(rng, n):
        for ch in part:
            rows = oracle.rank_rows(ch, n)
            for t in range(-4, n + 5):
                assert oracle.local_bound(t, ch) == int((rows < t).sum())


def test_localize_matches_numpy_clip_form():
    """The plain loops of oracle.localize against the closed clip form written
    with numpy broadcasting (same reading, independent code)."""
    rng = np.random.default_rng(9)
    n = 200
    v = [rng.integers(-300, 300, (2, 1, n)).astype(np.int32) for _ in range(4)]
    ch = [(5, 40), (90, 91), (120, 200)]
    a = np.array([c[0] for c in ch])[:, None, None, None]
    ln = np.array([c[1] - c[0] for c in ch])[:, None, None, None]
    clip = lambda t: np.clip(t[None].astype(np.int64) - a, 0, ln).sum(axis=0)
    for causal in (True, False):
        got = oracle.localize(*v, causal, ch, n)
        np.testing.assert_array_equal(got[0], clip(v[0]))
        np.testing.assert_array_equal(got[1], clip(v[1]))
        if causal:
            np.testing.assert_array_equal(got[2], 0)
            np.testing.assert_array_equal(got[3], clip(np.broadcast_to(np.arange(n), v[0].shape)))
        else:
            np.testing.assert_array_equal(got[2], clip(v[2]))
            np.testing.assert_array_equal(got[3], clip(v[3]))


@pytest.mark.parametrize("seed", range(6))
def test_localisation_on_arbitrary_int32_bounds(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(2, 120))
    v = [rng.integers(-30, n + 30, n).astype(np.int32) for _ in range(4)]
    for causal in (True, False):
        glob = oracle.dense_mask(n, causal, *v)
        for part in _chunkings(rng, n):
            for ch in part:
                l4 = oracle.localize(*[x[None, None] for x in v], causal, ch, n)
                rows = oracle.rank_rows(ch, n)
                loc = oracle.dense_mask(n, False, *[x[0, 0] for x in l4[:4]], n_rows=len(rows))
                np.testing.assert_array_equal(loc, glob[rows])


@pytest.mark.parametrize("family", ["causal", "document", "prefix_lm_document", "share_question"])
def test_rank_forward_and_backward_recompose_the_global_ones(family):
    B, H, n, d, dv = 1, 2, 80, 16, 8
    rng = np.random.default_rng(7)
    vec = I.stack_masks([I.make_mask(family, n, rng)])
    q, k, v, do = _rand((B, H, n, d), 1), _rand((B, H, n, d), 2), _rand((B, H, n, dv), 3), _rand((B, H, n, dv), 4)
    lts, lte, uts, ute, causal = vec
    go, gl = oracle.forward(q, k, v, causal, lts, lte, uts, ute)
    gq, gk, gv = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute)
    for part in _chunkings(rng, n):
        sk, sv = np.zeros_like(gk), np.zeros_like(gv)
        for ch in part:
            rows = oracle.rank_rows(ch, n)
            l4 = oracle.localize(lts, lte, uts, ute, causal, ch, n)
            lo, ll = oracle.forward(q[:, :, rows], k, v, False, *l4[:4])
            np.testing.assert_allclose(lo, go[:, :, rows], atol=1e-12)
            np.testing.assert_array_equal(np.isneginf(ll), np.isneginf(gl[:, :, rows]))
            fin = np.isfinite(ll)
            np.testing.assert_allclose(ll[fin], gl[:, :, rows][fin], atol=1e-12)
            lq, lk, lv = oracle.backward(q[:, :, rows], k, v, do[:, :, rows], False, *l4[:4])
            np.testing.assert_allclose(lq, gq[:, :, rows], atol=1e-12)
            sk += lk
            sv += lv
        np.testing.assert_allclose(sk, gk, atol=1e-11)
        np.testing.assert_allclose(sv, gv, atol=1e-11)


@pytest.mark.parametrize("nq,nk,causal", [(37, 53, False), (53, 37, False), (40, 40, True), (23, 61, True)])
def test_rectangular_matches_sdpa(nq, nk, causal):
    """Independent library check: SDPA (fp64, CPU) with the rectangular mask
    decoded by the oracle, forward and gradients; rows without an open key
    are compared separately (SDPA gives NaN there, the definition 0)."""
    d, dv = 16, 8
    rng = np.random.default_rng(nq * 1000 + nk)
    c = rng.integers(-5, nq + 5, nk)
    w = rng.integers(0, nq // 2 + 1, nk)
    lts, lte = (c - w).astype(np.int32), (c + w // 2).astype(np.int32)
    # every key hides row nq // 2, so one row has nothing open
    r0 = nq // 2
    lts, lte = np.minimum(lts, r0).astype(np.int32), np.maximum(lte, r0 + 1).astype(np.int32)
    uts, ute = np.zeros(nk, np.int32), rng.integers(0, nq // 3 + 1, nk).astype(np.int32)
    q, k, v, do = _rand((1, 1, nq, d), 11), _rand((1, 1, nk, d), 12), _rand((1, 1, nk, dv), 13), _rand((1, 1, nq, dv), 14)
    vec = [x[None, None] for x in (lts, lte, uts, ute)]
    o, lse = oracle.forward(q, k, v, causal, *vec)
    dq, dk, dvv = oracle.backward(q, k, v, do, causal, *vec)
    masked = oracle.dense_mask(nk, causal, lts, lte, uts, ute, n_rows=nq)
    live = ~masked.all(axis=1)
    assert live.any() and not live.all()
    tq, tk, tv = (torch.tensor(x[0, 0], requires_grad=True) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq[live][None], tk[None], tv[None], attn_mask=torch.from_numpy(~masked[live])[None])[0]
    ref.backward(torch.from_numpy(do[0, 0][live]))
    np.testing.assert_allclose(o[0, 0][live], ref.detach().numpy(), atol=1e-12)
    np.testing.assert_array_equal(o[0, 0][~live], 0.0)
    assert np.isneginf(lse[0, 0][~live]).all()
    np.testing.assert_allclose(dq[0, 0][live], tq.grad.numpy()[live], atol=1e-11)
    np.testing.assert_array_equal(dq[0, 0][~live], 0.0)
    np.testing.assert_allclose(dk[0, 0], tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dvv[0, 0], tv.grad.numpy(), atol=1e-11)


@pytest.mark.parametrize("seed", range(10))
def test_rectangular_tile_classes_sound(seed):
    rng = np.random.default_rng(200 + seed)
    nq, nk = int(rng.integers(1, 150)), int(rng.integers(1, 150))
    sizes = [1, 2, 3, 5, 8, 16, 32]
    bq, bk = int(rng.choice(sizes)), int(rng.choice(sizes))
    c = rng.integers(-10, nq + 10, nk)
    w = rng.integers(0, nq + 20, nk)
    v4 = [(c - w // 2), (c + w // 2), (c - w // 3), (c + w // 3)]
    v4 = [x.astype(np.int32) for x in v4]
    for causal in (True, False):
        masked = oracle.dense_mask(nk, causal, *v4, n_rows=nq)
        tab = oracle.kblock_minmax(1, 1, nk, bk, *[x[None, None] for x in v4], n_rows=nq)
        cls = oracle.classify(tab, nk, bq, bk, causal, n_rows=nq)[0, 0]
        nqb, nkb = -(-nq // bq), -(-nk // bk)
        assert cls.shape == (nqb, nkb)
        for a in range(nqb):
            for b in range(nkb):
                t = masked[a * bq:(a + 1) * bq, b * bk:(b + 1) * bk]
                brute = 0 if t.all() else (2 if not t.any() else 1)
                assert cls[a, b] == 1 or cls[a, b] == brute


def test_missing_lte_means_every_local_row():
    """lte absent: LTE is the row count, also when Nq > Nk."""
    nq, nk = 9, 4
    lts = np.array([2, 0, 9, 5], np.int32)
    m = oracle.dense_mask(nk, False, lts, None, n_rows=nq)
    for j in range(nk):
        np.testing.assert_array_equal(m[:, j], np.arange(nq) >= lts[j])
    tab = oracle.kblock_minmax(1, 1, nk, 4, lts[None, None], None, n_rows=nq)
    assert tab[0, 0, 0, 2] == nq and tab[0, 0, 0, 3] == nq


@pytest.mark.parametrize("seed", range(6))
def test_open_pair_count_rectangular(seed):
    """The O(Nk) open-pair count with Nq rows equals the dense count."""
    from sparse_masked_attention_amd import flops
    rng = np.random.default_rng(300 + seed)
    nq, nk = int(rng.integers(1, 120)), int(rng.integers(1, 120))
    v = [rng.integers(-10, nq + 10, nk).astype(np.int32) for _ in range(4)]
    for causal in (True, False):
        for lte in (v[1], None):
            dense = oracle.dense_mask(nk, causal, v[0], lte, v[2], v[3], n_rows=nq)
            got = flops.nnz_columns(nk, causal, v[0], lte, v[2], v[3], n_rows=nq)
            np.testing.assert_array_equal(got, (~dense).sum(axis=0))
