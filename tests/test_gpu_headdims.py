"""Parity for a Q/K head dim larger than V's: d = 192 with dv = 128 (bf16).

The README ("News") lists large head dims among FlashMask's features and
("Key Features") tabulates (d, dv) pairs with d the Q/K head dim and dv the V
head dim; the scale stays 1/sqrt(d) (README "Formulation"). Forward and
backward against the fp64 oracle, which takes dv from V's shape.
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

D, DV = 192, 128


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def inputs_qkvd(B, H, N, seed):
    q = I.randn((B, H, N, D), seed)
    k = I.randn((B, H, N, D), seed + 1)
    v = I.randn((B, H, N, DV), seed + 2)
    do = I.randn((B, H, N, DV), seed + 3)
    return q, k, v, do


def run(q, k, v, do, vec, fcounts=None, bcounts=None):
    m = mask_from(vec)
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    o, lse = fm.fwd(qd, kd, vd, m, tile_counts=fcounts)
    dq, dk, dv = fm.bwd(qd, kd, vd, o, lse, dod, m, tile_counts=bcounts)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def compare(q, k, v, do, vec, got, heads=None):
    lts, lte, uts, ute, causal = vec
    ro, rl = oracle.forward(q, k, v, causal, lts, lte, uts, ute, heads=heads)
    rq, rk, rv = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute, heads=heads)
    sel = (lambda x: x) if heads is None else (lambda x: np.stack([x[b, h] for b, h in heads]))
    o, lse, dq, dk, dv = (to_np(x) for x in got)
    assert o.shape[-1] == DV and dq.shape[-1] == D and dk.shape[-1] == D and dv.shape[-1] == DV
    rf, rb = replays(q, k, v, do, vec, heads=heads)
    check_bf16("O", sel(o), sel(ro), replay=rf[0])
    check_lse(sel(lse), sel(rl), BF16_ATOL)
    check_bf16("dQ", sel(dq), sel(rq), replay=rb[0])
    check_bf16("dK", sel(dk), sel(rk), replay=rb[1])
    check_bf16("dV", sel(dv), sel(rv), replay=rb[2])


FAMILIES = ["causal", "document", "share_question", "sliding_window", "block_sparse",
            "prefix_lm_document", "all_open"]


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("N", [129, 1000])
def test_families_d192_dv128(family, N):
    B, H = 1, 2
    say(f"d192/dv128 family={family} N={N}")
    q, k, v, do = inputs_qkvd(B, H, N, 7000)
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(13))])
    compare(q, k, v, do, vec, run(q, k, v, do, vec))


@pytest.mark.parametrize("N", [1, 7, 64, 130])
def test_small_and_ragged(N):
    say(f"d192/dv128 ragged N={N}")
    q, k, v, do = inputs_qkvd(1, 1, N, 7100)
    vec = I.stack_masks([I.make_mask("document", N, np.random.default_rng(5))])
    compare(q, k, v, do, vec, run(q, k, v, do, vec))


def test_tile_counts_and_determinism():
    """Tile counters follow the d = 192 tile shapes; gradients repeat bitwise."""
    B, H, N = 2, 2, 700
    say("d192/dv128 tile counts and determinism")
    q, k, v, do = inputs_qkvd(B, H, N, 7200)
    vec = I.stack_masks([I.make_mask("prefix_lm_document", N, np.random.default_rng(b)) for b in range(B)])
    fc = torch.zeros(3, dtype=torch.int64, device="cuda")
    bc = torch.zeros(3, dtype=torch.int64, device="cuda")
    got1 = run(q, k, v, do, vec, fcounts=fc, bcounts=bc)
    got2 = run(q, k, v, do, vec)
    lts, lte, uts, ute, causal = vec
    for is_bwd, counts in ((False, fc), (True, bc)):
        bq, bk = fm.tile_shape(is_bwd, D, torch.bfloat16)
        t = oracle.kblock_minmax(B, 1, N, bk, lts, lte, uts, ute)
        ref = oracle.classify_counts(oracle.classify(t, N, bq, bk, causal)) * H
        assert counts.cpu().numpy().tolist() == ref.tolist(), (is_bwd, bq, bk)
    for a, b in zip(got1, got2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("family", ["document", "causal"])
def test_full_size_sampled_heads(family):
    """B=1 H=4 N=8192: every output, oracle on two sampled heads."""
    B, H, N = 1, 4, 8192
    say(f"d192/dv128 full size family={family}")
    q, k, v, do = inputs_qkvd(B, H, N, 7300)
    vec = I.config_masks(5, family, n=N, batch=B)
    got = run(q, k, v, do, vec)
    compare(q, k, v, do, vec, got, heads=[(0, 0), (0, 3)])
