"""Pins of the bf16 rounding replay (oracle/bf16_replay.py), which bounds the
error a bf16 evaluation of the method must make on a given input.

  * its rounding function equals torch's float32 -> bfloat16 conversion
    (round to nearest, ties to even), on random values and on exact ties;
  * with rounding switched off it is the oracle (forward and backward), so
    the rest of the replay is the same arithmetic as the pinned definition;
  * the forward's error is inside the bound rounding p to bf16 (relative
    error at most u = 2^-9) and O to bf16 allow: |dO_i| <= (2u / (1 - u))
    max |v| + u |O_i| per row;
  * rounding really happens: the replayed outputs are bf16 values and
    differ from the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import bf16_replay as R
from sparse_masked_attention_amd import inputs as I

U = 2.0 ** -9


def test_round_bf16_equals_torch_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000) * 10.0 ** rng.integers(-30, 30, 100_000),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-42])])
    x32 = x.astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(R.round_bf16(x32.astype(np.float64)), want)


def test_round_bf16_ties_go_to_even():
    # a float32 whose low 16 bits are exactly 0x8000 sits halfway between two
    # bf16 values; it rounds to the one with an even last kept bit
    hi = np.arange(0x3F80, 0x3F80 + 64, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32).astype(np.float64)
    got = R.round_bf16(ties).astype(np.float32).view(np.uint32) >> 16
    want = np.where(hi % 2 == 0, hi, hi + 1)
    np.testing.assert_array_equal(got, want)
    want_t = torch.from_numpy(ties.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(R.round_bf16(ties).astype(np.float32), want_t)


def _case(family, n=70, B=1, H=2, d=16, dv=8, seed=0):
    rng = np.random.default_rng(seed)
    vec = I.stack_masks([I.make_mask(family, n, rng) for _ in range(B)])
    q = I.randn((B, H, n, d), 10 + seed)
    k = I.randn((B, H, n, d), 20 + seed)
    v = I.randn((B, H, n, dv), 30 + seed)
    do = I.randn((B, H, n, dv), 40 + seed)
    return q, k, v, do, vec


@pytest.mark.parametrize("family", ["causal", "document", "prefix_lm_document", "all_open"])
def test_without_rounding_the_replay_is_the_oracle(family):
    q, k, v, do, vec = _case(family)
    lts, lte, uts, ute, causal = vec
    o, lse = R.forward(q, k, v, causal, lts, lte, uts, ute, rounding=False)
    ro, rl = oracle.forward(q, k, v, causal, lts, lte, uts, ute)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-6)   # the replay keeps LSE in float32
    got = R.backward(q, k, v, do, causal, lts, lte, uts, ute, rounding=False)
    ref = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, atol=2e-6)   # through the float32 LSE


def test_without_rounding_with_sink_and_empty_rows():
    n = 40
    lts = np.full(n, 10, np.int32)
    lte = np.full(n, 14, np.int32)            # rows 10..13 see nothing
    vec = (lts[None, None], lte[None, None], np.zeros((1, 1, n), np.int32),
           (np.arange(n) // 2).astype(np.int32)[None, None], False)
    q, k, v, do = (I.randn((1, 2, n, 8), 70 + t) for t in range(4))
    sink = np.array([0.7, -1.3], np.float32)
    o, lse = R.forward(q, k, v, *vec[4:], *vec[:4], sink=sink, rounding=False)
    ro, rl = oracle.forward(q, k, v, vec[4], *vec[:4], sink=sink)
    np.testing.assert_allclose(o, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-6)
    assert (o[:, :, 10:14] == 0).all()
    got = R.backward(q, k, v, do, vec[4], *vec[:4], sink=sink, rounding=False)
    ref = oracle.backward(q, k, v, do, vec[4], *vec[:4], sink=sink)
    for g, r in zip(got, ref[:3]):
        np.testing.assert_allclose(g, r, atol=2e-6)


@pytest.mark.parametrize("family", ["causal", "document", "sliding_window", "all_open"])
def test_forward_error_within_the_rounding_bound(family):
    q, k, v, do, vec = _case(family, n=90, d=32, dv=32, seed=3)
    lts, lte, uts, ute, causal = vec
    o, _ = R.forward(q, k, v, causal, lts, lte, uts, ute)
    ro, _ = oracle.forward(q, k, v, causal, lts, lte, uts, ute)
    for b in range(o.shape[0]):
        for h in range(o.shape[1]):
            vmax = np.abs(v[b, h]).max()
            bound = 2 * U / (1 - U) * vmax + U * np.abs(ro[b, h]).max(axis=1) + 1e-12
            err = np.abs(o[b, h] - ro[b, h]).max(axis=1)
            assert (err <= bound).all()


def test_rounding_happens():
    q, k, v, do, vec = _case("document", n=64, d=32, dv=32, seed=5)
    lts, lte, uts, ute, causal = vec
    o, _ = R.forward(q, k, v, causal, lts, lte, uts, ute)
    dq, dk, dv = R.backward(q, k, v, do, causal, lts, lte, uts, ute)
    ref = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute)
    for x in (o, dq, dk, dv):
        np.testing.assert_array_equal(R.round_bf16(x), x)     # bf16 values
    for x, r in zip((dq, dk, dv), ref):
        err = np.abs(x - r).max()
        assert 0 < err < 0.05
