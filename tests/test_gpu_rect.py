"""Nq query rows against Nk keys on the GPU, and the row localisation of one
context-parallel rank's share (FlashMask-3 abstract: each rank localises the
column-wise mask without communication, then attends its rows to all keys).

Parity against the fp64 oracle (rectangular form, pinned in
test_oracle_rect.py). The oracle's mask of a rank's share is always built
from the global vectors by the oracle's own localisation (oracle.localize,
pinned by brute force against the rows of the global dense mask); the GPU
side localises with flashmask_localize, whose output is also compared bit
for bit with oracle.localize.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm
from gpu_util import (BF16_ATOL, FP32_ATOL, Replay, replays, check_bf16, check_fp32, check_lse, mask_from,
                      say, to_dev, to_np)
from _lib_fixture import ensure_built

pytestmark = pytest.mark.gpu

FAMILIES = ["causal", "document", "share_question", "sliding_window", "block_sparse",
            "prefix_lm_document", "all_open"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


zigzag = I.zigzag_chunks


def gpu_localize(vec, n, chunks):
    """flashmask_localize on the GPU; its four outputs are checked bit for bit
    against the oracle's localisation of the same global vectors."""
    m = mask_from(vec)
    B = np.asarray(vec[0]).shape[0]          # every family here carries lts
    lm = fm.localize(m, B, n, n, chunks)
    torch.cuda.synchronize()
    ref = oracle.localize(*vec[:4], vec[4], chunks, n)
    for got, want in zip((lm.lts, lm.lte, lm.uts, lm.ute), ref[:4]):
        np.testing.assert_array_equal(got.cpu().numpy(), want)
    return lm


def oracle_local(vec, n, chunks):
    """The oracle's local vectors of the share, from the global ones."""
    return list(oracle.localize(*vec[:4], vec[4], chunks, n)[:4])


def run_rect(q, k, v, do, lm, dtype=torch.bfloat16, fcounts=None):
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    o, lse = fm.fwd(qd, kd, vd, lm, tile_counts=fcounts)
    dq, dk, dv = fm.bwd(qd, kd, vd, o, lse, dod, lm)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def compare_rect(q, k, v, do, l4, got, fp32=False, heads=None):
    """Oracle parity of a rank's share (bf16: the bf16 rounding replay of the
    same problem bounds max-abs where the method's rounding alone passes
    2e-2; see gpu_util.check_bf16)."""
    ro, rl = oracle.forward(q, k, v, False, *l4, heads=heads)
    rq, rk, rv = oracle.backward(q, k, v, do, False, *l4, heads=heads)
    sel = (lambda x: x) if heads is None else (lambda x: np.stack([x[b, h] for b, h in heads]))
    o, lse, dq, dk, dv = (to_np(x) for x in got)
    check_lse(sel(lse), sel(rl), FP32_ATOL if fp32 else BF16_ATOL)
    if fp32:
        for name, g, r in (("O", o, ro), ("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            check_fp32(name, sel(g), sel(r))
        return
    rf, rb = replays(q, k, v, do, (*l4, False), heads=heads)
    check_bf16("O", sel(o), sel(ro), replay=rf[0])
    check_bf16("dQ", sel(dq), sel(rq), replay=rb[0])
    check_bf16("dK", sel(dk), sel(rk), replay=rb[1])
    check_bf16("dV", sel(dv), sel(rv), replay=rb[2])


@pytest.mark.parametrize("family", FAMILIES)
def test_gpu_localize_equals_oracle(family):
    n, B = 1000, 2
    say(f"localize family={family}")
    vec = I.stack_masks([I.make_mask(family, n, np.random.default_rng(20 + b)) for b in range(B)])
    for chunks in ([(0, n)], [(0, 250)], [(250, 500), (750, 1000)], zigzag(n, 4, 1),
                   [(3, 17), (100, 101), (640, 999)]):
        gpu_localize(vec, n, chunks)     # compares with oracle.localize


def test_gpu_localize_arbitrary_int32():
    rng = np.random.default_rng(5)
    n = 777
    v = [rng.integers(-2**31, 2**31 - 1, n, dtype=np.int64).astype(np.int32)[None, None] for _ in range(4)]
    v[0][0, 0, :100] = rng.integers(-50, n + 50, 100)
    for causal in (True, False):
        vec = (v[0], v[1], v[2], v[3], causal)
        for chunks in ([(0, 300)], zigzag(n, 3, 2)):
            gpu_localize(vec, n, chunks)     # compares with oracle.localize


@pytest.mark.parametrize("mask_seed", [11, 31])
@pytest.mark.parametrize("family", FAMILIES)
def test_rank_shares_bf16(family, mask_seed):
    """Each of 4 zig-zag ranks: local vectors on the GPU, its rows against all
    keys, forward and backward against the oracle's rectangular problem built
    from the global vectors.

    Mask seed 31: the document mask has rows whose dS terms nearly cancel, and
    rounding dS to bf16 (the matrix operand) alone puts one dK element of
    rank 1 2.154e-2 from the fp64 value (rel-L2 3.0e-3; oracle.bf16_replay
    gives that figure), so there the max-abs is held to the replay's
    (gpu_util.check_bf16)."""
    B, H, n, d = 1, 2, 1000, 128
    say(f"rank shares family={family} mask_seed={mask_seed}")
    rng = np.random.default_rng(mask_seed)
    vec = I.stack_masks([I.make_mask(family, n, rng)])
    q, k, v, do = (I.randn((B, H, n, d), 3000 + t) for t in range(4))
    for r in range(4):
        chunks = zigzag(n, 4, r)
        rows = oracle.rank_rows(chunks, n)
        lm = gpu_localize(vec, n, chunks)
        l4 = oracle_local(vec, n, chunks)
        got = run_rect(q[:, :, rows], k, v, do[:, :, rows], lm)
        compare_rect(q[:, :, rows], k, v, do[:, :, rows], l4, got)


@pytest.mark.parametrize("nq,nk", [(300, 700), (700, 300), (129, 1000), (1000, 257), (1000, 65)])
@pytest.mark.parametrize("causal", [True, False])
def test_rectangular_random_bounds(nq, nk, causal):
    """Arbitrary bounds on Nq rows for Nk keys; causal is j > i in local rows.
    Few keys for many rows make |dV| large: at 1000 x 65 it reaches 7.9, and
    rounding it to bf16 alone takes most of the 2e-2 absolute bound (the
    bf16 rounding replay bounds max-abs there; gpu_util.check_bf16)."""
    B, H, d = 1, 2, 64
    say(f"rect nq={nq} nk={nk} causal={causal}")
    rng = np.random.default_rng(nq + 7 * nk)
    c = rng.integers(-20, nq + 20, nk)
    w = rng.integers(0, nq // 2 + 2, nk)
    l4 = [(c - w).astype(np.int32)[None, None], (c + w // 2).astype(np.int32)[None, None],
          np.zeros((1, 1, nk), np.int32), rng.integers(0, nq // 4 + 1, nk).astype(np.int32)[None, None]]
    vec = (l4[0], l4[1], l4[2], l4[3], causal)
    q, do = I.randn((B, H, nq, d), 3100), I.randn((B, H, nq, d), 3101)
    k, v = I.randn((B, H, nk, d), 3102), I.randn((B, H, nk, d), 3103)
    m = mask_from(vec)
    got = run_rect(q, k, v, do, m)
    ro, rl = oracle.forward(q, k, v, causal, *l4)
    rq, rk, rv = oracle.backward(q, k, v, do, causal, *l4)
    o, lse, dq, dk, dv = (to_np(x) for x in got)
    rf = Replay(lambda: oracle.bf16_replay.forward(q, k, v, causal, *l4))
    rb = Replay(lambda: oracle.bf16_replay.backward(q, k, v, do, causal, *l4))
    check_bf16("O", o, ro, replay=rf[0])
    check_lse(lse, rl, BF16_ATOL)
    check_bf16("dQ", dq, rq, replay=rb[0])
    check_bf16("dK", dk, rk, replay=rb[1])
    check_bf16("dV", dv, rv, replay=rb[2])


def test_rectangular_fp32_and_tile_counts():
    B, H, n, d = 1, 2, 600, 64
    say("rect fp32 and tile counts")
    vec = I.stack_masks([I.make_mask("document", n, np.random.default_rng(2))])
    chunks = zigzag(n, 3, 0)
    rows = oracle.rank_rows(chunks, n)
    lm = gpu_localize(vec, n, chunks)
    l4 = oracle_local(vec, n, chunks)
    q, k, v, do = (I.randn((B, H, n, d), 3200 + t, bf16=False) for t in range(4))
    got = run_rect(q[:, :, rows], k, v, do[:, :, rows], lm, dtype=torch.float32)
    compare_rect(q[:, :, rows], k, v, do[:, :, rows], l4, got, fp32=True)
    counts = torch.zeros(3, dtype=torch.int64, device="cuda")
    run_rect(q[:, :, rows], k, v, do[:, :, rows], lm, fcounts=counts)
    bq, bk = fm.tile_shape(False, d, torch.bfloat16)
    t = oracle.kblock_minmax(B, 1, n, bk, *l4, n_rows=len(rows))
    ref = oracle.classify_counts(oracle.classify(t, n, bq, bk, False, n_rows=len(rows))) * H
    assert counts.cpu().numpy().tolist() == ref.tolist()


def test_empty_sides():
    B, H, d = 1, 2, 128
    say("rect empty sides")
    q = to_dev(I.randn((B, H, 100, d), 3300), torch.bfloat16)
    k0 = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    m0 = fm.Mask(None, None, None, None, True)
    o, lse = fm.fwd(q, k0, k0, m0)
    dq, dk, dv = fm.bwd(q, k0, k0, o, lse, q, m0)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse)) and torch.all(dq == 0)
    k = to_dev(I.randn((B, H, 50, d), 3301), torch.bfloat16)
    q0 = torch.empty((B, H, 0, d), dtype=torch.bfloat16, device="cuda")
    lse0 = torch.empty((B, H, 0), dtype=torch.float32, device="cuda")
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(k, 7.0)
    fm.bwd(q0, k, k, q0, lse0, q0, m0, grads=(torch.empty_like(q0), dk, dv))
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


@pytest.mark.parametrize("family", ["document", "causal"])
def test_full_size_rank_share(family):
    """B=1 H=32 N=8192: rank 1 of 4 (zig-zag), all outputs, oracle on sampled heads."""
    B, H, n, d = 1, 32, 8192, 128
    say(f"full-size rank share family={family}")
    vec = I.config_masks(5, family, n=n, batch=B)
    chunks = zigzag(n, 4, 1)
    rows = oracle.rank_rows(chunks, n)
    lm = gpu_localize(vec, n, chunks)
    l4 = oracle_local(vec, n, chunks)
    q, k, v, do = (I.randn((B, H, n, d), I.qkv_seed(5, t)) for t in range(4))
    got = run_rect(q[:, :, rows], k, v, do[:, :, rows], lm)
    for t in got:
        assert bool(torch.isfinite(t).all()), "non-finite output"
    compare_rect(q[:, :, rows], k, v, do[:, :, rows], l4, got, heads=[(0, 0), (0, 13), (0, 31)])
