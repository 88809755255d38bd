"""Backward parity: dQ, dK, dV from the HIP path against the fp64 oracle.

As a user would, the backward is fed the GPU forward's O and logsumexp; the
oracle recomputes its own probabilities from Q, K, V.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm
from gpu_util import check_bf16, check_fp32, mask_from, qkvo, replays, say, to_dev, to_np
from _lib_fixture import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def run_case(q, k, v, do, vec, dtype=torch.bfloat16, counts=None):
    m = mask_from(vec)
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    o, lse = fm.fwd(qd, kd, vd, m)
    dq, dk, dv = fm.bwd(qd, kd, vd, o, lse, dod, m, tile_counts=counts)
    torch.cuda.synchronize()
    return dq, dk, dv


def compare(q, k, v, do, vec, dq, dk, dv, heads=None, fp32=False):
    lts, lte, uts, ute, causal = vec
    rq, rk, rv = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute, heads=heads)
    sel = (lambda x: x) if heads is None else (lambda x: np.stack([x[b, h] for b, h in heads]))
    if fp32:
        for name, g, r in (("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            check_fp32(name, sel(to_np(g)), sel(r))
        return
    _, rb = replays(q, k, v, do, vec, heads=heads)
    for i, (name, g, r) in enumerate((("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv))):
        check_bf16(name, sel(to_np(g)), sel(r), replay=rb[i])


FAMILIES = ["causal", "document", "share_question", "sliding_window", "block_sparse",
            "prefix_lm_document", "all_open"]


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("N", [129, 1000])
@pytest.mark.parametrize("d", [64, 128])
def test_families(family, N, d):
    B, H = 1, 2
    say(f"bwd family={family} N={N} d={d}")
    q, k, v, do = qkvo(B, H, N, d, 2000, with_do=True)
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(11))])
    dq, dk, dv = run_case(q, k, v, do, vec)
    compare(q, k, v, do, vec, dq, dk, dv)


@pytest.mark.parametrize("family", ["document", "prefix_lm_document", "sliding_window", "causal"])
def test_head_dim_256(family):
    B, H, N, d = 1, 2, 555, 256
    say(f"bwd family={family} N={N} d={d}")
    q, k, v, do = qkvo(B, H, N, d, 2400, with_do=True)
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(12))])
    dq, dk, dv = run_case(q, k, v, do, vec)
    compare(q, k, v, do, vec, dq, dk, dv)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("family", ["document", "prefix_lm_document", "all_open"])
def test_fp32(family, d):
    B, H, N = 1, 2, 300
    say(f"bwd fp32 family={family} N={N} d={d}")
    q, k, v, do = qkvo(B, H, N, d, 2500, bf16=False, with_do=True)
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(13))])
    dq, dk, dv = run_case(q, k, v, do, vec, dtype=torch.float32)
    compare(q, k, v, do, vec, dq, dk, dv, fp32=True)


@pytest.mark.parametrize("N", [1, 7, 64, 130])
def test_small_and_ragged(N):
    say(f"bwd ragged N={N}")
    q, k, v, do = qkvo(1, 2, N, 128, 2100, with_do=True)
    for fam in ["causal", "all_open"]:
        vec = I.stack_masks([I.make_mask(fam, N, np.random.default_rng(0))])
        dq, dk, dv = run_case(q, k, v, do, vec)
        compare(q, k, v, do, vec, dq, dk, dv)


def test_tile_counts_d256_and_fp32():
    B, H, N = 1, 2, 700
    vec = I.stack_masks([I.make_mask("document", N, np.random.default_rng(3))])
    lts, lte, uts, ute, causal = vec
    for d, dtype, bf in ((256, torch.bfloat16, True), (128, torch.float32, False)):
        say(f"bwd tile counts d={d} {dtype}")
        q, k, v, do = qkvo(B, H, N, d, 2600, bf16=bf, with_do=True)
        counts = torch.zeros(3, dtype=torch.int64, device="cuda")
        run_case(q, k, v, do, vec, dtype=dtype, counts=counts)
        bq, bk = fm.tile_shape(True, d, dtype)
        t = oracle.kblock_minmax(B, 1, N, bk, lts, lte, uts, ute)
        ref = oracle.classify_counts(oracle.classify(t, N, bq, bk, causal)) * H
        assert counts.cpu().numpy().tolist() == ref.tolist()


def test_bf16_backward_is_deterministic():
    B, H, N, d = 1, 4, 1500, 128
    say("bwd determinism")
    q, k, v, do = qkvo(B, H, N, d, 2700, with_do=True)
    vec = I.stack_masks([I.make_mask("share_question", N, np.random.default_rng(2))])
    a = run_case(q, k, v, do, vec)
    b = run_case(q, k, v, do, vec)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_fp32_backward_is_deterministic():
    """The fp32 dQ comes from its own query-major pass (no atomics), so all
    three gradients repeat bitwise."""
    B, H, N, d = 1, 2, 700, 64
    say("bwd fp32 determinism")
    q, k, v, do = qkvo(B, H, N, d, 2750, bf16=False, with_do=True)
    vec = I.stack_masks([I.make_mask("document", N, np.random.default_rng(5))])
    a = run_case(q, k, v, do, vec, dtype=torch.float32)
    b = run_case(q, k, v, do, vec, dtype=torch.float32)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_fully_masked_rows():
    N = 400
    say("bwd empty rows")
    lts = np.full(N, 100, np.int32)
    lte = np.full(N, 150, np.int32)                    # rows 100..149 hidden everywhere
    uts = np.zeros(N, np.int32)
    ute = (np.arange(N) // 3).astype(np.int32)
    vec = (lts[None, None], lte[None, None], uts[None, None], ute[None, None], False)
    q, k, v, do = qkvo(1, 2, N, 128, 2200, with_do=True)
    dq, dk, dv = run_case(q, k, v, do, vec)
    compare(q, k, v, do, vec, dq, dk, dv)
    assert np.all(to_np(dq)[0, :, 100:150] == 0)


def test_tile_counts_match_oracle_classes():
    B, H, N, d = 2, 2, 1100, 128
    say("bwd tile counts")
    q, k, v, do = qkvo(B, H, N, d, 2300, with_do=True)
    vec = I.stack_masks([I.make_mask("document", N, np.random.default_rng(b)) for b in range(B)])
    counts = torch.zeros(3, dtype=torch.int64, device="cuda")
    run_case(q, k, v, do, vec, counts=counts)
    bq, bk = fm.tile_shape(True, d, torch.bfloat16)
    lts, lte, uts, ute, causal = vec
    t = oracle.kblock_minmax(B, 1, N, bk, lts, lte, uts, ute)
    ref = oracle.classify_counts(oracle.classify(t, N, bq, bk, causal)) * H
    assert counts.cpu().numpy().tolist() == ref.tolist()


def test_long_sequence_list_in_rounds():
    """Nq = 65600 rows (1025 query blocks of 64): the 128 global keys see every
    row, so their key block's visible-tile list exceeds the 1024-entry list and
    the dK/dV pass walks it in two rounds (the only backward case that does).
    Every other key is open to a 512-row band from its own row (wide enough
    that the global keys' share of each row, and so their |dV| summed over
    65600 rows, stays well inside the bf16 bound). Checked on
    sampled rows and keys of one head, against the oracle's sampled backward
    (all rows evaluated: every row adds to the global keys' dK and dV)."""
    B, H, N, d = 1, 8, 65600, 128
    say(f"bwd long list-in-rounds B={B} H={H} N={N} d={d}")
    j = np.arange(N)
    glob = j < 128
    lts = np.where(glob, N, j + 512).astype(np.int32)[None, None]  # masked below the band
    lte = np.full((1, 1, N), N, np.int32)
    uts = np.zeros((1, 1, N), np.int32)
    ute = np.where(glob, 0, j).astype(np.int32)[None, None]        # masked above it
    vec = (lts, lte, uts, ute, False)
    q, k, v, do = (I.randn((B, H, N, d), 70_000 + t) for t in range(4))
    dq, dk, dv = run_case(q, k, v, do, vec)
    h = 5
    rows = [0, 1, 127, 128, 20_000, 65_599]
    keys = [0, 1, 63, 64, 127, 128, 1000, 40_000, 65_599]
    rq, rk, rv = oracle.backward_sampled(q[0, h], k[0, h], v[0, h], do[0, h], False,
                                         lts[0, 0], lte[0, 0], uts[0, 0], ute[0, 0],
                                         rows=rows, keys=keys)
    check_bf16("dQ", to_np(dq)[0, h, rows], rq)
    check_bf16("dK", to_np(dk)[0, h, keys], rk)
    check_bf16("dV", to_np(dv)[0, h, keys], rv)
