"""Forward parity: the HIP path against the fp64 oracle on the same inputs."""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm
from gpu_util import (BF16_ATOL, FP32_ATOL, check_bf16, check_fp32, check_lse, mask_from,
                      qkvo, say, to_dev, to_np)
from _lib_fixture import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def run_fwd(q, k, v, vectors, dtype, scale=None, table=None, counts=None):
    m = mask_from(vectors)
    o, lse = fm.fwd(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), m, scale=scale,
                    table=table, tile_counts=counts)
    torch.cuda.synchronize()
    return o, lse


def oracle_fwd(q, k, v, vectors, scale=None, heads=None):
    lts, lte, uts, ute, causal = vectors
    return oracle.forward(q, k, v, causal, lts, lte, uts, ute, scale=scale, heads=heads)


def test_c1_tiny_fp32_document():
    """fp32, B=1 H=2 N=256 d=64, causal document mask of 3 documents."""
    c = I.CONFIGS[1]
    say("fwd C1 fp32")
    q, k, v = (I.randn((1, 2, 256, 64), I.qkv_seed(1, t), bf16=False) for t in range(3))
    vec = I.config_masks(1, "document3")
    o, lse = run_fwd(q, k, v, vec, torch.float32)
    ro, rl = oracle_fwd(q, k, v, vec)
    check_fp32("O", to_np(o), ro)
    check_lse(to_np(lse), rl, FP32_ATOL)


FAMILIES = ["document", "causal", "all_open", "share_question", "sliding_window",
            "prefix_lm_document", "block_sparse"]


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("N", [129, 1000])
def test_families_bf16_d128(family, N):
    B, H, d = 2, 2, 128
    say(f"fwd bf16 family={family} N={N} d={d}")
    q, k, v = qkvo(B, H, N, d, 500)
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(b)) for b in range(B)])
    o, lse = run_fwd(q, k, v, vec, torch.bfloat16)
    ro, rl = oracle_fwd(q, k, v, vec)
    check_bf16("O", to_np(o), ro)
    check_lse(to_np(lse), rl, BF16_ATOL)


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("family", ["document", "prefix_lm_document", "sliding_window"])
def test_head_dims_bf16(d, family):
    B, H, N = 1, 2, 777
    say(f"fwd bf16 family={family} N={N} d={d}")
    q, k, v = qkvo(B, H, N, d, 600)
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(3))])
    o, lse = run_fwd(q, k, v, vec, torch.bfloat16)
    ro, rl = oracle_fwd(q, k, v, vec)
    check_bf16("O", to_np(o), ro)
    check_lse(to_np(lse), rl, BF16_ATOL)


@pytest.mark.parametrize("family", ["document", "prefix_lm_document", "all_open"])
def test_fp32_d128(family):
    B, H, N, d = 1, 2, 300, 128
    say(f"fwd fp32 family={family} N={N} d={d}")
    q, k, v = qkvo(B, H, N, d, 700, bf16=False)
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(4))])
    o, lse = run_fwd(q, k, v, vec, torch.float32)
    ro, rl = oracle_fwd(q, k, v, vec)
    check_fp32("O", to_np(o), ro)
    check_lse(to_np(lse), rl, FP32_ATOL)


@pytest.mark.parametrize("N", [1, 2, 7, 64, 65, 127, 128, 130])
def test_small_and_ragged(N):
    say(f"fwd ragged N={N}")
    q, k, v = qkvo(1, 3, N, 128, 800)
    for fam in ["causal", "all_open"]:
        vec = I.stack_masks([I.make_mask(fam, N, np.random.default_rng(0))])
        o, lse = run_fwd(q, k, v, vec, torch.bfloat16)
        ro, rl = oracle_fwd(q, k, v, vec)
        check_bf16("O", to_np(o), ro)
        check_lse(to_np(lse), rl, BF16_ATOL)


def test_fully_masked_rows_and_out_of_range_values():
    """Rows hidden from every key output 0 with LSE -inf; any int32 is legal."""
    N, H = 500, 2
    say("fwd empty rows")
    rng = np.random.default_rng(5)
    lts = rng.integers(-1000, N + 1000, N).astype(np.int32)
    lte = (lts + rng.integers(0, 400, N)).astype(np.int32)
    lts[:] = np.minimum(lts, 200)
    lte[:] = np.maximum(lte, 260)                       # rows 200..259 hidden everywhere
    uts = rng.integers(-5, N + 5, N).astype(np.int32)
    ute = (uts + rng.integers(-20, 60, N)).astype(np.int32)
    ute[:5] = np.iinfo(np.int32).max
    uts[:5] = np.iinfo(np.int32).min
    vec = (lts[None, None], lte[None, None], uts[None, None], ute[None, None], False)
    q, k, v = qkvo(1, H, N, 128, 900)
    o, lse = run_fwd(q, k, v, vec, torch.bfloat16)
    ro, rl = oracle_fwd(q, k, v, vec)
    assert np.isneginf(rl[0, 0, 200:260]).all()
    check_bf16("O", to_np(o), ro)
    check_lse(to_np(lse), rl, BF16_ATOL)
    assert np.all(to_np(o)[0, :, 200:260] == 0)


def test_per_head_masks_and_null_vectors():
    N, H = 333, 3
    say("fwd per-head masks / NULL vectors")
    q, k, v = qkvo(1, H, N, 128, 1000)
    ms = [I.make_mask("document", N, np.random.default_rng(s)) for s in range(H)]
    lts = np.stack([m.lts for m in ms])[None]
    vec = (lts, None, None, None, True)                 # lte NULL -> N
    o, lse = run_fwd(q, k, v, vec, torch.bfloat16)
    ro, rl = oracle_fwd(q, k, v, vec)
    check_bf16("O per-head", to_np(o), ro)
    vec = (None, None, None, None, False)               # no mask at all
    o, _ = run_fwd(q, k, v, vec, torch.bfloat16)
    ro, _ = oracle_fwd(q, k, v, vec)
    check_bf16("O no-mask", to_np(o), ro)


def test_explicit_scale():
    N = 200
    q, k, v = qkvo(1, 2, N, 64, 1100)
    vec = I.stack_masks([I.make_mask("sliding_window", N, np.random.default_rng(0))])
    o, lse = run_fwd(q, k, v, vec, torch.bfloat16, scale=0.3)
    ro, rl = oracle_fwd(q, k, v, vec, scale=0.3)
    check_bf16("O", to_np(o), ro)
    check_lse(to_np(lse), rl, BF16_ATOL)


@pytest.mark.parametrize("family", ["document", "prefix_lm_document", "block_sparse"])
def test_tile_counts_match_oracle_classes(family):
    B, H, N, d = 2, 3, 1500, 128
    say(f"fwd tile counts family={family}")
    q, k, v = qkvo(B, H, N, d, 1200)
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(b + 7)) for b in range(B)])
    counts = torch.zeros(3, dtype=torch.int64, device="cuda")
    run_fwd(q, k, v, vec, torch.bfloat16, counts=counts)
    bq, bk = fm.tile_shape(False, d, torch.bfloat16)
    lts, lte, uts, ute, causal = vec
    t = oracle.kblock_minmax(B, 1, N, bk, lts, lte, uts, ute)
    ref = oracle.classify_counts(oracle.classify(t, N, bq, bk, causal)) * H
    assert counts.cpu().numpy().tolist() == ref.tolist()


def test_repeatable_and_precomputed_table_and_canary():
    B, H, N, d = 1, 4, 2000, 128
    say("fwd repeatability / table / canary")
    q, k, v = qkvo(B, H, N, d, 1300)
    vec = I.stack_masks([I.make_mask("share_question", N, np.random.default_rng(1))])
    m = mask_from(vec)
    qd, kd, vd = (to_dev(x, torch.bfloat16) for x in (q, k, v))
    o1, l1 = fm.fwd(qd, kd, vd, m)
    o2, l2 = fm.fwd(qd, kd, vd, m)
    table, _ = fm.tile_classify(m, B, N, 128, fm.table_block(), classes=False)
    o3, l3 = fm.fwd(qd, kd, vd, m, table=table)
    # canary: outputs inside larger buffers filled with a pattern
    big_o = torch.full((B * H * N * d + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    big_l = torch.full((B * H * N + 4096,), 7.0, dtype=torch.float32, device="cuda")
    o4, l4 = fm.fwd(qd, kd, vd, m, out=big_o[:B * H * N * d].view(B, H, N, d),
                    lse=big_l[:B * H * N].view(B, H, N))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    assert torch.equal(o1, o4) and torch.equal(l1, l4)
    assert torch.all(big_o[B * H * N * d:] == 7.0) and torch.all(big_l[B * H * N:] == 7.0)
