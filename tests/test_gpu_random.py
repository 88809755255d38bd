"""Randomised parity sweep on the GPU: seeded random combinations of dtype,
head dims (d, dv), batch, heads, shared or per-head masks, Nq != Nk, mask
structure, causal flag and sink bias, each checked end to end (forward and
backward) against the fp64 oracle at the parity tolerances.

Sizes stay small (the oracle takes well under a second per case) but span
several tiles and ragged tails on both sides. The key count is kept at least
half the row count: with very few keys for many rows |dV| grows until bf16
rounding of dV alone approaches the absolute bound (see test_gpu_rect.py).

For seeds 13 and 17 the bf16 method itself (oracle.bf16_replay: P rounded
to bf16 as the operand of dV = P^T dO, dS rounded to bf16, outputs rounded;
everything else exact) already gives dV max-abs 2.107e-2 and 2.064e-2
against the oracle (rel-L2 2-3e-3), above the fixed 2e-2: there the
max-abs is held to 1.05 x the replay's (gpu_util.check_bf16); seed 18's
replay reaches 1.828e-2 and every other seed's at most 1.54e-2.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm
from gpu_util import (BF16_ATOL, FP32_ATOL, Replay, check_bf16, check_fp32, check_lse, say, to_dev,
                      to_np)
from _lib_fixture import ensure_built

pytestmark = pytest.mark.gpu

FAMILIES = ["causal", "document", "share_question", "sliding_window", "block_sparse",
            "prefix_lm_document", "all_open"]
BF16_DIMS = [(64, 64), (128, 128), (256, 256), (192, 128)]
FP32_DIMS = [(64, 64), (128, 128)]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def random_bounds(rng, nq, nk, hm, B):
    """Arbitrary int32 interval bounds (some outside [0, Nq]) on nq rows for
    nk keys: a lower interval around a random centre and a short upper one."""
    c = rng.integers(-20, nq + 20, (B, hm, nk))
    w = rng.integers(0, nq // 2 + 2, (B, hm, nk))
    lts = (c - w).astype(np.int32)
    lte = (c + w // 2).astype(np.int32)
    uts = np.zeros((B, hm, nk), np.int32)
    ute = rng.integers(0, nq // 4 + 1, (B, hm, nk)).astype(np.int32)
    return lts, lte, uts, ute


def family_bounds(rng, n, hm, B, family):
    """The named family's vectors for every (b, mask head), [B, hm, n]."""
    ms = [[I.make_mask(family, n, rng) for _ in range(hm)] for _ in range(B)]
    causal = ms[0][0].causal
    lts = np.array([[m.lts for m in row] for row in ms], np.int32)
    lte = np.array([[m.lte for m in row] for row in ms], np.int32)
    if causal:
        return lts, lte, None, None, True
    uts = np.array([[m.uts for m in row] for row in ms], np.int32)
    ute = np.array([[m.ute for m in row] for row in ms], np.int32)
    return lts, lte, uts, ute, False


def draw_case(seed):
    rng = np.random.default_rng(50_000 + seed)
    fp32 = rng.random() < 0.2
    d, dv = (FP32_DIMS if fp32 else BF16_DIMS)[rng.integers(0, 2 if fp32 else 4)]
    B = int(rng.integers(1, 3))
    H = int(rng.integers(1, 5))
    hm = H if rng.random() < 0.3 else 1
    nk = int(rng.integers(1, 640))
    if rng.random() < 0.4:
        nq = int(rng.integers(1, 2 * nk + 2))        # rectangular: random bounds
        causal = bool(rng.random() < 0.5)
        lts, lte, uts, ute = random_bounds(rng, nq, nk, hm, B)
        vec = (lts, lte, None, None, True) if causal else (lts, lte, uts, ute, False)
        family = "random"
    else:
        nq = nk
        family = FAMILIES[rng.integers(0, len(FAMILIES))]
        vec = family_bounds(rng, nk, hm, B, family)
    sink = rng.normal(0.0, 2.0, H).astype(np.float32) if rng.random() < 0.3 else None
    return dict(rng=rng, fp32=fp32, d=d, dv=dv, B=B, H=H, hm=hm, nq=nq, nk=nk, family=family,
                vec=vec, sink=sink)


SEEDS = list(range(27))


@pytest.mark.parametrize("seed", SEEDS)
def test_random_case(seed):
    c = draw_case(seed)
    B, H, nq, nk, d, dv = c["B"], c["H"], c["nq"], c["nk"], c["d"], c["dv"]
    lts, lte, uts, ute, causal = c["vec"]
    dtype = torch.float32 if c["fp32"] else torch.bfloat16
    say(f"random seed={seed} {'fp32' if c['fp32'] else 'bf16'} d={d} dv={dv} B={B} H={H} "
        f"hm={c['hm']} nq={nq} nk={nk} family={c['family']} causal={causal} "
        f"sink={'yes' if c['sink'] is not None else 'no'}")
    bf = not c["fp32"]
    q = I.randn((B, H, nq, d), 60_000 + 4 * seed, bf16=bf)
    k = I.randn((B, H, nk, d), 60_001 + 4 * seed, bf16=bf)
    v = I.randn((B, H, nk, dv), 60_002 + 4 * seed, bf16=bf)
    do = I.randn((B, H, nq, dv), 60_003 + 4 * seed, bf16=bf)
    m = fm.Mask.from_numpy(lts, lte, uts, ute, causal)
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    sink_t = None if c["sink"] is None else torch.from_numpy(c["sink"]).cuda()
    o, lse = fm.fwd(qd, kd, vd, m, sink=sink_t)
    grads = fm.bwd(qd, kd, vd, o, lse, dod, m, sink=sink_t)
    torch.cuda.synchronize()

    ro, rl = oracle.forward(q, k, v, causal, lts, lte, uts, ute, sink=c["sink"])
    ref = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute, sink=c["sink"])
    check_lse(to_np(lse), rl, FP32_ATOL if c["fp32"] else BF16_ATOL)
    if c["fp32"]:
        check_fp32("O", to_np(o), ro)
        for name, got, want in zip(["dQ", "dK", "dV"], grads[:3], ref[:3]):
            check_fp32(name, to_np(got), want)
    else:
        rf = Replay(lambda: oracle.bf16_replay.forward(q, k, v, causal, lts, lte, uts, ute, sink=c["sink"]))
        rb = Replay(lambda: oracle.bf16_replay.backward(q, k, v, do, causal, lts, lte, uts, ute,
                                                        sink=c["sink"]))
        check_bf16("O", to_np(o), ro, replay=rf[0])
        for i, (name, got, want) in enumerate(zip(["dQ", "dK", "dV"], grads[:3], ref[:3])):
            check_bf16(name, to_np(got), want, replay=rb[i])
    if c["sink"] is not None:
        ds, rs = to_np(grads[3]), ref[3]
        err = np.abs(ds - rs)
        say(f"  dsink: max_abs={err.max():.3e}")
        tol = (1e-4 if c["fp32"] else 2e-2) + (1e-5 if c["fp32"] else 5e-3) * np.abs(rs)
        assert (err <= tol).all(), (ds, rs)
