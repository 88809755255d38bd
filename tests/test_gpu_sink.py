"""Sink bias on the GPU against the fp64 oracle (the reading of the README's
"sink bias" is pinned in test_oracle_sink.py): one more always-open softmax
entry per head with logit s_h and a zero value vector."""
import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm
from gpu_util import (BF16_ATOL, FP32_ATOL, check_bf16, check_fp32, check_lse, mask_from, replays, say,
                      to_dev, to_np)
from _lib_fixture import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def run(q, k, v, do, m, sink, dtype=torch.bfloat16):
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    s = torch.from_numpy(np.asarray(sink, np.float32)).cuda()
    o, lse = fm.fwd(qd, kd, vd, m, sink=s)
    dq, dk, dv, ds = fm.bwd(qd, kd, vd, o, lse, dod, m, sink=s)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv, ds


def compare(q, k, v, do, vec, sink, got, fp32=False):
    lts, lte, uts, ute, causal = vec
    ro, rl = oracle.forward(q, k, v, causal, lts, lte, uts, ute, sink=sink)
    rq, rk, rv, rs = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute, sink=sink)
    o, lse, dq, dk, dv, ds = (to_np(x) for x in got)
    check_lse(lse, rl, FP32_ATOL if fp32 else BF16_ATOL)
    if fp32:
        for name, g, r in (("O", o, ro), ("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv)):
            check_fp32(name, g, r)
    else:
        rf, rb = replays(q, k, v, do, vec, sink=np.asarray(sink, np.float32))
        check_bf16("O", o, ro, replay=rf[0])
        for i, (name, g, r) in enumerate((("dQ", dq, rq), ("dK", dk, rk), ("dV", dv, rv))):
            check_bf16(name, g, r, replay=rb[i])
    err = np.abs(ds - rs)
    say(f"  dsink: max_abs={err.max():.3e} ref={np.round(rs, 3)}")
    tol = (1e-4 if fp32 else 2e-2) + (1e-5 if fp32 else 5e-3) * np.abs(rs)
    assert (err <= tol).all(), (ds, rs)


FAMILIES = ["causal", "document", "share_question", "sliding_window", "block_sparse",
            "prefix_lm_document", "all_open"]


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("N", [129, 1000])
def test_sink_families_bf16(family, N):
    B, H, d = 1, 2, 128
    say(f"sink family={family} N={N}")
    q, k, v, do = (I.randn((B, H, N, d), 4000 + t) for t in range(4))
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(17))])
    sink = np.array([0.5, -1.5])
    compare(q, k, v, do, vec, sink, run(q, k, v, do, mask_from(vec), sink))


def test_sink_fp32_and_empty_rows():
    """fp32; rows 40..47 see no key: O = 0 and LSE = s there."""
    B, H, N, d = 1, 2, 300, 64
    say("sink fp32 and empty rows")
    q, k, v, do = (I.randn((B, H, N, d), 4100 + t, bf16=False) for t in range(4))
    lts, lte, uts, ute, causal = I.stack_masks([I.make_mask("document", N, np.random.default_rng(3))])
    lts = np.minimum(lts, 40).astype(np.int32)
    lte = np.maximum(lte, 48).astype(np.int32)
    vec = (lts, lte, uts, ute, causal)
    sink = np.array([1.25, -0.75])
    got = run(q, k, v, do, mask_from(vec), sink, dtype=torch.float32)
    compare(q, k, v, do, vec, sink, got, fp32=True)
    o, lse = to_np(got[0]), to_np(got[1])
    assert (o[:, :, 40:48] == 0).all()
    np.testing.assert_allclose(lse[0, :, 40:48], np.repeat(sink[:, None], 8, 1), atol=1e-6)


def test_large_sink_does_not_overflow():
    B, H, N, d = 1, 2, 256, 128
    say("sink large logit")
    q, k, v, do = (I.randn((B, H, N, d), 4200 + t) for t in range(4))
    vec = I.stack_masks([I.make_mask("causal", N, np.random.default_rng(1))])
    sink = np.array([60.0, -60.0])          # exp(60) overflows bf16/fp16 ranges if taken raw
    got = run(q, k, v, do, mask_from(vec), sink)
    assert all(torch.isfinite(t).all() for t in got)
    compare(q, k, v, do, vec, sink, got)


def test_sink_on_a_rank_share_and_deterministic():
    B, H, n, d = 1, 2, 1000, 128
    say("sink rank share")
    vec = I.stack_masks([I.make_mask("document", n, np.random.default_rng(11))])
    e = np.linspace(0, n, 9).astype(int)
    chunks = [(int(e[2]), int(e[3])), (int(e[5]), int(e[6]))]
    rows = oracle.rank_rows(chunks, n)
    l4 = oracle.localize(*vec[:4], vec[4], chunks, n)      # the oracle's side
    q, k, v, do = (I.randn((B, H, n, d), 4300 + t) for t in range(4))
    sink = np.array([0.3, 2.0])
    lvec = (l4[0], l4[1], l4[2], l4[3], False)
    lm = fm.localize(mask_from(vec), B, n, n, chunks)      # the GPU's side
    g1 = run(q[:, :, rows], k, v, do[:, :, rows], lm, sink)
    compare(q[:, :, rows], k, v, do[:, :, rows], lvec, sink, g1)
    g2 = run(q[:, :, rows], k, v, do[:, :, rows], lm, sink)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
