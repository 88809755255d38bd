"""Parity under a second tile configuration (lib/libflashmask_alt.so, built
with FM_ALT_TILES: one 32-key block per forward inner step, 32-row backward
query steps at every head dim, so the d <= 128 dK/dV pass runs in its
non-persistent form, and a shorter forward tile list, so long rows take
more list rounds).

The kernels' LDS staging, barriers and list handling then run with other
tile sizes, stage sizes and timing; an ordering mistake that the default
configuration happens to hide would show here. Every case is checked
against the fp64 oracle, not against the default library.
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

DIMS = [(64, 64), (128, 128), (256, 256), (192, 128)]
FAMILIES = ["causal", "document", "share_question", "sliding_window", "block_sparse", "all_open"]


@pytest.fixture(scope="module", autouse=True)
def _alt_library():
    ensure_built()
    with fm.library(fm.ALT_LIB_PATH):
        yield


def _inputs(B, H, N, d, dv, seed):
    return (I.randn((B, H, N, d), seed), I.randn((B, H, N, d), seed + 1),
            I.randn((B, H, N, dv), seed + 2), I.randn((B, H, N, dv), seed + 3))


def _run(q, k, v, do, vec, fcounts=None, bcounts=None):
    m = mask_from(vec)
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    o, lse = fm.fwd(qd, kd, vd, m, tile_counts=fcounts)
    dq, dk, dv = fm.bwd(qd, kd, vd, o, lse, dod, m, tile_counts=bcounts)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _compare(q, k, v, do, vec, got):
    lts, lte, uts, ute, causal = vec
    ro, rl = oracle.forward(q, k, v, causal, lts, lte, uts, ute)
    ref = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute)
    o, lse, dq, dk, dv = (to_np(x) for x in got)
    rf, rb = replays(q, k, v, do, vec)
    check_bf16("O", o, ro, replay=rf[0])
    check_lse(lse, rl, BF16_ATOL)
    for i, (name, g, r) in enumerate(zip(("dQ", "dK", "dV"), (dq, dk, dv), ref)):
        check_bf16(name, g, r, replay=rb[i])


def test_alt_library_reports_its_tile_shape():
    assert fm.tile_shape(True, 128, torch.bfloat16) == (32, 128)
    assert fm.tile_shape(True, 64, torch.bfloat16) == (32, 128)
    assert fm.tile_shape(False, 128, torch.bfloat16) == (128, 64)


@pytest.mark.parametrize("family", FAMILIES)
@pytest.mark.parametrize("N", [129, 1000])
@pytest.mark.parametrize("d,dv", DIMS)
def test_families(d, dv, family, N):
    say(f"alt tiles d={d} dv={dv} family={family} N={N}")
    q, k, v, do = _inputs(1, 2, N, d, dv, 9000)
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(23))])
    _compare(q, k, v, do, vec, _run(q, k, v, do, vec))


@pytest.mark.parametrize("d,dv", DIMS)
def test_tile_counts_and_determinism(d, dv):
    B, H, N = 2, 2, 700
    say(f"alt tiles d={d} dv={dv} tile counts and determinism")
    q, k, v, do = _inputs(B, H, N, d, dv, 9100)
    vec = I.stack_masks([I.make_mask("prefix_lm_document", N, np.random.default_rng(40 + b)) for b in range(B)])
    fc = torch.zeros(3, dtype=torch.int64, device="cuda")
    bc = torch.zeros(3, dtype=torch.int64, device="cuda")
    got1 = _run(q, k, v, do, vec, fcounts=fc, bcounts=bc)
    got2 = _run(q, k, v, do, vec)
    lts, lte, uts, ute, causal = vec
    for is_bwd, counts in ((False, fc), (True, bc)):
        bq, bk = fm.tile_shape(is_bwd, d, torch.bfloat16)
        t = oracle.kblock_minmax(B, 1, N, bk, lts, lte, uts, ute)
        ref = oracle.classify_counts(oracle.classify(t, N, bq, bk, causal)) * H
        assert counts.cpu().numpy().tolist() == ref.tolist(), (is_bwd, bq, bk)
    for a, b in zip(got1, got2):
        assert torch.equal(a, b)
    _compare(q, k, v, do, vec, got1)


def test_long_rows_take_several_list_rounds():
    """N = 40000, causal: a late query block sees 625 key blocks, more than
    the shorter tile list holds, so its tiles are walked in rounds; 512
    stratified late rows against the oracle."""
    B, H, N, d = 1, 1, 40000, 64
    say(f"alt tiles long rows N={N}")
    q, k, v = (I.randn((B, H, N, d), 9200 + t) for t in range(3))
    vec = I.stack_masks([I.make_mask("causal", N, np.random.default_rng(0))])
    m = mask_from(vec)
    o, lse = fm.fwd(*(to_dev(x, torch.bfloat16) for x in (q, k, v)), m)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(1).choice(np.arange(N - 4096, N), 512, replace=False))
    lts, lte, uts, ute, causal = vec
    ro, rl = oracle.forward_rows(q[0, 0], k[0, 0], v[0, 0], N, causal, oracle.mask_row(lts, 0, 0),
                                 oracle.mask_row(lte, 0, 0), None, None, rows=rows)
    check_bf16("O rows", to_np(o[0, 0])[rows], ro)
    check_lse(to_np(lse[0, 0])[rows], rl, BF16_ATOL)
