"""Key-block table and tile classes on the GPU equal the oracle bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm
from gpu_util import mask_from, say
from _lib_fixture import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def _run(vectors, B, N, bq, bk):
    lts, lte, uts, ute, causal = vectors
    present = [v for v in (lts, lte, uts, ute) if v is not None]
    hm = present[0].shape[1] if present else 1
    m = mask_from(vectors)
    table, cls = fm.tile_classify(m, B, N, bq, bk)
    torch.cuda.synchronize()
    ref_t = oracle.kblock_minmax(B, hm, N, bk, lts, lte, uts, ute)
    ref_c = oracle.classify(ref_t, N, bq, bk, causal)
    assert np.array_equal(table.cpu().numpy(), ref_t), "table differs"
    assert np.array_equal(cls.cpu().numpy(), ref_c), "classes differ"


@pytest.mark.parametrize("family", ["document", "causal", "all_open", "share_question",
                                    "sliding_window", "prefix_lm_document", "block_sparse"])
@pytest.mark.parametrize("N", [1, 7, 129, 1000, 8192])
def test_families(family, N):
    say(f"classify family={family} N={N}")
    B = 2
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(10 + b)) for b in range(B)])
    for bq, bk in [(128, 64), (64, 128), (128, 128)]:
        _run(vec, B, N, bq, bk)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("causal", [True, False])
def test_arbitrary_int32_values(seed, causal):
    rng = np.random.default_rng(seed)
    B, hm, N = 2, 3, int(rng.integers(1, 3000))
    say(f"classify arbitrary seed={seed} causal={causal} N={N}")
    lo, hi = np.iinfo(np.int32).min, np.iinfo(np.int32).max
    v = [rng.integers(-50, N + 50, (B, hm, N)).astype(np.int32) for _ in range(4)]
    v[0][0, 0, :3] = [lo, hi, 0]
    v[1][0, 0, :3] = [hi, lo, N]
    vec = (v[0], v[1], None if causal else v[2], None if causal else v[3], causal)
    for bq, bk in [(128, 64), (1, 1), (7, 100), (64, 3000)]:
        _run(vec, B, N, bq, bk)


def test_missing_vectors_take_neutral_values():
    N, B = 300, 1
    say("classify missing vectors")
    lts = I.causal_document(N, [100, 200]).lts[None, None]
    _run((lts, None, None, None, True), B, N, 128, 64)
    _run((None, None, None, None, True), B, N, 128, 64)
    _run((None, None, None, None, False), B, N, 100, 30)
    uts = np.zeros((1, 1, N), np.int32)
    ute = (np.arange(N, dtype=np.int32) // 2)[None, None]
    _run((lts, None, uts, ute, False), B, N, 64, 64)
