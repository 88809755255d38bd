"""The backward's persistent dK/dV pass when every workgroup runs several
work items, with the forward and dQ pass on the same inputs.

The dK/dV pass keeps one workgroup per compute unit resident; each takes
(batch, head, 128-key block) items from work queues and starts its next
item before it writes the last one. These cases have several times more
items than resident workgroups (256 on 256 compute units), with per-batch
document masks, so an item set up from the wrong table row or classified
with stale bounds shows as wrong rows. Both queue layouts are covered: eight
per-XCD queues (B*H a multiple of 8) and a single queue. Each case runs
three times on one workspace: the outputs are bitwise the same every time
(the queue counters are set up afresh by each call) and match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm
from gpu_util import check_bf16, check_lse, BF16_ATOL, mask_from, replays, say, to_dev, to_np
from _lib_fixture import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def _case(B, H, N, d, seed):
    q, k, v, do = (I.randn((B, H, N, d), seed + t) for t in range(4))
    rng = np.random.default_rng(seed)
    vec = I.stack_masks([I.make_mask("document", N, rng) for _ in range(B)])
    return q, k, v, do, vec


@pytest.mark.parametrize("B,H,N,d", [(24, 16, 333, 64),    # 1152 dK/dV items, 8 queues
                                     (77, 5, 200, 64),     # 770 items, one queue
                                     (8, 16, 600, 128)])   # 640 items, 8 queues
def test_many_items_per_workgroup(B, H, N, d):
    say(f"persistent dK/dV pass B={B} H={H} N={N} d={d}")
    q, k, v, do, vec = _case(B, H, N, d, 7300 + d)
    lts, lte, uts, ute, causal = vec
    m = mask_from(vec)
    qd, kd, vd, dod = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
    wsf = torch.zeros(fm.workspace_size(False, B, H, N, d, d, m.hm, torch.bfloat16),
                      dtype=torch.uint8, device="cuda")
    wsb = torch.zeros(fm.workspace_size(True, B, H, N, d, d, m.hm, torch.bfloat16),
                      dtype=torch.uint8, device="cuda")
    runs = []
    for _ in range(3):
        o, lse = fm.fwd(qd, kd, vd, m, workspace=wsf)
        g = fm.bwd(qd, kd, vd, o, lse, dod, m, workspace=wsb)
        torch.cuda.synchronize()
        runs.append((o, lse) + tuple(g))
    for r in runs[1:]:
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), runs[0], r):
            assert torch.equal(a, b), f"{name} differs between calls"
    o, lse, dq, dk, dv = runs[0]
    ro, rl = oracle.forward(q, k, v, causal, lts, lte, uts, ute)
    check_bf16("O", to_np(o), ro)
    check_lse(to_np(lse), rl, BF16_ATOL)
    rq, rk, rv = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute)
    _, rb = replays(q, k, v, do, vec)
    for i, (name, got, ref) in enumerate(zip(("dQ", "dK", "dV"), (dq, dk, dv), (rq, rk, rv))):
        check_bf16(name, to_np(got), ref, replay=rb[i])
