"""flashmask_bwd_noalloc (the backward without a workspace argument, for
callers that cannot allocate) against flashmask_bwd_qk with a caller-owned
workspace: same inputs, bitwise the same dQ, dK, dV (and dsink), and the
oracle's parity bar, on two calls in a row, the second smaller than the
first (the static scratch keeps the first call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm
from gpu_util import check_bf16, mask_from, replays, say, to_dev, to_np
from _lib_fixture import ensure_built

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc_bwd(qd, kd, vd, o, lse, dod, m, sink=None):
    B, H, Nq, d = qd.shape
    Nk, dv = kd.shape[2], vd.shape[-1]
    dq, dk, dvv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    dsink = None if sink is None else torch.empty(H, dtype=torch.float32, device="cuda")
    st = fm.lib().flashmask_bwd_noalloc(
        ptr(qd), ptr(kd), ptr(vd), ptr(o), ptr(lse), ptr(dod), ptr(m.lts), ptr(m.lte), ptr(m.uts),
        ptr(m.ute), m.hm, None, B, H, Nq, Nk, d, dv, 1, int(m.causal), ctypes.c_float(0.0), ptr(sink),
        ptr(dq), ptr(dk), ptr(dvv), ptr(dsink), None,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fm.status_string(st)
    return (dq, dk, dvv) if sink is None else (dq, dk, dvv, dsink)


# the first call is the larger one; the second, smaller, reuses the scratch
CASES = [
    dict(B=2, H=4, N=1500, d=128, family="share_question", sink=True),
    dict(B=1, H=2, N=300, d=64, family="document", sink=False),
]


def test_noalloc_backward_equals_workspace_backward():
    for c in CASES:
        B, H, N, d = c["B"], c["H"], c["N"], c["d"]
        say(f"noalloc bwd B={B} H={H} N={N} d={d} family={c['family']} sink={c['sink']}")
        q, k, v, do = (I.randn((B, H, N, d), 6100 + t) for t in range(4))
        vec = I.stack_masks([I.make_mask(c["family"], N, np.random.default_rng(40 + b)) for b in range(B)])
        m = mask_from(vec)
        qd, kd, vd, dod = (to_dev(x, torch.bfloat16) for x in (q, k, v, do))
        sink = torch.linspace(-1.0, 1.5, H, device="cuda") if c["sink"] else None
        o, lse = fm.fwd(qd, kd, vd, m, sink=sink)
        ref_ws = fm.bwd(qd, kd, vd, o, lse, dod, m, sink=sink)
        got = noalloc_bwd(qd, kd, vd, o, lse, dod, m, sink=sink)
        torch.cuda.synchronize()
        for a, b in zip(got, ref_ws):
            assert torch.equal(a, b)
        lts, lte, uts, ute, causal = vec
        sk = None if sink is None else sink.cpu().numpy()
        ref = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute, sink=sk)
        _, rb = replays(q, k, v, do, vec, sink=sk)
        for i, name in enumerate(("dQ", "dK", "dV")):
            check_bf16(name, to_np(got[i]), ref[i], replay=rb[i])
        if sink is not None:
            err = np.abs(to_np(got[3]) - ref[3])
            assert (err <= 2e-2 + 5e-3 * np.abs(ref[3])).all()
