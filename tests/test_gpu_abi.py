"""The C ABI on the GPU, called directly through ctypes.

  * The square entry points flashmask_tile_classify, flashmask_fwd and
    flashmask_bwd (Nq = Nk = N, no sink), with their argument lists written
    out here, in bf16 and fp32: outputs against the oracle, bitwise against
    the rectangular entry points the binding uses, and inside guarded
    buffers so a write outside its tensor shows.
  * Every output of the backward (and of the forward) inside guarded buffers
    for every compiled (d, dv) and dtype at N in {1, 7, 129, 1000}.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm
from gpu_util import (BF16_ATOL, FP32_ATOL, check_bf16, check_fp32, check_lse, mask_from, replays,
                      say, to_dev, to_np)
from _lib_fixture import ensure_built

pytestmark = pytest.mark.gpu

PAD = 4096          # guard elements on each side (keeps 16-byte alignment)
GUARD = 7.0         # guard value (exact in bf16 and fp32)
BF16_DIMS = [(64, 64), (128, 128), (256, 256), (192, 128), (512, 512)]
FP32_DIMS = [(64, 64), (128, 128), (256, 256), (192, 128)]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


class Guarded:
    """A tensor of `shape` inside a buffer with PAD guard elements before and after."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape))
        self.buf = torch.full((n + 2 * PAD,), GUARD, dtype=dtype, device="cuda")
        self.t = self.buf[PAD:PAD + n].view(*shape)
        self.n = n

    def intact(self):
        return bool((self.buf[:PAD] == GUARD).all()) and bool((self.buf[PAD + self.n:] == GUARD).all())


def ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def code(dtype):
    return 1 if dtype == torch.bfloat16 else 0


def check_grads(q, k, v, do, vec, got, ref, bf):
    if not bf:
        for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
            check_fp32(name, to_np(g), r)
        return
    _, rb = replays(q, k, v, do, vec)
    for i, (name, g, r) in enumerate(zip(("dQ", "dK", "dV"), got, ref)):
        check_bf16(name, to_np(g), r, replay=rb[i])


def vec_ptrs(m: fm.Mask):
    return [ptr(x) for x in (m.lts, m.lte, m.uts, m.ute)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("family", ["document", "prefix_lm_document"])
def test_square_entry_points(dtype, family):
    B, H, N, d = 2, 2, 333, 64
    bf = dtype == torch.bfloat16
    say(f"square entry points {family} {dtype}")
    lib = fm.lib()
    q, k, v, do = (I.randn((B, H, N, d), 5100 + t, bf16=bf) for t in range(4))
    vec = I.stack_masks([I.make_mask(family, N, np.random.default_rng(30 + b)) for b in range(B)])
    lts, lte, uts, ute, causal = vec
    m = mask_from(vec)
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    hm = m.hm

    # flashmask_tile_classify (square): table and class map, guarded
    bt = lib.flashmask_table_block()
    bq, bk = 128, bt
    nkb, nqb = -(-N // bk), -(-N // bq)
    table = Guarded((B, hm, nkb, 8), torch.int32)
    cls = Guarded((B, hm, nqb, nkb), torch.int8)
    st = lib.flashmask_tile_classify(*vec_ptrs(m), B, hm, N, int(causal), bq, bk,
                                     ptr(table.t), ptr(cls.t), stream())
    assert st == 0
    torch.cuda.synchronize()
    assert table.intact() and cls.intact()
    ref_t = oracle.kblock_minmax(B, hm, N, bk, lts, lte, uts, ute)
    np.testing.assert_array_equal(table.t.cpu().numpy(), ref_t)
    np.testing.assert_array_equal(cls.t.cpu().numpy(), oracle.classify(ref_t, N, bq, bk, causal))

    # flashmask_fwd (square), once with the precomputed table and once without
    ws_f = lib.flashmask_workspace_size(0, B, H, N, d, d, hm, code(dtype))
    wsf = torch.empty(max(ws_f, 1), dtype=torch.uint8, device="cuda")
    outs = []
    for tab in (table.t, None):
        o = Guarded((B, H, N, d), dtype)
        lse = Guarded((B, H, N), torch.float32)
        st = lib.flashmask_fwd(ptr(qd), ptr(kd), ptr(vd), *vec_ptrs(m), hm, ptr(tab),
                               B, H, N, d, d, code(dtype), int(causal), ctypes.c_float(0.0),
                               ptr(o.t), ptr(lse.t), None, ptr(wsf), ctypes.c_size_t(wsf.numel()),
                               stream())
        assert st == 0
        torch.cuda.synchronize()
        assert o.intact() and lse.intact()
        outs.append((o, lse))
    (o, lse), (o2, lse2) = outs
    assert torch.equal(o.t, o2.t) and torch.equal(lse.t, lse2.t)
    ro, rl = oracle.forward(q, k, v, causal, lts, lte, uts, ute)
    (check_bf16 if bf else check_fp32)("O", to_np(o.t), ro)
    check_lse(to_np(lse.t), rl, BF16_ATOL if bf else FP32_ATOL)
    o_qk, l_qk = fm.fwd(qd, kd, vd, m)
    torch.cuda.synchronize()
    assert torch.equal(o.t, o_qk) and torch.equal(lse.t, l_qk)

    # flashmask_bwd (square)
    ws_b = lib.flashmask_workspace_size(1, B, H, N, d, d, hm, code(dtype))
    wsb = torch.empty(ws_b, dtype=torch.uint8, device="cuda")
    dq, dk, dv = (Guarded((B, H, N, d), dtype) for _ in range(3))
    counts = torch.zeros(3, dtype=torch.int64, device="cuda")
    st = lib.flashmask_bwd(ptr(qd), ptr(kd), ptr(vd), ptr(o.t), ptr(lse.t), ptr(dod), *vec_ptrs(m), hm,
                           ptr(table.t), B, H, N, d, d, code(dtype), int(causal), ctypes.c_float(0.0),
                           ptr(dq.t), ptr(dk.t), ptr(dv.t), ptr(counts), ptr(wsb),
                           ctypes.c_size_t(wsb.numel()), stream())
    assert st == 0
    torch.cuda.synchronize()
    assert dq.intact() and dk.intact() and dv.intact()
    rq, rk, rv = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute)
    check_grads(q, k, v, do, vec, (dq.t, dk.t, dv.t), (rq, rk, rv), bf)
    g_qk = fm.bwd(qd, kd, vd, o.t, lse.t, dod, m)
    torch.cuda.synchronize()
    for a, b in zip((dq.t, dk.t, dv.t), g_qk):
        assert torch.equal(a, b)
    # the backward's tile counters equal the oracle's class histogram
    tbq, tbk = fm.tile_shape(True, d, dtype)
    t2 = oracle.kblock_minmax(B, hm, N, tbk, lts, lte, uts, ute)
    ref = oracle.classify_counts(oracle.classify(t2, N, tbq, tbk, causal)) * H
    assert counts.cpu().numpy().tolist() == ref.tolist()


CASES = [(d, dv, torch.bfloat16) for d, dv in BF16_DIMS] + [(d, dv, torch.float32) for d, dv in FP32_DIMS]


@pytest.mark.parametrize("N", [1, 7, 129, 1000])
@pytest.mark.parametrize("d,dv,dtype", CASES)
def test_guarded_outputs(d, dv, dtype, N):
    B, H = 1, 2
    bf = dtype == torch.bfloat16
    say(f"guarded outputs d={d} dv={dv} {dtype} N={N}")
    q = I.randn((B, H, N, d), 5200, bf16=bf)
    k = I.randn((B, H, N, d), 5201, bf16=bf)
    v = I.randn((B, H, N, dv), 5202, bf16=bf)
    do = I.randn((B, H, N, dv), 5203, bf16=bf)
    vec = I.stack_masks([I.make_mask("document", N, np.random.default_rng(7))])
    lts, lte, uts, ute, causal = vec
    m = mask_from(vec)
    qd, kd, vd, dod = (to_dev(x, dtype) for x in (q, k, v, do))
    o = Guarded((B, H, N, dv), dtype)
    lse = Guarded((B, H, N), torch.float32)
    fm.fwd(qd, kd, vd, m, out=o.t, lse=lse.t)
    dq, dk = Guarded((B, H, N, d), dtype), Guarded((B, H, N, d), dtype)
    dvv = Guarded((B, H, N, dv), dtype)
    fm.bwd(qd, kd, vd, o.t, lse.t, dod, m, grads=(dq.t, dk.t, dvv.t))
    torch.cuda.synchronize()
    for name, g in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dvv)):
        assert g.intact(), f"{name}: a write outside the tensor"
    ro, rl = oracle.forward(q, k, v, causal, lts, lte, uts, ute)
    rq, rk, rv = oracle.backward(q, k, v, do, causal, lts, lte, uts, ute)
    (check_bf16 if bf else check_fp32)("O", to_np(o.t), ro)
    check_lse(to_np(lse.t), rl, BF16_ATOL if bf else FP32_ATOL)
    check_grads(q, k, v, do, vec, (dq.t, dk.t, dvv.t), (rq, rk, rv), bf)
