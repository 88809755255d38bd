"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching the GPU (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

from sparse_masked_attention_amd import _binding
from _lib_fixture import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashmask.h")

FM_SUCCESS, FM_INVALID, FM_NOT_SUPPORTED, FM_WS_SMALL, FM_HIP = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(flashmask_\w+)\s*\(", text)))


def test_header_declares_the_abi():
    names = declared_symbols()
    for n in ["flashmask_tile_classify", "flashmask_fwd", "flashmask_bwd",
              "flashmask_workspace_size", "flashmask_status_string", "flashmask_table_block",
              "flashmask_tile_shape", "flashmask_tile_classify_qk", "flashmask_fwd_qk",
              "flashmask_bwd_qk", "flashmask_workspace_size_qk", "flashmask_localize",
              "flashmask_max_chunks", "flashmask_bwd_noalloc"]:
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (flashmask_\w+)", out))
    for n in declared_symbols():
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for s in range(5):
        assert _binding.status_string(s)
    assert _binding.status_string(99) == "unknown status"


def test_table_block_and_tile_shapes(lib):
    import torch
    assert _binding.table_block() == 64
    assert _binding.tile_shape(False, 128, torch.bfloat16) == (128, 64)
    assert _binding.tile_shape(False, 256, torch.bfloat16) == (128, 64)
    assert _binding.tile_shape(False, 64, torch.float32) == (128, 64)
    assert _binding.tile_shape(True, 128, torch.bfloat16) == (64, 128)
    assert _binding.tile_shape(True, 256, torch.bfloat16) == (32, 64)   # the wide kernels' backward
    assert _binding.tile_shape(True, 64, torch.float32) == (32, 128)
    # d = 192 exists with dv = 128: bf16 (wide forward, 32-row backward) and fp32 (wide both ways)
    assert _binding.tile_shape(False, 192, torch.bfloat16) == (128, 64)
    assert _binding.tile_shape(True, 192, torch.bfloat16) == (32, 128)
    assert _binding.tile_shape(False, 192, torch.float32) == (128, 64)
    assert _binding.tile_shape(True, 192, torch.float32) == (32, 64)
    # the wide head dims: 64-key backward blocks (and 64-row forward blocks at bf16 512)
    assert _binding.tile_shape(False, 512, torch.bfloat16) == (64, 64)
    assert _binding.tile_shape(True, 512, torch.bfloat16) == (32, 64)
    assert _binding.tile_shape(False, 256, torch.float32) == (128, 64)
    assert _binding.tile_shape(True, 256, torch.float32) == (32, 64)
    with pytest.raises(_binding.FlashMaskError):
        _binding.tile_shape(False, 96, torch.bfloat16)
    with pytest.raises(_binding.FlashMaskError):
        _binding.tile_shape(True, 512, torch.float32)


def test_workspace_size(lib):
    import torch
    fwd = _binding.workspace_size(False, 1, 32, 8192, 128, 128, 1, torch.bfloat16)
    assert fwd == 128 * 8 * 4              # the table: 128 key blocks x 8 int32
    # table, then delta, base-2 LSE and rowsum(dS) (the sink gradient's), one
    # float per row each, then the dK/dV pass's 8 work-queue counters (256 bytes)
    bwd = _binding.workspace_size(True, 1, 32, 8192, 128, 128, 1, torch.bfloat16)
    assert bwd == 4096 + 3 * 32 * 8192 * 4 + 256
    # fp32 the same: its dQ pass needs no accumulator
    bwd32 = _binding.workspace_size(True, 1, 32, 8192, 128, 128, 1, torch.float32)
    assert bwd32 == bwd
    assert _binding.workspace_size(False, 1, 1, 10, 96, 96, 1, torch.bfloat16) == 0
    # (d, dv) = (192, 128) for bf16 and fp32; the workspace does not depend on dv
    assert _binding.workspace_size(True, 1, 32, 8192, 192, 128, 1, torch.bfloat16) == bwd
    assert _binding.workspace_size(True, 1, 32, 8192, 192, 192, 1, torch.bfloat16) == 0
    assert _binding.workspace_size(True, 1, 32, 8192, 192, 128, 1, torch.float32) == bwd32
    assert _binding.workspace_size(True, 1, 32, 8192, 192, 192, 1, torch.float32) == 0


def _fwd_call(lib, q=1, k=1, v=1, o=1, lse=1, hm=1, B=1, H=2, N=16, d=128, dv=128,
              dtype=1, causal=1, table=None, ws=None, ws_bytes=0, uts=None, ute=None):
    p = lambda x: None if x is None else ctypes.c_void_p(x * 256)
    return lib.flashmask_fwd(p(q), p(k), p(v), p(1), None, p(uts), p(ute), hm, p(table),
                             B, H, N, d, dv, dtype, causal, 0.0, p(o), p(lse), None,
                             p(ws), ws_bytes, None)


def test_fwd_argument_checks(lib):
    assert _fwd_call(lib, q=None) == FM_INVALID
    assert _fwd_call(lib, o=None) == FM_INVALID
    assert _fwd_call(lib, hm=3, H=4) == FM_INVALID
    assert _fwd_call(lib, B=-1) == FM_INVALID
    assert _fwd_call(lib, d=96, dv=96) == FM_NOT_SUPPORTED
    assert _fwd_call(lib, d=128, dv=64) == FM_NOT_SUPPORTED
    assert _fwd_call(lib, d=192, dv=192) == FM_NOT_SUPPORTED
    assert _fwd_call(lib, d=128, dv=192) == FM_NOT_SUPPORTED
    assert _fwd_call(lib, dtype=0, d=192, dv=192) == FM_NOT_SUPPORTED
    assert _fwd_call(lib, dtype=0, d=512, dv=512) == FM_NOT_SUPPORTED
    assert _fwd_call(lib, d=512, dv=256) == FM_NOT_SUPPORTED
    assert _fwd_call(lib, d=384, dv=384) == FM_NOT_SUPPORTED
    assert _fwd_call(lib, dtype=7) == FM_INVALID
    assert _fwd_call(lib, ws=None) == FM_WS_SMALL
    assert _fwd_call(lib, ws=1, ws_bytes=8) == FM_WS_SMALL
    # non-causal with only one of the upper vectors
    assert _fwd_call(lib, causal=0, uts=1, ute=None) == FM_INVALID
    # empty problems succeed without touching anything
    assert _fwd_call(lib, q=None, N=0) == FM_SUCCESS
    assert _fwd_call(lib, q=None, B=0) == FM_SUCCESS


def test_bwd_argument_checks(lib):
    p = lambda x: None if x is None else ctypes.c_void_p(x * 256)

    def call(dq=1, ws=1, ws_bytes=1 << 40, d=128, N=16):
        return lib.flashmask_bwd(p(1), p(1), p(1), p(1), p(1), p(1), p(1), None, None, None, 1, None,
                                 1, 2, N, d, d, 1, 1, 0.0, p(dq), p(1), p(1), None, p(ws),
                                 ws_bytes, None)
    assert call(dq=None) == FM_INVALID
    assert call(ws=None) == FM_WS_SMALL
    assert call(ws_bytes=16) == FM_WS_SMALL
    assert call(d=80) == FM_NOT_SUPPORTED
    assert call(dq=None, N=0) == FM_SUCCESS


def test_classify_argument_checks(lib):
    p = lambda x: None if x is None else ctypes.c_void_p(x * 256)
    assert lib.flashmask_tile_classify(p(1), p(1), None, None, 1, 1, 16, 1, 0, 64, p(1), None, None) == FM_INVALID
    assert lib.flashmask_tile_classify(p(1), p(1), None, None, 1, 1, 16, 1, 64, 64, None, None, None) == FM_INVALID
    assert lib.flashmask_tile_classify(p(1), p(1), None, None, 1, 0, 16, 1, 64, 64, p(1), None, None) == FM_INVALID
    assert lib.flashmask_tile_classify(p(1), p(1), p(1), None, 1, 1, 16, 0, 64, 64, p(1), None, None) == FM_INVALID
    assert lib.flashmask_tile_classify(None, None, None, None, 1, 1, 0, 1, 64, 64, None, None, None) == FM_SUCCESS


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    m = _binding.Mask(None, None, None, None, True)
    with pytest.raises(ValueError):
        _binding.fwd(q, q, q, m)


def test_rectangular_workspace_and_empty_sides(lib):
    import torch
    # table over Nk keys, delta, base-2 LSE and rowsum(dS) over Nq rows, queue counters
    # 5 key blocks x 32 bytes -> 256; 3 x (1 x 2 x 100 floats) -> 3 x 1024; 8 ints -> 256
    assert _binding.workspace_size(True, 1, 2, 100, 128, 128, 1, torch.bfloat16, Nk=300) == \
        256 + 3 * 1024 + 256
    assert _binding.workspace_size(False, 1, 2, 100, 128, 128, 1, torch.bfloat16, Nk=0) == 0
    p = lambda x: None if x is None else ctypes.c_void_p(x * 256)
    fwd = lambda Nq, Nk, q=1: lib.flashmask_fwd_qk(p(q), p(1), p(1), p(1), None, None, None, 1, None,
                                                   1, 2, Nq, Nk, 128, 128, 1, 1, 0.0, None, p(1), p(1),
                                                   None, p(1), 1 << 30, None)
    assert fwd(0, 64, q=None) == FM_SUCCESS       # no query row: nothing to do
    assert fwd(16, -1) == FM_INVALID
    assert fwd(-1, 16) == FM_INVALID
    bwd = lambda Nq, Nk: lib.flashmask_bwd_qk(p(1), p(1), p(1), p(1), p(1), p(1), p(1), None, None,
                                              None, 1, None, 1, 2, Nq, Nk, 128, 128, 1, 1, 0.0, None,
                                              p(1), p(1), p(1), None, None, p(1), 1 << 30, None)
    assert bwd(0, 0) == FM_SUCCESS
    assert bwd(-3, 5) == FM_INVALID


def test_localize_argument_checks(lib):
    assert lib.flashmask_max_chunks() == _binding.max_chunks() >= 8
    p = lambda x: None if x is None else ctypes.c_void_p(x * 256)

    def call(chunks, n_rows=100, Nk=16, causal=1, outs=1):
        arr = (ctypes.c_int32 * max(1, len(chunks)))(*chunks) if chunks else None
        n = len(chunks) // 2
        return lib.flashmask_localize(p(1), None, None, None, 1, 1, Nk, n_rows, causal, arr, n,
                                      p(outs), p(outs), p(outs), p(outs), None)
    assert call([]) == FM_INVALID                       # no chunk
    assert call([10, 5]) == FM_INVALID                  # empty range
    assert call([0, 10, 5, 20]) == FM_INVALID           # overlapping
    assert call([20, 30, 0, 10]) == FM_INVALID          # not sorted
    assert call([0, 101]) == FM_INVALID                 # past the last row
    assert call([-1, 4]) == FM_INVALID
    assert call(list(range(0, 2 * 65 * 1, 1)), n_rows=1000) == FM_INVALID  # too many chunks
    assert call([0, 10], Nk=0) == FM_SUCCESS            # no key column: nothing to write
    assert call([0, 10], outs=None) == FM_INVALID


def test_noalloc_rejects_problems_beyond_its_scratch(lib):
    """flashmask_bwd_noalloc refuses a problem whose workspace exceeds its
    static scratch (16 MiB) on the host, before anything is enqueued; bad
    arguments are refused as in the other entry points."""
    p = lambda v: ctypes.c_void_p(v)
    scratch = 16 << 20

    def call(B, H, Nq, Nk, d=128, dv=128, hm=1, dtype=1):
        return lib.flashmask_bwd_noalloc(p(16), p(16), p(16), p(16), p(16), p(16), p(16), None,
                                         None, None, hm, None, B, H, Nq, Nk, d, dv, dtype, 1,
                                         ctypes.c_float(0.0), None, p(16), p(16), p(16), None, None,
                                         None)
    # 3 float32 row arrays of B*H*Nq plus the table: 32 heads x 65536 rows is 24 MiB
    assert _binding.lib().flashmask_workspace_size_qk(1, 1, 32, 65536, 65536, 128, 128, 1, 1) > scratch
    assert call(1, 32, 65536, 65536) == FM_WS_SMALL
    assert call(1, 1, 100, 100, hm=2) == FM_INVALID          # hm not in {1, H}
    assert call(1, 1, 100, 100, d=96, dv=96) == FM_NOT_SUPPORTED
    assert call(0, 4, 100, 100) == FM_SUCCESS                 # empty problem: a no-op
