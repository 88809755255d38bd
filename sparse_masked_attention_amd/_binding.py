"""ctypes binding of libflashmask.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
only turns torch tensors into device pointers, allocates outputs and the
workspace with torch (the library itself never allocates), and passes the
current torch stream. It raises if the library has not been built: there is
no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = ["FlashMaskError", "Mask", "lib", "status_string", "table_block", "tile_shape",
           "workspace_size", "tile_classify", "fwd", "bwd", "localize", "max_chunks", "LIB_PATH",
           "ALT_LIB_PATH", "library"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libflashmask.so")
# the second tile configuration (built alongside; see build.py)
ALT_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libflashmask_alt.so")

FM_FP32 = 0
FM_BF16 = 1

_c_void_p = ctypes.c_void_p
_c_int = ctypes.c_int
_c_size_t = ctypes.c_size_t
_c_float = ctypes.c_float

_SIGNATURES = {
    "flashmask_status_string": (ctypes.c_char_p, [_c_int]),
    "flashmask_table_block": (_c_int, []),
    "flashmask_tile_shape": (_c_int, [_c_int, _c_int, _c_int, ctypes.POINTER(_c_int), ctypes.POINTER(_c_int)]),
    "flashmask_workspace_size": (_c_size_t, [_c_int] * 7 + [_c_int]),
    "flashmask_tile_classify": (_c_int, [_c_void_p] * 4 + [_c_int] * 6 + [_c_void_p, _c_void_p, _c_void_p]),
    "flashmask_fwd": (_c_int, [_c_void_p] * 3 + [_c_void_p] * 4 + [_c_int, _c_void_p]
                      + [_c_int] * 5 + [_c_int, _c_int, _c_float]
                      + [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "flashmask_bwd": (_c_int, [_c_void_p] * 6 + [_c_void_p] * 4 + [_c_int, _c_void_p]
                      + [_c_int] * 5 + [_c_int, _c_int, _c_float]
                      + [_c_void_p] * 4 + [_c_void_p, _c_size_t, _c_void_p]),
    "flashmask_workspace_size_qk": (_c_size_t, [_c_int] * 8 + [_c_int]),
    "flashmask_tile_classify_qk": (_c_int, [_c_void_p] * 4 + [_c_int] * 7 + [_c_void_p, _c_void_p, _c_void_p]),
    "flashmask_fwd_qk": (_c_int, [_c_void_p] * 3 + [_c_void_p] * 4 + [_c_int, _c_void_p]
                         + [_c_int] * 6 + [_c_int, _c_int, _c_float, _c_void_p]
                         + [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_size_t, _c_void_p]),
    "flashmask_bwd_qk": (_c_int, [_c_void_p] * 6 + [_c_void_p] * 4 + [_c_int, _c_void_p]
                         + [_c_int] * 6 + [_c_int, _c_int, _c_float, _c_void_p]
                         + [_c_void_p] * 5 + [_c_void_p, _c_size_t, _c_void_p]),
    "flashmask_bwd_noalloc": (_c_int, [_c_void_p] * 6 + [_c_void_p] * 4 + [_c_int, _c_void_p]
                              + [_c_int] * 6 + [_c_int, _c_int, _c_float, _c_void_p]
                              + [_c_void_p] * 5 + [_c_void_p]),
    "flashmask_max_chunks": (_c_int, []),
    "flashmask_localize": (_c_int, [_c_void_p] * 4 + [_c_int] * 5 + [_c_void_p, _c_int]
                           + [_c_void_p] * 4 + [_c_void_p]),
}

_lib = None


class FlashMaskError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


def _load(path: str):
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m sparse_masked_attention_amd.build`")
    handle = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    return handle


def lib():
    """Load libflashmask.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Inside the block, every call of this module goes to the library at
    ``path`` (same C ABI): the parity tests use it for the second tile
    configuration, ALT_LIB_PATH."""
    global _lib
    saved = _lib
    _lib = _load(path)
    try:
        yield _lib
    finally:
        _lib = saved


def status_string(status: int) -> str:
    return lib().flashmask_status_string(int(status)).decode()


def table_block() -> int:
    return int(lib().flashmask_table_block())


def tile_shape(is_bwd: bool, d: int, dtype: torch.dtype):
    bq, bk = _c_int(), _c_int()
    st = lib().flashmask_tile_shape(int(is_bwd), d, _dtype_code(dtype), ctypes.byref(bq), ctypes.byref(bk))
    if st != 0:
        raise FlashMaskError("flashmask_tile_shape", st)
    return bq.value, bk.value


def workspace_size(is_bwd: bool, B, H, N, d, dv, hm, dtype: torch.dtype, Nk: Optional[int] = None) -> int:
    """Workspace bytes; N query rows and Nk keys (default Nk = N)."""
    nk = N if Nk is None else Nk
    return int(lib().flashmask_workspace_size_qk(int(is_bwd), B, H, N, nk, d, dv, hm, _dtype_code(dtype)))


def max_chunks() -> int:
    return int(lib().flashmask_max_chunks())


@dataclass
class Mask:
    """The four int32 boundary vectors [B, hm, Nk] on the device (None = absent)."""
    lts: Optional[torch.Tensor]
    lte: Optional[torch.Tensor]
    uts: Optional[torch.Tensor]
    ute: Optional[torch.Tensor]
    causal: bool

    @property
    def hm(self) -> int:
        for t in (self.lts, self.uts, self.lte, self.ute):
            if t is not None:
                return int(t.shape[1])
        return 1

    @staticmethod
    def from_numpy(lts, lte, uts, ute, causal, device="cuda"):
        conv = lambda a: None if a is None else torch.from_numpy(a).to(device=device, dtype=torch.int32).contiguous()
        return Mask(conv(lts), conv(lte), conv(uts), conv(ute), bool(causal))


def _dtype_code(dtype: torch.dtype) -> int:
    if dtype == torch.bfloat16:
        return FM_BF16
    if dtype == torch.float32:
        return FM_FP32
    raise ValueError(f"unsupported dtype {dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _sink(sink: Optional[torch.Tensor], H: int) -> Optional[torch.Tensor]:
    if sink is None:
        return None
    if sink.dtype != torch.float32 or sink.numel() != H:
        raise ValueError("sink must be float32 with one logit per head")
    return sink.contiguous()


def _check(fn: str, st: int):
    if st != 0:
        raise FlashMaskError(fn, st)


def _mask_ptrs(mask: Mask):
    for t in (mask.lts, mask.lte, mask.uts, mask.ute):
        if t is not None and t.dtype != torch.int32:
            raise ValueError("mask vectors must be int32")
    return _ptr(mask.lts), _ptr(mask.lte), _ptr(mask.uts), _ptr(mask.ute)


def tile_classify(mask: Mask, B: int, N: int, block_q: int, block_k: int, classes: bool = True,
                  table: Optional[torch.Tensor] = None, Nk: Optional[int] = None):
    """(table int32 [B,hm,ceil(Nk/block_k),8], classes int8 [B,hm,nqb,nkb] or None)
    for N query rows and Nk keys (default Nk = N).

    ``table``: optional preallocated output for the table."""
    dev = next(t for t in (mask.lts, mask.lte, mask.uts, mask.ute) if t is not None).device \
        if any(t is not None for t in (mask.lts, mask.lte, mask.uts, mask.ute)) else torch.device("cuda")
    hm = mask.hm
    nk = N if Nk is None else Nk
    nkb = -(-nk // block_k)
    nqb = -(-N // block_q)
    if table is None:
        table = torch.empty((B, hm, nkb, 8), dtype=torch.int32, device=dev)
    cls = torch.empty((B, hm, nqb, nkb), dtype=torch.int8, device=dev) if classes else None
    st = lib().flashmask_tile_classify_qk(*_mask_ptrs(mask), B, hm, N, nk, int(mask.causal), block_q,
                                          block_k, _ptr(table), _ptr(cls), _stream(dev))
    _check("flashmask_tile_classify", st)
    return table, cls


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: Mask, scale: Optional[float] = None,
        table: Optional[torch.Tensor] = None, tile_counts: Optional[torch.Tensor] = None,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None):
    """O [B,H,Nq,dv] (q's dtype) and logsumexp [B,H,Nq] float32.

    q [B,H,Nq,d], k [B,H,Nk,d], v [B,H,Nk,dv]; the mask vectors have Nk
    entries (Nq == Nk is the plain case). sink: optional float32 [H] sink
    logits."""
    B, H, N, d = q.shape
    Nk = k.shape[2]
    dv = v.shape[-1]
    if (k.shape[:2] != q.shape[:2] or k.shape[-1] != d or v.shape[:3] != k.shape[:3]
            or k.dtype != q.dtype or v.dtype != q.dtype):
        raise ValueError("q, k, v shapes/dtypes disagree")
    o = torch.empty((B, H, N, dv), dtype=q.dtype, device=q.device) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    ws_bytes = workspace_size(False, B, H, N, d, dv, mask.hm, q.dtype, Nk=Nk)
    ws = workspace
    if ws is None and table is None and ws_bytes > 0:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    st = lib().flashmask_fwd_qk(_ptr(q), _ptr(k), _ptr(v), *_mask_ptrs(mask), mask.hm, _ptr(table),
                                B, H, N, Nk, d, dv, _dtype_code(q.dtype), int(mask.causal),
                                0.0 if scale is None else float(scale), _ptr(_sink(sink, H)),
                                _ptr(o), _ptr(l), _ptr(tile_counts), _ptr(ws),
                                0 if ws is None else ws.numel(), _stream(q.device))
    _check("flashmask_fwd_qk", st)
    return o, l


def bwd(q, k, v, o, lse, dout, mask: Mask, scale: Optional[float] = None,
        table: Optional[torch.Tensor] = None, tile_counts: Optional[torch.Tensor] = None,
        workspace: Optional[torch.Tensor] = None, grads=None, sink: Optional[torch.Tensor] = None):
    """(dQ, dK, dV) in q's dtype (shapes as in fwd); with a sink also
    d loss / d sink (float32 [H]) as a fourth result."""
    B, H, N, d = q.shape
    Nk = k.shape[2]
    dv = v.shape[-1]
    if grads is None:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dvv = torch.empty_like(v)
    else:
        dq, dk, dvv = grads
    dsink = None if sink is None else torch.empty(H, dtype=torch.float32, device=q.device)
    ws_bytes = workspace_size(True, B, H, N, d, dv, mask.hm, q.dtype, Nk=Nk)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = lib().flashmask_bwd_qk(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout),
                                *_mask_ptrs(mask), mask.hm, _ptr(table),
                                B, H, N, Nk, d, dv, _dtype_code(q.dtype), int(mask.causal),
                                0.0 if scale is None else float(scale), _ptr(_sink(sink, H)),
                                _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(dsink), _ptr(tile_counts), _ptr(ws),
                                ws.numel(), _stream(q.device))
    _check("flashmask_bwd_qk", st)
    return (dq, dk, dvv) if sink is None else (dq, dk, dvv, dsink)


def localize(mask: Mask, B: int, Nk: int, n_rows: int, chunks) -> Mask:
    """The mask restricted to one rank's query rows, computed on the GPU by
    flashmask_localize: chunks are (q0, q1) global row ranges, sorted and
    disjoint; the result is non-causal with all four vectors [B, hm, Nk]."""
    import numpy as np
    c = np.ascontiguousarray(np.asarray(chunks, np.int32).reshape(-1, 2))
    dev = next((t.device for t in (mask.lts, mask.lte, mask.uts, mask.ute) if t is not None),
               torch.device("cuda"))
    hm = mask.hm
    outs = [torch.empty((B, hm, Nk), dtype=torch.int32, device=dev) for _ in range(4)]
    st = lib().flashmask_localize(*_mask_ptrs(mask), B, hm, Nk, n_rows, int(mask.causal),
                                  c.ctypes.data_as(ctypes.c_void_p), int(c.shape[0]),
                                  *[_ptr(t) for t in outs], _stream(dev))
    _check("flashmask_localize", st)
    return Mask(outs[0], outs[1], outs[2], outs[3], False)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
