"""Helpers shared by the GPU parity tests: seeded inputs, device transfer and
the error metrics and tolerances the parity bar states.

Tolerances (per output tensor, in float64 against the fp64 oracle on the
same bf16-rounded inputs): bf16 max-abs <= 2e-2 and relative L2 <= 5e-3;
fp32 max-abs <= 1e-5. Logsumexp: -inf entries must match exactly, finite
entries use the same absolute bound.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from sparse_masked_attention_amd import inputs as I
from sparse_masked_attention_amd import _binding as fm

BF16_ATOL = 2e-2
BF16_RL2 = 5e-3
FP32_ATOL = 1e-5


_METRICS = None


def say(*a):
    """Print (flushed) and append to gpurun_out/parity_metrics.txt when that folder exists."""
    global _METRICS
    print(*a, flush=True)
    sys.stdout.flush()
    if _METRICS is None:
        import os
        out = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "gpurun_out")
        _METRICS = open(os.path.join(out, "parity_metrics.txt"), "a") if os.path.isdir(out) else False
    if _METRICS:
        _METRICS.write(" ".join(str(x) for x in a) + "\n")
        _METRICS.flush()


def to_dev(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """float32 array (already bf16-exact for bf16 runs) -> device tensor."""
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def qkvo(B, H, N, d, seed_base, bf16=True, with_do=False):
    """Seeded Q, K, V (and dO) float32 arrays, bf16-representable when bf16."""
    shapes = (B, H, N, d)
    out = [I.randn(shapes, seed_base + t, bf16=bf16) for t in range(4 if with_do else 3)]
    return out


def mask_from(vectors, device="cuda") -> fm.Mask:
    lts, lte, uts, ute, causal = vectors
    return fm.Mask.from_numpy(lts, lte, uts, ute, causal, device=device)


def metrics(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    denom = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / denom) if denom > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def check_bf16(name, got, ref, atol=BF16_ATOL, rl2=BF16_RL2):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    ma, rel = metrics(got, ref)
    say(f"  {name}: max_abs={ma:.3e} rel_l2={rel:.3e}")
    assert ma <= atol and rel <= rl2, f"{name}: max_abs {ma:.3e} rel_l2 {rel:.3e}"


def check_fp32(name, got, ref, atol=FP32_ATOL):
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    ma, _ = metrics(got, ref)
    say(f"  {name}: max_abs={ma:.3e}")
    assert ma <= atol, f"{name}: max_abs {ma:.3e}"


def check_lse(got, ref, atol):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    ninf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf_ref), "logsumexp -inf pattern differs"
    fin = ~ninf_ref
    if fin.any():
        ma = float(np.abs(got[fin] - ref[fin]).max())
        say(f"  lse: max_abs={ma:.3e}")
        assert ma <= atol, f"lse max_abs {ma:.3e}"
