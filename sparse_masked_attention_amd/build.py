"""Compile the HIP sources into lib/libflashmask.so for gfx950 (hipcc, ahead of time).

Usage: python -m sparse_masked_attention_amd.build   (or __graft_entry__.build())
Objects are compiled in parallel into _build/ at the repository root, then
linked into one shared library that exports the C ABI of include/flashmask.h.

The same sources are also built a second time with FM_ALT_TILES into
lib/libflashmask_alt.so: a second tile configuration (one 32-key block per
forward inner step, 32-row backward query steps at every head dim, a
shorter forward tile list) that only the parity tests load, so that an LDS
race or a tiling assumption that happens to hold for one configuration is
tested under another.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "lib", "libflashmask.so")
ALT_LIB = os.path.join(PKG, "lib", "libflashmask_alt.so")
SOURCES = ["fm_api.hip", "fm_classify.hip", "fm_fwd.hip", "fm_bwd.hip", "fm_localize.hip",
           "fm_wide.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-inline-asm", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(job) -> str:
    src, alt = job
    out = os.path.join(BUILD, "alt") if alt else BUILD
    obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *(["-DFM_ALT_TILES"] if alt else []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}{' (FM_ALT_TILES)' if alt else ''}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    shutil.move(tmp, lib)


def build(verbose: bool = True, alt: bool = True) -> str:
    """Build lib/libflashmask.so (and, with alt, lib/libflashmask_alt.so)."""
    os.makedirs(os.path.join(BUILD, "alt"), exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    jobs = [(src, False) for src in SOURCES] + ([(src, True) for src in SOURCES] if alt else [])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(SOURCES)], LIB)
    if verbose:
        print(f"built {LIB}")
    if alt:
        _link(objs[len(SOURCES):], ALT_LIB)
        if verbose:
            print(f"built {ALT_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
