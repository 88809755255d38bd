"""The C ABI layer's argument and size checks under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

fm_api.hip is compiled again with both sanitizers on its host code only
(each -fsanitize flag behind -Xarch_host; the device code is built as
usual) and linked with the other objects of the normal build and
tests/sanitize/abi_driver.c. The driver calls every entry point with
arguments the checks must turn away (null and misaligned pointers, bad
sizes, sizes too large to address, unsupported dims, bad chunk lists) and
the size and shape queries, each with the status it must return. Nothing
reaches a kernel launch. Runs only where no GPU is present (the driver's
pointers are made up).
"""
import os
import shutil
import subprocess

import pytest
import torch

from _lib_fixture import ensure_built

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_masked_attention_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN = ["address", "undefined"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@pytest.mark.skipif(torch.cuda.is_available(), reason="the driver's made-up pointers are for a host without a GPU")
@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)), reason="ROCm compilers not found")
def test_abi_checks_clean_under_asan_and_ubsan(tmp_path):
    ensure_built()
    others = [os.path.join(BUILD, f) for f in ("fm_classify.o", "fm_fwd.o", "fm_bwd.o", "fm_localize.o",
                                               "fm_wide.o")]
    if not all(os.path.exists(o) for o in others):     # library present, objects cleaned away
        from sparse_masked_attention_amd import build
        build.build(verbose=False)
    assert all(os.path.exists(o) for o in others), "objects of the normal build are missing"
    san_host = [f for s in SAN for f in ("-Xarch_host", f"-fsanitize={s}")]
    api_o = str(tmp_path / "fm_api_san.o")
    _run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *san_host,
          "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
          "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(CSRC, "fm_api.hip"), "-o", api_o])
    drv_o = str(tmp_path / "abi_driver.o")
    _run([CLANG, "-O1", "-g", "-std=c11", f"-fsanitize={','.join(SAN)}", "-fno-sanitize-recover=all",
          "-I", os.path.join(ROOT, "include"), "-c", os.path.join(ROOT, "tests", "sanitize", "abi_driver.c"),
          "-o", drv_o])
    exe = str(tmp_path / "abi_driver")
    _run([CLANGXX, f"-fsanitize={','.join(SAN)}", drv_o, api_o, *others, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    out = r.stdout + r.stderr
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert "0 failure(s)" in r.stdout
