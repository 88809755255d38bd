"""Shared test helpers: make sure the library is built before use."""
import os

from sparse_masked_attention_amd import _binding


def ensure_built():
    """Build libflashmask.so only if it is missing (the GPU machine gets it prebuilt)."""
    if not os.path.exists(_binding.LIB_PATH):
        from sparse_masked_attention_amd import build
        build.build(verbose=False)
    return _binding.lib()
