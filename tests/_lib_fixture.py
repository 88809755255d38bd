"""Shared test helpers: make sure the library is built before use."""
import os

from sparse_masked_attention_amd import _binding


def ensure_built():
    """Build the libraries (libflashmask.so and the second tile configuration,
    libflashmask_alt.so) only if one is missing (the GPU machine gets them prebuilt)."""
    if not (os.path.exists(_binding.LIB_PATH) and os.path.exists(_binding.ALT_LIB_PATH)):
        from sparse_masked_attention_amd import build
        build.build(verbose=False)
    return _binding.lib()
