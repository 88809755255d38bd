"""MI355X (gfx950) exact attention with FlashMask's column-wise sparse mask.

The computation lives in libflashmask.so (HIP kernels behind the C ABI of
include/flashmask.h). This package holds the ctypes binding, the seeded
synthetic input generators and the exact FLOP counter used for throughput.
"""
from ._binding import (FlashMaskError, Mask, bwd, fwd, lib, status_string, table_block,
                       tile_classify, tile_shape, workspace_size, LIB_PATH)

__all__ = ["FlashMaskError", "Mask", "bwd", "fwd", "lib", "status_string", "table_block",
           "tile_classify", "tile_shape", "workspace_size", "LIB_PATH"]
