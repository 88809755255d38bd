"""Plain fp64 CPU oracle of column-wise sparse masked attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this package; only
the tests, the smoke check and the CPU-baseline leg of the benchmark do. It
shares no code with the HIP path. Every function states the definition it
writes out; see each module's docstring for the passages followed.

Pins (tests/test_oracle_pins.py): every function here is checked against
something other than itself (textbook attention, finite differences, brute
force, closed forms, hand-worked fixtures).
"""
from .attention import (dense_mask, mask_row, forward, forward_rows, backward, backward_sampled,
                        softmax_probs)
from .tables import kblock_minmax, classify, classify_counts, nnz_dense
from .localize import rank_rows, local_bound, localize
from . import bf16_replay
from . import families

__all__ = ["dense_mask", "mask_row", "forward", "forward_rows", "backward",
           "backward_sampled", "softmax_probs", "kblock_minmax", "classify", "classify_counts",
           "nnz_dense", "rank_rows", "local_bound", "localize", "bf16_replay", "families"]
