"""Oracle of the row localisation of one context-parallel rank's share
(test infrastructure only; the library never calls it).

The FlashMask-3 abstract says each rank localises the column-wise mask with
no communication ("clip-shift-max") before it attends its own query rows to
all keys. The pages give the name, not the formula. Reading taken: the rank
holds the global query rows of some chunks [q0_c, q1_c), sorted and
disjoint, and numbers them 0, 1, ... in that order. A global row bound t
(a start or an end of a half-open row interval stored for a key column)
becomes

    local(t) = sum over chunks c of clip(t - q0_c, 0, q1_c - q0_c)

i.e. shift t to the chunk's start, clip it to the chunk (the "max" with 0 is
the lower clip), and add the chunk lengths it covers. A global interval
[a, b) then holds exactly the local rows whose global rows it held. The
causal edge (global rows i < j hidden from key j) becomes the upper interval
[0, local(j)), so the local mask is the non-causal four-vector form.

Everything here is plain Python integer arithmetic, element by element; the
pin is brute force (tests/test_oracle_rect.py): the dense mask decoded from
the local vectors equals the rows of the global dense mask the rank holds.
"""
from __future__ import annotations

import numpy as np

__all__ = ["rank_rows", "local_bound", "localize"]


def _chunks(chunks, n_rows):
    out = [(int(a), int(b)) for a, b in np.asarray(chunks, np.int64).reshape(-1, 2)]
    if not out:
        raise ValueError("no chunks")
    prev = 0
    for a, b in out:
        if a < prev or b <= a or b > n_rows:
            raise ValueError("chunks must be sorted, disjoint, non-empty and inside [0, n_rows]")
        prev = b
    return out


def rank_rows(chunks, n_rows):
    """Global row of each local row: the chunks' rows in order."""
    rows = []
    for a, b in _chunks(chunks, n_rows):
        rows.extend(range(a, b))
    return np.array(rows, np.int64)


def local_bound(t: int, chunks) -> int:
    """local(t): the number of the rank's rows that lie before global row t."""
    total = 0
    for a, b in chunks:
        total += min(max(t - a, 0), b - a)
    return total


def localize(lts, lte, uts, ute, causal, chunks, n_rows):
    """The four local vectors (int32 [B, hm, Nk] each) of the mask restricted to
    the rank's rows, and the local causal flag (False).

    Vector conventions follow the oracle's: lts None means no lower interval;
    lte None means LTE = n_rows; with causal False, uts/ute None means no upper
    interval. The outputs always hold all four vectors, with the empty
    intervals [Nq, Nq) and [0, 0) where nothing is hidden.
    """
    ch = _chunks(chunks, n_rows)
    nq = sum(b - a for a, b in ch)
    ref = next((v for v in (lts, lte, uts, ute) if v is not None), None)
    if ref is None:
        raise ValueError("pass at least one vector")
    shape = np.asarray(ref).shape
    B, hm, nk = shape
    out = [np.zeros(shape, np.int64) for _ in range(4)]
    for b in range(B):
        for h in range(hm):
            for j in range(nk):
                if lts is None:
                    l_lts = l_lte = nq
                else:
                    end = n_rows if lte is None else int(lte[b][h][j])
                    l_lts = local_bound(int(lts[b][h][j]), ch)
                    l_lte = local_bound(end, ch)
                if causal:
                    l_uts, l_ute = 0, local_bound(j, ch)
                elif uts is not None and ute is not None:
                    l_uts = local_bound(int(uts[b][h][j]), ch)
                    l_ute = local_bound(int(ute[b][h][j]), ch)
                else:
                    l_uts, l_ute = 0, 0
                out[0][b, h, j], out[1][b, h, j] = l_lts, l_lte
                out[2][b, h, j], out[3][b, h, j] = l_uts, l_ute
    return tuple(x.astype(np.int32) for x in out) + (False,)
