"""Routing inputs for the gated merge: which kept row each evicted token is
merged into.  The SelKV page's routing section is not part of its text, so
the merge takes routing as an input; this module makes one such input, the
nearest kept position of the same head (ties to the earlier kept position).
It is an input recipe, shared by the tests and the benchmark, and holds
none of the gate or merge arithmetic.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def nearest_position_routes(offsets: np.ndarray, idx: np.ndarray, n_c: int
                            ) -> Tuple[np.ndarray, np.ndarray]:
    """CSR routing lists: for every kept row t (global row of the CSR kept
    set), the evicted positions of its head whose nearest kept position is
    idx[t], ascending.  Returns (src_offsets int64 [total+1], src_idx int32)."""
    offsets = np.asarray(offsets, dtype=np.int64)
    idx = np.asarray(idx, dtype=np.int64)
    total = int(offsets[-1])
    counts = np.zeros(total, dtype=np.int64)
    lists = []
    for lh in range(offsets.size - 1):
        a, b = int(offsets[lh]), int(offsets[lh + 1])
        kept = idx[a:b]
        if kept.size == 0:
            continue
        mask = np.ones(n_c, dtype=bool)
        mask[kept] = False
        ev = np.flatnonzero(mask)
        k = np.searchsorted(kept, ev)
        lo = np.clip(k - 1, 0, kept.size - 1)
        hi = np.clip(k, 0, kept.size - 1)
        pick = np.where(np.abs(ev - kept[lo]) <= np.abs(kept[hi] - ev), lo, hi)
        rows = a + pick
        order = np.lexsort((ev, rows))
        lists.append((rows[order], ev[order]))
        np.add.at(counts, rows, 1)
    src_offsets = np.zeros(total + 1, dtype=np.int64)
    np.cumsum(counts, out=src_offsets[1:])
    if lists:
        rows = np.concatenate([r for r, _ in lists])
        src = np.concatenate([e for _, e in lists])
        src = src[np.argsort(rows, kind="stable")]
    else:
        src = np.zeros(0, dtype=np.int64)
    return src_offsets, src.astype(np.int32)
