"""Float64 CPU oracle for the SelKV soft cosine gate and a gated merge.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The library's product
path never calls it, and it shares no code with the GPU kernels.

What the SelKV page ("Selective KV cache merging", section 1, the first of
its two mechanisms) fixes: every evicted token is routed to a merge target
among the kept tokens; the gate g = max(cos(v_e, v_t), 0), the cosine
similarity of the evicted token's value vector and the target's, sets how
strongly it is merged: g near 1 merges fully, g = 0 drops it, values in
between merge partially.  The page's text ends with its section 3.1, so the
routing (its section 3.4), the merge formula and the attention compensation
are not on it.

Readings taken here:
  - routing is an input: for every kept row, the list of evicted positions
    of the same head routed to it (any routing rule can produce it);
  - the gate compares the evicted value with the target's original value;
    a zero-length vector has no direction and gets g = 0;
  - merge: the kept row becomes the weighted mean of itself (weight 1) and
    its routed tokens (weight g each), for keys and values alike:
        x_t' = (x_t + sum_e g_e x_e) / (1 + sum_e g_e);
    with every g = 0 this is plain eviction, with every g = 1 a uniform mean;
  - the merge mass sum_e g_e of every kept row is reported (the quantity a
    count-based compensation would use).

Parity unpinned for the merged rows as the page's method: the merge formula
is not on the page, so the pins of merge() check this reading (closed forms
of the weighted mean, planted mistakes), not the page.  The gate itself is
pinned against the page's definition.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def soft_cosine_gate(v_e: np.ndarray, v_t: np.ndarray) -> float:
    """g = max(cos(v_e, v_t), 0); 0 when either vector has zero length."""
    v_e = np.asarray(v_e, dtype=np.float64)
    v_t = np.asarray(v_t, dtype=np.float64)
    ne, nt = np.sqrt(np.dot(v_e, v_e)), np.sqrt(np.dot(v_t, v_t))
    if ne == 0.0 or nt == 0.0:
        return 0.0
    return max(float(np.dot(v_e, v_t) / (ne * nt)), 0.0)


def merge_compact(k_ctx: np.ndarray, v_ctx: np.ndarray, offsets: np.ndarray,
                  idx: np.ndarray, src_offsets: np.ndarray, src_idx: np.ndarray
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Gated merge of routed tokens into the kept rows.

    k_ctx, v_ctx : (L, H, n_c, d) float arrays
    offsets, idx : CSR kept set (row t of head lh keeps position idx[t])
    src_offsets  : (total + 1,) CSR over kept rows of the routed positions
    src_idx      : positions j in the kept row's head; out-of-range entries
                   are ignored (gate 0)
    returns k_out, v_out (total, d) float64, gate (n_src,), mass (total,)
    """
    L, H, n_c, d = k_ctx.shape
    total = int(offsets[-1])
    k_out = np.zeros((total, d))
    v_out = np.zeros((total, d))
    gate = np.zeros(int(src_offsets[-1]))
    mass = np.zeros(total)
    for lh in range(L * H):
        l, h = divmod(lh, H)
        K = np.asarray(k_ctx[l, h], dtype=np.float64)
        V = np.asarray(v_ctx[l, h], dtype=np.float64)
        for t in range(int(offsets[lh]), int(offsets[lh + 1])):
            kt, vt = K[idx[t]], V[idx[t]]
            ksum, vsum, wsum = kt.copy(), vt.copy(), 1.0
            for s in range(int(src_offsets[t]), int(src_offsets[t + 1])):
                j = int(src_idx[s])
                if not 0 <= j < n_c:
                    continue
                g = soft_cosine_gate(V[j], vt)
                gate[s] = g
                ksum += g * K[j]
                vsum += g * V[j]
                wsum += g
            k_out[t] = ksum / wsum
            v_out[t] = vsum / wsum
            mass[t] = wsum - 1.0
    return k_out, v_out, gate, mass
