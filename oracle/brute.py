"""Scalar brute force for tiny shapes - TEST INFRASTRUCTURE ONLY.

A second, independent rendering of the same definitions as oracle.kvzip, in
plain Python loops with exactly rounded sums (math.fsum) and no NumPy, no
max-shift and no log-sum-exp: each probability is the ratio exp(x_j) / sum of
exp over the keys the row sees.  Used only to pin the NumPy oracle on shapes
small enough for loops (n_c <= ~16, d <= ~8).

Definitions (KVzip page "KVzip: Query-Agnostic KV Cache Compression with
Context Reconstruction", section 3.2 and its displayed max equation; section
4.1 for the r% budget):
  row (g, i) of the repeat pass sees the n_c cached keys and new keys 0..i;
  A[g, i, j] = exp(x_j) / sum_{j' seen} exp(x_j'), x_j = scale * <q_gi, k_j>;
  S[j] = max over g, i of A[g, i, j] for cached keys j < n_c.
"""
from __future__ import annotations

import itertools
import math
from typing import List, Sequence, Tuple


def brute_scores(q: Sequence, k_ctx: Sequence, k_new: Sequence, scale: float
                 ) -> Tuple[List[float], List[List[float]], List[List[List[float]]]]:
    """q: G x n_in x d nested lists; k_ctx: n_c x d; k_new: n_in x d.
    returns (S[n_c], lse[G][n_in], A[G][n_in][n_c + n_in])."""
    G = len(q)
    n_in = len(q[0])
    n_c = len(k_ctx)
    keys = [list(r) for r in k_ctx] + [list(r) for r in k_new]
    S = [0.0] * n_c
    lse = [[0.0] * n_in for _ in range(G)]
    A = [[[0.0] * (n_c + n_in) for _ in range(n_in)] for _ in range(G)]
    for g in range(G):
        for i in range(n_in):
            seen = list(range(n_c)) + [n_c + t for t in range(i + 1)]
            x = {}
            for j in seen:
                x[j] = scale * math.fsum(qa * kb for qa, kb in zip(q[g][i], keys[j]))
            z = math.fsum(math.exp(x[j]) for j in seen)
            lse[g][i] = math.log(z)
            for j in seen:
                A[g][i][j] = math.exp(x[j]) / z
                if j < n_c and A[g][i][j] > S[j]:
                    S[j] = A[g][i][j]
    return S, lse, A


def brute_topk(scores: Sequence[float], k: int) -> List[int]:
    """Enumerate every k-subset; return the unique one in which every kept
    entry precedes every dropped entry in the order (higher score, then lower
    index).  Raises if the count of such subsets is not exactly one."""
    n = len(scores)

    def before(a: int, b: int) -> bool:
        return scores[a] > scores[b] or (scores[a] == scores[b] and a < b)

    found = []
    for sub in itertools.combinations(range(n), k):
        kept = set(sub)
        if all(before(a, b) for a in kept for b in range(n) if b not in kept):
            found.append(list(sub))
    if len(found) != 1:
        raise AssertionError(f"{len(found)} valid subsets")
    return found[0]
