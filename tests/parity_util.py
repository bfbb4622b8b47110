"""Helpers shared by the GPU parity tests: upload of generated inputs, the
oracle side of each comparison, and the tolerance / near-tie rules.

Tolerances (scores): |s_gpu - S| <= SCORE_ATOL + SCORE_RTOL * S elementwise,
S the float64 oracle score.  lse: |lse_gpu - lse| <= LSE_ATOL + LSE_RTOL*|lse|;
an lse error e moves every probability of its row by a factor exp(e), so the
lse bound is set to a tenth of the score's relative budget.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

SCORE_RTOL = 2e-3
SCORE_ATOL = 1e-6
LSE_ATOL = 2e-4
LSE_RTOL = 1e-6


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_scores(gpu: np.ndarray, ref: np.ndarray, what: str = "scores") -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    bound = SCORE_ATOL + SCORE_RTOL * np.abs(ref)
    bad = np.flatnonzero(err > bound)
    if bad.size:
        i = bad[0]
        raise AssertionError(
            f"{what}: {bad.size} of {ref.size} outside tolerance; first at {i}: "
            f"gpu={gpu.flat[i]!r} oracle={ref.flat[i]!r}")
    return float((err / np.maximum(np.abs(ref), 1e-30)).max())


def check_lse(gpu: np.ndarray, ref: np.ndarray, what: str = "lse") -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    err = np.abs(gpu - ref)
    bound = LSE_ATOL + LSE_RTOL * np.abs(ref)
    bad = np.flatnonzero(err > bound)
    if bad.size:
        i = bad[0]
        raise AssertionError(
            f"{what}: {bad.size} of {ref.size} outside tolerance; first at {i}: "
            f"gpu={gpu.flat[i]!r} oracle={ref.flat[i]!r}")
    return float(err.max())


def near_tie_band(ref_scores: np.ndarray, k: int):
    """(lo, hi) band around the k-th largest oracle score within which the
    order of GPU scores may legitimately differ from the oracle's: outside it
    the score tolerance alone decides membership."""
    tau = np.sort(ref_scores)[::-1][k - 1]
    r, a = SCORE_RTOL, SCORE_ATOL
    lo = (tau * (1 - r) - 2 * a) / (1 + r)
    hi = (tau * (1 + r) + 2 * a) / (1 - r)
    return lo, hi


def check_topk_band(kept: np.ndarray, ref_scores: np.ndarray, k: int) -> int:
    """Kept set chosen from GPU scores: exactly k distinct positions, all keys
    above the band kept, all below it dropped.  Returns the band population."""
    kept = np.asarray(kept)
    assert kept.size == k and np.unique(kept).size == k
    assert np.all(np.diff(kept) > 0), "kept positions must be ascending"
    lo, hi = near_tie_band(ref_scores, k)
    above = np.flatnonzero(ref_scores > hi)
    below = np.flatnonzero(ref_scores < lo)
    ks = set(kept.tolist())
    assert all(int(j) in ks for j in above), "a key above the near-tie band was dropped"
    assert not any(int(j) in ks for j in below), "a key below the near-tie band was kept"
    return int(np.sum((ref_scores >= lo) & (ref_scores <= hi)))


def check_valid_topk(scores: np.ndarray, kept: np.ndarray, k: int) -> None:
    """A kept set of flat positions is a valid top-k of these very scores,
    ties to the lower position (a property check that needs no oracle):
    k distinct ascending positions, no dropped score above the smallest kept
    one, and the kept scores equal to it are the lowest such positions."""
    scores = np.asarray(scores).reshape(-1)
    kept = np.asarray(kept, dtype=np.int64)
    assert kept.size == k and np.all(np.diff(kept) > 0), "k ascending positions"
    mask = np.zeros(scores.size, dtype=bool)
    mask[kept] = True
    thr = scores[mask].min()
    assert not np.any(scores[~mask] > thr), "a dropped score outranks a kept one"
    eq = np.flatnonzero(scores == thr)
    n_kept_eq = int(np.count_nonzero(mask[eq]))
    assert np.all(mask[eq[:n_kept_eq]]), "ties must go to the lower position"


def flat_kept(offsets: np.ndarray, idx: np.ndarray, n_c: int) -> np.ndarray:
    """Flat positions (l*H + h)*n_c + j of a CSR kept set."""
    counts = np.diff(offsets)
    heads = np.repeat(np.arange(counts.size, dtype=np.int64), counts)
    return heads * n_c + idx[:offsets[-1]].astype(np.int64)


def oracle_head(gen: dict, scale: float, workers: int = 1):
    q, kc, kn = oracle.workload_head_inputs(gen)
    if workers > 1:
        return oracle.head_scores_parallel(q, kc, kn, scale, workers=workers)
    return oracle.head_scores(q, kc, kn, scale)


def head_kept(offsets: np.ndarray, idx: np.ndarray, lh: int) -> np.ndarray:
    return idx[offsets[lh]:offsets[lh + 1]]
