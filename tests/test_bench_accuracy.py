"""bench.py's per-run accuracy fields: the largest relative score error, the
within-tolerance flag and the near-tie band around each head's budget threshold
(KVzip page, "KVzip: Query-Agnostic KV Cache Compression with Context
Reconstruction", section 4.1), on hand-made scores whose answers are known."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _f32(x):
    """Scores exactly representable in fp32, as the GPU returns them."""
    return np.asarray(x, np.float32).astype(np.float64)


def _one_head(S, gpu, kept_idx, keep):
    n = S.size
    ref = {(0, 0): S}
    scores = gpu.reshape(1, 1, n).astype(np.float32)
    offsets = np.array([0, kept_idx.size], np.int64)
    return bench.accuracy_fields(ref, scores, offsets, kept_idx.astype(np.int32), keep, 0)


def test_exact_scores_and_a_clean_threshold():
    # 10 well-separated scores, keep 3: tau = 0.8, band = scores within
    # ~0.2 % of 0.8: only 0.8 itself
    S = _f32([0.1, 0.9, 0.2, 0.8, 0.3, 0.7, 0.4, 0.6, 0.5, 1.0])
    f = _one_head(S, S, np.array([1, 3, 9]), 0.3)
    assert f["max_rel_err"] == 0.0 and f["scores_within_tol"]
    assert f["near_tie_band"] == 1 and f["topk_outside_band_ok"]
    assert f["heads_checked"] == 1


def test_band_population_and_relative_error():
    # keys 3 and 5 sit 0.1 % apart at the threshold: both in the band, and
    # either may be kept
    S = _f32([0.1, 0.9, 0.2, 0.8, 0.3, 0.8008, 0.4, 0.6, 0.5, 1.0])
    gpu = S * (1 + 1e-3)          # 0.1 % high everywhere: within tolerance
    f = _one_head(S, gpu, np.array([1, 3, 9]), 0.3)
    assert abs(f["max_rel_err"] - 1e-3) < 1e-6 and f["scores_within_tol"]
    assert f["near_tie_band"] == 2 and f["topk_outside_band_ok"]


def test_violations_are_reported():
    S = _f32([0.1, 0.9, 0.2, 0.8, 0.3, 0.7, 0.4, 0.6, 0.5, 1.0])
    gpu = S.copy()
    gpu[2] *= 1.01                # 1 % off: outside the 2e-3 tolerance
    f = _one_head(S, gpu, np.array([1, 2, 9]), 0.3)   # and key 3 (0.8) dropped for key 2
    assert abs(f["max_rel_err"] - 0.01) < 1e-6 and not f["scores_within_tol"]
    assert not f["topk_outside_band_ok"]


def test_no_reference_gives_nulls():
    f = bench.accuracy_fields(None, None, None, None, 0.3, 0)
    assert f["max_rel_err"] is None and f["heads_checked"] == 0
