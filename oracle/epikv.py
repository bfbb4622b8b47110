"""Float64 CPU oracle for the attention-free EpiKV token score.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The library's product
path never calls it, and it shares no code with the GPU kernels.

What it computes, in the notation of the EpiKV page ("EpiKV", section 3.2,
hidden-state variation signal, equations 1 to 3):

* Eq. 1: for layer l and position t, g_l(t) is the L2 norm of the change of
  the hidden state, h_l(t) - h_l(t-1).
* Eq. 2 (raw score): s(t) is the rolling mean of g over a causal window of
  the past w = 64 positions in band A minus the same in band B; tokens with
  high s are kept.
* Eq. 3 (time-trend correction, the page's main variant): each g_l(t) is
  replaced by its causal rolling z-score (g_l(t) - mu_l(t)) / (sigma_l(t) +
  eps), mu and sigma the mean and standard deviation of g_l over the window,
  and the score is z_A(t) - z_B(t).
* Section 3.1 (problem setting): a budget of K tokens; the K highest-scoring
  positions stay in the cache of every layer and head, the rest are dropped.

Readings taken where the page is silent or loose:
  - position 0 has no predecessor, so g(0) is undefined: it is stored as 0,
    no window contains it, and every score of position 0 is 0;
  - the window of position t >= 1 holds the defined positions
    max(1, t - w + 1) .. t, the current one included (the page calls the
    window causal over positions <= t); it is the same window for eq. 2's
    rolling mean and eq. 3's mean and deviation;
  - sigma is the population standard deviation (divide by the window count);
  - eps is a caller argument (1e-6 by default);
  - bands: the page names bands of layers (7-13, 18-25) but scores with one
    layer from each (10 and 21); a band here is any set of layers and its
    value is the mean over its layers, which is eq. 2 / eq. 3 exactly when
    each band holds one layer;
  - ties in the top-K go to the lower position; kept positions ascend; -0.0
    and +0.0 are equal.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np

DEFAULT_WINDOW = 64
DEFAULT_EPS = 1e-6


def hidden_deltas(h: np.ndarray) -> np.ndarray:
    """Eq. 1.  h: (n, D) hidden states of one layer (any float dtype).
    Returns g (n,) float64 with g[t] = ||h[t] - h[t-1]||_2 and g[0] = 0."""
    h = np.asarray(h, dtype=np.float64)
    n = h.shape[0]
    g = np.zeros(n)
    for t in range(1, n):
        diff = h[t] - h[t - 1]
        g[t] = np.sqrt(np.dot(diff, diff))
    return g


def window(t: int, w: int) -> range:
    """Positions of the causal window of position t (empty for t = 0)."""
    if t < 1:
        return range(0)
    return range(max(1, t - w + 1), t + 1)


def rolling_mean(g: np.ndarray, w: int = DEFAULT_WINDOW) -> np.ndarray:
    """Eq. 2's g-hat: mean of g over the window of each position."""
    g = np.asarray(g, dtype=np.float64)
    out = np.zeros(g.shape[0])
    for t in range(g.shape[0]):
        win = window(t, w)
        if len(win):
            out[t] = np.mean(g[win.start:win.stop])
    return out


def rolling_zscore(g: np.ndarray, w: int = DEFAULT_WINDOW,
                   eps: float = DEFAULT_EPS) -> np.ndarray:
    """Eq. 3: z(t) = (g(t) - mean) / (population std + eps) over the window."""
    g = np.asarray(g, dtype=np.float64)
    out = np.zeros(g.shape[0])
    for t in range(g.shape[0]):
        win = window(t, w)
        if len(win):
            x = g[win.start:win.stop]
            mu = np.mean(x)
            sigma = np.sqrt(np.mean((x - mu) ** 2))
            out[t] = (g[t] - mu) / (sigma + eps)
    return out


def token_scores(g_a: Sequence[np.ndarray], g_b: Sequence[np.ndarray],
                 w: int = DEFAULT_WINDOW, eps: float = DEFAULT_EPS,
                 detrend: bool = True) -> np.ndarray:
    """Eq. 3 (detrend=True, the main variant) or eq. 2 (detrend=False):
    band A's mean per-layer statistic minus band B's."""
    if len(g_a) < 1 or len(g_b) < 1:
        raise ValueError("each band needs at least one layer")
    stat = (lambda g: rolling_zscore(g, w, eps)) if detrend else (lambda g: rolling_mean(g, w))
    a = np.mean([stat(g) for g in g_a], axis=0)
    b = np.mean([stat(g) for g in g_b], axis=0)
    return a - b


def select_tokens(scores: np.ndarray, k: int) -> np.ndarray:
    """Section 3.1's budget: the k highest-scoring positions (ties to the
    lower position), ascending, as int32."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    if not 1 <= k <= n:
        raise ValueError("need 1 <= k <= n")
    order = np.lexsort((np.arange(n), -scores))
    return np.sort(order[:k]).astype(np.int32)


def compact_tokens(k_cache: np.ndarray, v_cache: np.ndarray, idx: np.ndarray):
    """The kept positions of every (layer, head): (L, H, n, d) -> (L, H, K, d),
    bit copies."""
    return np.take(k_cache, idx, axis=2), np.take(v_cache, idx, axis=2)
