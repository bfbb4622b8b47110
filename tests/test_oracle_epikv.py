"""Pins of the EpiKV oracle (EpiKV page, section 3.2, equations 1 to 3, and
section 3.1's top-K budget) against closed forms, exact rational arithmetic,
independent library routines and brute force."""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import epikv as E
from oracle.brute import brute_topk


# ---- eq. 1: hidden-state change ------------------------------------------
def test_deltas_pythagorean():
    h = np.array([[0, 0], [3, 4], [3, 4], [0, 0], [5, 12]], dtype=np.float64)
    assert E.hidden_deltas(h).tolist() == [0.0, 5.0, 0.0, 5.0, 13.0]
    assert E.hidden_deltas(h[:1]).tolist() == [0.0]


def test_deltas_match_math_dist():
    rng = np.random.default_rng(1)
    h = rng.normal(size=(30, 17))
    g = E.hidden_deltas(h)
    for t in range(1, 30):
        assert abs(g[t] - math.dist(h[t], h[t - 1])) < 1e-13 * (1 + g[t])


def test_deltas_of_a_ray_are_constant():
    u = np.array([1.0, -2.0, 2.0])          # |u| = 3
    h = np.outer(np.arange(10) * 0.5, u) + 7.0
    assert np.allclose(E.hidden_deltas(h)[1:], 1.5, rtol=0, atol=1e-13)


# ---- the window ------------------------------------------------------------
def test_window_positions():
    assert list(E.window(0, 4)) == []
    assert list(E.window(1, 4)) == [1]
    assert list(E.window(3, 4)) == [1, 2, 3]
    assert list(E.window(4, 4)) == [1, 2, 3, 4]
    assert list(E.window(9, 4)) == [6, 7, 8, 9]
    assert list(E.window(9, 1)) == [9]


# ---- eq. 2: rolling mean ---------------------------------------------------
def test_rolling_mean_ramp_closed_form():
    w, n = 8, 40
    g = np.arange(n, dtype=np.float64)       # g(t) = t
    m = E.rolling_mean(g, w)
    assert m[0] == 0.0
    for t in range(1, n):
        want = (t + 1) / 2 if t < w else t - (w - 1) / 2
        assert abs(m[t] - want) < 1e-12


def test_rolling_mean_constant():
    g = np.full(50, 2.5)
    g[0] = 0.0
    m = E.rolling_mean(g, 64)
    assert m[0] == 0.0 and np.all(m[1:] == 2.5)


# ---- eq. 3: rolling z-score ------------------------------------------------
def test_zscore_ramp_closed_form():
    # window of m consecutive integers ending at t: mean t - (m-1)/2,
    # population variance (m^2 - 1) / 12
    w, n, eps = 16, 60, 1e-6
    g = np.arange(n, dtype=np.float64)
    z = E.rolling_zscore(g, w, eps)
    assert z[0] == 0.0 and z[1] == 0.0       # no window / one sample
    for t in range(2, n):
        m = min(t, w)
        want = ((m - 1) / 2) / (math.sqrt((m * m - 1) / 12) + eps)
        assert abs(z[t] - want) < 1e-12 * (1 + want), t


def test_zscore_constant_is_zero():
    g = np.full(100, 3.0)
    assert np.all(E.rolling_zscore(g, 64) == 0.0)


def test_zscore_exact_rationals():
    rng = np.random.default_rng(2)
    w, eps = 5, 1e-6
    g = rng.integers(0, 20, size=25).astype(np.float64)
    z = E.rolling_zscore(g, w, eps)
    for t in range(1, 25):
        xs = [Fraction(int(g[j])) for j in range(max(1, t - w + 1), t + 1)]
        mu = sum(xs) / len(xs)
        var = sum((x - mu) ** 2 for x in xs) / len(xs)
        want = float(Fraction(int(g[t])) - mu) / (math.sqrt(float(var)) + eps)
        assert abs(z[t] - want) < 1e-12 * (1 + abs(want)), t


def test_zscore_samuelson_bound_and_affine_invariance():
    rng = np.random.default_rng(3)
    g = rng.lognormal(size=400)
    w = 64
    z = E.rolling_zscore(g, w, 1e-300)      # eps > 0 but negligible
    for t in range(2, 400):
        m = min(t, w)
        # Samuelson: a sample is within sqrt(m - 1) population deviations of the mean
        assert abs(z[t]) <= math.sqrt(m - 1) + 1e-12
    z2 = E.rolling_zscore(3.0 * g + 11.0, w, 1e-300)
    assert np.allclose(z2[2:], z[2:], rtol=1e-9, atol=1e-9)


# ---- combined score ----------------------------------------------------------
def test_score_bands():
    rng = np.random.default_rng(4)
    ga, gb = rng.lognormal(size=200), rng.lognormal(size=200)
    const = np.full(200, 1.0)
    za = E.rolling_zscore(ga)
    assert np.array_equal(E.token_scores([ga], [const]), za - 0.0)
    assert np.array_equal(E.token_scores([gb], [ga]), -E.token_scores([ga], [gb]))
    assert np.allclose(E.token_scores([ga, ga], [gb]), E.token_scores([ga], [gb]), atol=1e-15)
    # raw variant (eq. 2) on a ramp against a constant band
    ramp = np.arange(200, dtype=np.float64)
    raw = E.token_scores([ramp], [const], detrend=False)
    assert raw[0] == 0.0
    assert abs(raw[150] - ((150 - 31.5) - 1.0)) < 1e-12
    with pytest.raises(ValueError):
        E.token_scores([], [gb])


# ---- section 3.1: top-K -----------------------------------------------------
@pytest.mark.parametrize("seed", range(8))
def test_select_tokens_brute(seed):
    rng = np.random.default_rng(50 + seed)
    n = 6 + seed % 6
    s = (rng.integers(-3, 3, size=n) / 2.0).astype(np.float64)
    s[rng.integers(n)] = -0.0
    for k in range(1, n + 1):
        assert E.select_tokens(s, k).tolist() == brute_topk(list(s), k)


def test_select_tokens_signed_zero_and_errors():
    s = np.array([-0.0, 0.0, -1.0, 0.0])
    assert E.select_tokens(s, 1).tolist() == [0]   # -0.0 == +0.0: lower position
    assert E.select_tokens(s, 3).tolist() == [0, 1, 3]
    with pytest.raises(ValueError):
        E.select_tokens(s, 0)
    with pytest.raises(ValueError):
        E.select_tokens(s, 5)


def test_compact_tokens():
    rng = np.random.default_rng(6)
    k = rng.integers(0, 2 ** 16, size=(2, 3, 20, 4), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(2, 3, 20, 4), dtype=np.uint16)
    idx = np.array([0, 5, 6, 19], dtype=np.int32)
    ko, vo = E.compact_tokens(k, v, idx)
    assert ko.shape == (2, 3, 4, 4)
    for l in range(2):
        for h in range(3):
            for t, j in enumerate(idx):
                assert np.array_equal(ko[l, h, t], k[l, h, j])
                assert np.array_equal(vo[l, h, t], v[l, h, j])


# ---- planted mistakes: each must be caught by a pin above -----------------
def _zscore_sample_std(g, w=E.DEFAULT_WINDOW, eps=E.DEFAULT_EPS):
    g = np.asarray(g, dtype=np.float64)
    out = np.zeros(g.shape[0])
    for t in range(g.shape[0]):
        win = E.window(t, w)
        if len(win) > 1:
            x = g[win.start:win.stop]
            out[t] = (g[t] - x.mean()) / (x.std(ddof=1) + eps)
    return out


def _zscore_variance(g, w=E.DEFAULT_WINDOW, eps=E.DEFAULT_EPS):
    g = np.asarray(g, dtype=np.float64)
    out = np.zeros(g.shape[0])
    for t in range(g.shape[0]):
        win = E.window(t, w)
        if len(win):
            x = g[win.start:win.stop]
            out[t] = (g[t] - x.mean()) / (x.var() + eps)
    return out


def _scores_swapped(g_a, g_b, w=E.DEFAULT_WINDOW, eps=E.DEFAULT_EPS, detrend=True):
    return E.__dict__["_orig_token_scores"](g_b, g_a, w, eps, detrend)


def _deltas_l1(h):
    h = np.asarray(h, dtype=np.float64)
    g = np.zeros(h.shape[0])
    g[1:] = np.abs(np.diff(h, axis=0)).sum(axis=1)
    return g


_PINS = [test_deltas_pythagorean, test_window_positions, test_rolling_mean_ramp_closed_form,
         test_zscore_ramp_closed_form, test_zscore_exact_rationals, test_score_bands]


@pytest.mark.parametrize("name,attr,mutant", [
    ("window excludes t", "window",
     lambda t, w: range(max(1, t - w), t) if t >= 1 else range(0)),
    ("window includes position 0", "window",
     lambda t, w: range(max(0, t - w + 1), t + 1) if t >= 1 else range(0)),
    ("sample deviation", "rolling_zscore", _zscore_sample_std),
    ("variance instead of deviation", "rolling_zscore", _zscore_variance),
    ("bands swapped", "token_scores", _scores_swapped),
    ("L1 norm of the change", "hidden_deltas", _deltas_l1),
])
def test_planted_mistakes_are_caught(monkeypatch, name, attr, mutant):
    monkeypatch.setitem(E.__dict__, "_orig_token_scores", E.token_scores)
    monkeypatch.setattr(E, attr, mutant)
    caught = 0
    for pin in _PINS:
        try:
            pin()
        except (AssertionError, ValueError, ZeroDivisionError):
            caught += 1
    assert caught >= 1, f"no pin catches: {name}"
