"""Pins of the SelKV gate oracle (SelKV page, section 1: g = max(cos, 0))
and of the gated merge read from it."""
import math

import numpy as np
import pytest
import scipy.spatial.distance as ssd

from oracle import selkv as S


def test_gate_closed_forms():
    u = np.array([1.0, 2.0, -2.0])
    assert S.soft_cosine_gate(u, 3.5 * u) == pytest.approx(1.0, abs=1e-15)
    assert S.soft_cosine_gate(u, -u) == 0.0
    assert S.soft_cosine_gate(np.array([1.0, 0.0]), np.array([0.0, 5.0])) == 0.0
    assert S.soft_cosine_gate(np.array([1.0, 0.0]), np.array([1.0, 1.0])) == \
        pytest.approx(1 / math.sqrt(2), abs=1e-15)
    assert S.soft_cosine_gate(np.array([1.0, 0.0]), np.array([-1.0, 1.0])) == 0.0
    assert S.soft_cosine_gate(np.zeros(3), u) == 0.0
    assert S.soft_cosine_gate(u, np.zeros(3)) == 0.0


def test_gate_matches_scipy_cosine():
    rng = np.random.default_rng(0)
    for _ in range(50):
        a, b = rng.normal(size=16), rng.normal(size=16)
        want = max(1.0 - ssd.cosine(a, b), 0.0)
        assert abs(S.soft_cosine_gate(a, b) - want) < 1e-12
        assert abs(S.soft_cosine_gate(a, b) - S.soft_cosine_gate(b, a)) < 1e-15
        assert abs(S.soft_cosine_gate(2.5 * a, 0.1 * b) - S.soft_cosine_gate(a, b)) < 1e-12


def _one_head(K, V, kept, routes):
    """Single (l, h) with kept positions and per-kept-row routed lists."""
    offsets = np.array([0, len(kept)])
    src_off = np.concatenate([[0], np.cumsum([len(r) for r in routes])])
    src_idx = np.array([j for r in routes for j in r], dtype=np.int64)
    return S.merge_compact(K[None, None], V[None, None], offsets, np.array(kept),
                           src_off, src_idx)


def test_merge_drop_and_uniform_mean():
    rng = np.random.default_rng(1)
    d = 4
    K, V = rng.normal(size=(6, d)), rng.normal(size=(6, d))
    # no routes: plain compaction
    ko, vo, g, m = _one_head(K, V, [1, 4], [[], []])
    assert np.array_equal(ko, K[[1, 4]]) and np.array_equal(vo, V[[1, 4]])
    assert m.tolist() == [0.0, 0.0] and g.size == 0
    # routed values opposite to the target: gate 0, dropped
    V2 = V.copy()
    V2[0] = -2.0 * V2[1]
    ko, vo, g, m = _one_head(K, V2, [1, 4], [[0], []])
    assert g.tolist() == [0.0] and np.array_equal(ko[0], K[1]) and np.array_equal(vo[0], V2[1])
    # routed values parallel to the target: gate 1, uniform mean of the group
    V3 = V.copy()
    V3[0], V3[2] = 0.5 * V3[1], 3.0 * V3[1]
    ko, vo, g, m = _one_head(K, V3, [1, 4], [[0, 2], []])
    assert np.allclose(g, 1.0, atol=1e-15) and m[0] == pytest.approx(2.0)
    assert np.allclose(ko[0], (K[1] + K[0] + K[2]) / 3, atol=1e-14)
    assert np.allclose(vo[0], V3[1] * (1 + 0.5 + 3.0) / 3, atol=1e-14)


def test_merge_partial_weight_closed_form():
    # target value (1, 0), routed value (1, 1): g = 1/sqrt(2)
    K = np.array([[2.0, 0.0], [0.0, 4.0]])
    V = np.array([[1.0, 0.0], [1.0, 1.0]])
    ko, vo, g, m = _one_head(K, V, [0], [[1]])
    gg = 1 / math.sqrt(2)
    assert g[0] == pytest.approx(gg, abs=1e-15) and m[0] == pytest.approx(gg, abs=1e-15)
    assert np.allclose(ko[0], (K[0] + gg * K[1]) / (1 + gg), atol=1e-15)
    assert np.allclose(vo[0], (V[0] + gg * V[1]) / (1 + gg), atol=1e-15)


def test_merge_invalid_source_ignored_and_heads_separate():
    rng = np.random.default_rng(2)
    L, H, n, d = 1, 2, 5, 3
    K, V = rng.normal(size=(L, H, n, d)), rng.normal(size=(L, H, n, d))
    offsets = np.array([0, 1, 2])
    idx = np.array([0, 0])
    src_off = np.array([0, 2, 3])
    src_idx = np.array([-1, 7, 3])     # two invalid for head 0, one valid for head 1
    ko, vo, g, m = S.merge_compact(K, V, offsets, idx, src_off, src_idx)
    assert np.array_equal(ko[0], K[0, 0, 0]) and g[0] == 0.0 and g[1] == 0.0
    gg = S.soft_cosine_gate(V[0, 1, 3], V[0, 1, 0])
    assert g[2] == gg
    assert np.allclose(vo[1], (V[0, 1, 0] + gg * V[0, 1, 3]) / (1 + gg), atol=1e-15)


# ---- planted mistakes: each must be caught by a pin above -----------------
def _cos(a, b):
    a, b = np.asarray(a, float), np.asarray(b, float)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    return 0.0 if na == 0 or nb == 0 else float(a @ b / (na * nb))


_PINS = [test_gate_closed_forms, test_gate_matches_scipy_cosine,
         test_merge_drop_and_uniform_mean, test_merge_partial_weight_closed_form]


def _merge_unnormalised(k_ctx, v_ctx, offsets, idx, src_offsets, src_idx):
    ko, vo, g, m = S.__dict__["_orig_merge"](k_ctx, v_ctx, offsets, idx, src_offsets, src_idx)
    return ko * (1.0 + m[:, None]), vo * (1.0 + m[:, None]), g, m


def _merge_count_weighted(k_ctx, v_ctx, offsets, idx, src_offsets, src_idx):
    ko, vo, g, m = S.__dict__["_orig_merge"](k_ctx, v_ctx, offsets, idx, src_offsets, src_idx)
    cnt = np.diff(src_offsets).astype(float)
    f = (1.0 + m) / (1.0 + cnt)
    return ko * f[:, None], vo * f[:, None], g, m


@pytest.mark.filterwarnings("ignore::RuntimeWarning")   # mutants may divide by zero
@pytest.mark.parametrize("name,attr,mutant", [
    ("no clamp at 0", "soft_cosine_gate", lambda a, b: _cos(a, b)),
    ("absolute cosine", "soft_cosine_gate", lambda a, b: abs(_cos(a, b))),
    ("merge not normalised", "merge_compact", _merge_unnormalised),
    ("normalised by count", "merge_compact", _merge_count_weighted),
])
def test_planted_mistakes_are_caught(monkeypatch, name, attr, mutant):
    monkeypatch.setitem(S.__dict__, "_orig_merge", S.merge_compact)
    monkeypatch.setattr(S, attr, mutant)
    caught = 0
    for pin in _PINS:
        try:
            pin()
        except (AssertionError, ValueError, ZeroDivisionError):
            caught += 1
    assert caught >= 1, f"no pin catches: {name}"
