"""Seeded input generator: determinism, rounding, structure and shapes (CPU)."""
import numpy as np
import pytest

import synth
from synth import configs as C


def test_bf16_round_to_nearest_even_edges():
    one = 1.0
    vals = np.array([
        one,                          # exact
        one + 2.0 ** -8,              # halfway 1 .. 1+2^-7 -> even (1)
        one + 3 * 2.0 ** -8,          # halfway 1+2^-7 .. 1+2^-6 -> even (1+2^-6)
        one + 2.0 ** -8 + 2.0 ** -20,  # above halfway -> up
        -1.5,
        one + 2.0 ** -8 + 2.0 ** -30,  # float32 step drops 2^-30, then tie -> even
        65504.0,
    ])
    got = synth.f64_to_bf16_bits(vals).tolist()
    assert got == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xBFC0, 0x3F80, 0x477F + 1]
    back = synth.bf16_bits_to_f32(np.array(got, dtype=np.uint16))
    assert back[0] == 1.0 and back[4] == -1.5


def test_head_determinism_and_independence():
    w = synth.TINY
    a = synth.generate_head(w, 0, 0)
    b = synth.generate_head(w, 0, 0)
    for k in a:
        assert np.array_equal(a[k], b[k])
    # one part alone equals the same part of the full draw
    only_k = synth.generate_head(w, 0, 0, ("k_ctx",))
    assert np.array_equal(only_k["k_ctx"], a["k_ctx"])
    w2 = synth.LLAMA8B_8K.shrink(n_c=64, n_prompt=4, L=2, H=2)
    h00 = synth.generate_head(w2, 0, 0, ("q",))["q"]
    h01 = synth.generate_head(w2, 0, 1, ("q",))["q"]
    assert not np.array_equal(h00, h01)


def test_shapes_match_workloads():
    for w in synth.ALL:
        s = w.shrink(n_c=min(w.n_c, 300), L=1, H=1)
        d = synth.generate_head(s, 0, 0)
        assert d["q"].shape == (s.G, s.n_in, s.d)
        assert d["k_ctx"].shape == (s.n_c, s.d)
        assert d["k_new"].shape == (s.n_in, s.d)
        assert d["v_ctx"].shape == (s.n_c, s.d)
        assert all(v.dtype == np.uint16 for v in d.values())
    assert synth.LLAMA8B_8K.scale == np.float32(1.0 / np.sqrt(128.0))


def test_sinks_present():
    w = synth.LLAMA8B_8K.shrink(n_c=256)
    k = synth.bf16_bits_to_f32(synth.generate_head(w, 0, 0, ("k_ctx",))["k_ctx"])
    norms = np.linalg.norm(k, axis=1)
    assert norms[:4].min() > 3.0 * np.median(norms[4:])


def test_span_repeat_exact_copies():
    w = synth.LLAMA8B_128K.shrink(n_c=3 * C.SPAN_PERIOD + 200)
    d = synth.generate_head(w, 0, 0, ("k_ctx", "v_ctx"))
    for part in ("k_ctx", "v_ctx"):
        x = d[part]
        for k in (1, 2, 3):
            a = C.SPAN_PERIOD * k + C.SPAN_SRC
            assert np.array_equal(x[a:a + C.SPAN_LEN], x[C.SPAN_SRC:C.SPAN_SRC + C.SPAN_LEN])
        # sinks are not copied
        assert not np.array_equal(x[C.SPAN_PERIOD:C.SPAN_PERIOD + 4], x[:4])


def test_near_duplicates_present():
    w = synth.QWEN14B_32K.shrink(n_c=2000)
    k = synth.bf16_bits_to_f32(synth.generate_head(w, 0, 0, ("k_ctx",))["k_ctx"]).astype(np.float64)
    # nearest earlier neighbour distance: copied rows sit within the noise of
    # their source (unless the source row was itself overwritten later)
    close = 0
    for p in range(5, 2000):
        dist = np.linalg.norm(k[4:p] - k[p], axis=1).min()
        close += dist < 0.5
    n_copy = int(0.1 * 2000)
    assert 0.8 * n_copy <= close <= n_copy


def test_student_t_heavy_tails():
    w = synth.GEMMA12B_16K.shrink(n_c=4000)
    k = synth.bf16_bits_to_f32(synth.generate_head(w, 0, 0, ("k_ctx",))["k_ctx"])
    norms = np.linalg.norm(k, axis=1)
    # |t_3| has a heavy tail: the top norm is far above the median
    assert norms.max() > 8.0 * np.median(norms)


def test_generate_workload_matches_heads():
    w = synth.LLAMA8B_8K.shrink(n_c=40, n_prompt=3, L=2, H=2)
    full = synth.generate_workload(w, workers=2)
    for l in range(2):
        for h in range(2):
            d = synth.generate_head(w, l, h)
            for k in d:
                assert np.array_equal(full[k][l, h], d[k])


def test_nearest_position_routes():
    off = np.array([0, 2, 3])
    idx = np.array([1, 5, 3])
    so, si = synth.nearest_position_routes(off, idx, 8)
    assert so.tolist() == [0, 3, 6, 13]
    assert si.tolist() == [0, 2, 3, 4, 6, 7, 0, 1, 2, 4, 5, 6, 7]
    # every evicted position routed exactly once, to its nearest kept one
    rng = np.random.default_rng(0)
    n_c = 500
    kept = [np.sort(rng.choice(n_c, size=s, replace=False)) for s in (1, 50, 499)]
    off = np.concatenate([[0], np.cumsum([k.size for k in kept])])
    idx = np.concatenate(kept)
    so, si = synth.nearest_position_routes(off, idx, n_c)
    for h, k in enumerate(kept):
        rows = range(off[h], off[h + 1])
        got = np.concatenate([si[so[t]:so[t + 1]] for t in rows])
        assert sorted(got.tolist()) == sorted(set(range(n_c)) - set(k.tolist()))
        for t in rows:
            for j in si[so[t]:so[t + 1]]:
                assert abs(j - idx[t]) == np.abs(k - j).min()


def test_extreme_profiles_seeded_and_shaped():
    """The extreme-logit inputs are reproducible per (l, h) and their cached-key
    norms follow the requested profile."""
    for prof in synth.EXTREME_PROFILES:
        a = synth.generate_extreme_workload(prof, 1, 2, 2, 64, 300, 5)
        b = synth.generate_extreme_workload(prof, 1, 2, 2, 64, 300, 5)
        for k in a:
            assert np.array_equal(a[k], b[k])
        assert not np.array_equal(a["k_ctx"][0, 0], a["k_ctx"][0, 1])
        norms = np.linalg.norm(synth.bf16_bits_to_f32(a["k_ctx"][0, 0]).astype(np.float64), axis=1)
        if prof == "rising":
            assert norms[-30:].mean() > 10 * norms[:30].mean()
        elif prof == "falling":
            assert norms[:30].mean() > 10 * norms[-30:].mean()
        else:
            assert np.sum(norms > 20 * np.median(norms)) >= 1
