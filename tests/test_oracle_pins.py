"""Pins for the float64 oracle (CPU only).

Each test ties the oracle to something other than itself: the hand-derived
worked example under tests/golden/, closed forms, invariants of the
definition, library routines for special cases, and a scalar brute force on
tiny shapes.  Definitions: KVzip page ("KVzip: Query-Agnostic KV Cache
Compression with Context Reconstruction") section 3.2 for the score,
section 4.1 for the budget; SelKV page section 3.1 for the floor rule.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
import oracle.kvzip as OK
from oracle.brute import brute_scores, brute_topk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split("=", 1)
            out[k.strip()] = [t.strip() for t in v.split(",")]
    return out


def _val(tok):
    if tok.startswith("ln "):
        return math.log(float(Fraction(tok[3:])))
    return float(Fraction(tok))


def _rand_head(rng, G, n_c, n_prompt, d, amp=1.0):
    n_in = n_c + n_prompt
    return (amp * rng.standard_normal((G, n_in, d)),
            amp * rng.standard_normal((n_c, d)),
            amp * rng.standard_normal((n_in, d)))


# ---------------------------------------------------------------------------
# worked example (hand-derived rationals)
# ---------------------------------------------------------------------------
def test_golden_worked_example():
    gdat = _parse_golden("worked_example.txt")
    k_ctx = np.array([[_val(t)] for t in gdat["k_ctx"]])
    k_new = np.array([[_val(t)] for t in gdat["k_new"]])
    q = np.array([[[_val(t)] for t in gdat["q_g0"]],
                  [[_val(t)] for t in gdat["q_g1"]]])
    S, lse = oracle.head_scores(q, k_ctx, k_new, 1.0)
    np.testing.assert_allclose(S, [_val(t) for t in gdat["S"]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], [_val(t) for t in gdat["lse_g0"]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[1], [_val(t) for t in gdat["lse_g1"]], rtol=0, atol=1e-14)
    r = _val(gdat["keep_ratio"][0])
    off, idx = oracle.select(S[None, None, :], r, 0)
    assert off.tolist() == [0, 1]
    assert idx.tolist() == [int(t) for t in gdat["kept"]]


def test_golden_topk_ties():
    gdat = _parse_golden("topk_ties.txt")
    s = np.array([_val(t) for t in gdat["scores"]])
    for key, val in gdat.items():
        if not key.startswith("ratio"):
            continue
        r = float(key.split()[1])
        k = oracle.keep_count(len(s), r)
        assert oracle.topk_ascending(s, k).tolist() == [int(t) for t in val], key


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("G,n_c,n_prompt,d", [(1, 1, 0, 3), (4, 7, 3, 5), (2, 33, 2, 8), (3, 300, 5, 16)])
def test_zero_queries_closed_form(G, n_c, n_prompt, d):
    rng = np.random.default_rng(1)
    q, k_ctx, k_new = _rand_head(rng, G, n_c, n_prompt, d, amp=3.0)
    q[:] = 0.0
    S, lse = oracle.head_scores(q, k_ctx, k_new, 0.37)
    n_in = n_c + n_prompt
    # every row is uniform over the n_c + i + 1 keys it sees
    np.testing.assert_allclose(lse, np.log(n_c + np.arange(n_in) + 1.0)[None, :].repeat(G, 0),
                               rtol=0, atol=1e-13)
    # the largest share a cached key gets is in row 0: 1 / (n_c + 1)
    np.testing.assert_allclose(S, np.full(n_c, 1.0 / (n_c + 1)), rtol=1e-14, atol=0)


def test_single_cached_key_sigmoid():
    # n_c = 1, n_prompt = 0: the only row sees k_ctx[0] and k_new[0], so
    # A[g, 0, 0] = logistic(scale * q_g . (k_ctx[0] - k_new[0]))
    rng = np.random.default_rng(2)
    for trial in range(20):
        G, d = 1 + trial % 4, 1 + trial % 6
        q, k_ctx, k_new = _rand_head(rng, G, 1, 0, d, amp=2.0)
        scale = float(rng.uniform(0.05, 2.0))
        S, lse = oracle.head_scores(q, k_ctx, k_new, scale)
        diff = scale * (q[:, 0, :] @ (k_ctx[0] - k_new[0]))
        assert S[0] == pytest.approx(scipy.special.expit(diff).max(), rel=1e-13, abs=1e-300)
        x0 = scale * (q[:, 0, :] @ k_ctx[0])
        x1 = scale * (q[:, 0, :] @ k_new[0])
        np.testing.assert_allclose(lse[:, 0], np.logaddexp(x0, x1), rtol=1e-14)


def test_single_visible_key_lse_is_logit():
    # with one dominating key (others pushed to -inf by a huge gap) the lse
    # equals that logit
    q = np.array([[[1.0]]])
    k_ctx = np.array([[300.0]])
    k_new = np.array([[-300.0]])
    S, lse = oracle.head_scores(q, k_ctx, k_new, 1.0)
    assert lse[0, 0] == pytest.approx(300.0, abs=1e-12)
    assert S[0] == 1.0


def test_rows_match_library_softmax():
    rng = np.random.default_rng(3)
    G, n_c, n_prompt, d = 2, 11, 4, 6
    q, k_ctx, k_new = _rand_head(rng, G, n_c, n_prompt, d, amp=1.5)
    k_all = np.concatenate([k_ctx, k_new])
    n_in = n_c + n_prompt
    scale = 0.41
    for g in range(G):
        a, lse = oracle.attention_rows(q[g], np.arange(n_in), k_all, n_c, scale)
        for i in range(n_in):
            nv = n_c + i + 1
            x = scale * (k_all[:nv] @ q[g, i])
            np.testing.assert_allclose(a[i, :nv], scipy.special.softmax(x), rtol=1e-13, atol=1e-300)
            assert np.all(a[i, nv:] == 0.0)
            assert lse[i] == pytest.approx(scipy.special.logsumexp(x), rel=1e-14)


# ---------------------------------------------------------------------------
# invariants of the definition
# ---------------------------------------------------------------------------
def test_scores_in_unit_interval_and_rows_sum_to_one():
    rng = np.random.default_rng(4)
    q, k_ctx, k_new = _rand_head(rng, 3, 64, 5, 8, amp=2.5)
    S, _ = oracle.head_scores(q, k_ctx, k_new, 0.5)
    assert np.all(S > 0) and np.all(S <= 1.0)
    a, _ = oracle.attention_rows(q[0], np.arange(69), np.concatenate([k_ctx, k_new]), 64, 0.5)
    np.testing.assert_allclose(a.sum(axis=1), 1.0, atol=1e-13)


def test_context_permutation_equivariance():
    rng = np.random.default_rng(5)
    q, k_ctx, k_new = _rand_head(rng, 2, 40, 3, 8)
    perm = rng.permutation(40)
    S, lse = oracle.head_scores(q, k_ctx, k_new, 0.35)
    S2, lse2 = oracle.head_scores(q, k_ctx[perm], k_new, 0.35)
    np.testing.assert_allclose(S2, S[perm], rtol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)


def test_key_translation_invariance():
    rng = np.random.default_rng(6)
    q, k_ctx, k_new = _rand_head(rng, 2, 30, 4, 8)
    c = rng.standard_normal(8)
    scale = 0.3
    S, lse = oracle.head_scores(q, k_ctx, k_new, scale)
    S2, lse2 = oracle.head_scores(q, k_ctx + c, k_new + c, scale)
    np.testing.assert_allclose(S2, S, rtol=1e-11)
    np.testing.assert_allclose(lse2 - lse, scale * (q @ c), atol=1e-11)


def test_query_head_duplication():
    rng = np.random.default_rng(7)
    q, k_ctx, k_new = _rand_head(rng, 2, 25, 2, 6)
    S, lse = oracle.head_scores(q, k_ctx, k_new, 0.4)
    q4 = np.concatenate([q, q[::-1]], axis=0)
    S4, lse4 = oracle.head_scores(q4, k_ctx, k_new, 0.4)
    np.testing.assert_array_equal(S4, S)
    np.testing.assert_array_equal(lse4[:2], lse)


def test_dominant_aligned_key():
    rng = np.random.default_rng(8)
    u = rng.standard_normal(16)
    u /= np.linalg.norm(u)
    q, k_ctx, k_new = _rand_head(rng, 2, 50, 3, 16, amp=0.1)
    q += u
    k_ctx[0] = 200.0 * u
    S, _ = oracle.head_scores(q, k_ctx, k_new, 0.25)
    assert S[0] > 1.0 - 1e-12
    assert np.all(S[1:] < 1e-6)


# ---------------------------------------------------------------------------
# scalar brute force on tiny shapes
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(12))
def test_brute_force_agreement(seed):
    rng = np.random.default_rng(100 + seed)
    G = 1 + seed % 3
    n_c = 1 + (seed * 5) % 8
    n_prompt = seed % 4
    d = 1 + seed % 4
    q, k_ctx, k_new = _rand_head(rng, G, n_c, n_prompt, d, amp=1.3)
    scale = float(rng.uniform(0.2, 1.5))
    S, lse = oracle.head_scores(q, k_ctx, k_new, scale)
    Sb, lseb, Ab = brute_scores(q.tolist(), k_ctx.tolist(), k_new.tolist(), scale)
    np.testing.assert_allclose(S, Sb, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(lse, lseb, rtol=1e-12, atol=1e-12)
    k_all = np.concatenate([k_ctx, k_new])
    for g in range(G):
        a, _ = oracle.attention_rows(q[g], np.arange(n_c + n_prompt), k_all, n_c, scale)
        np.testing.assert_allclose(a, np.array(Ab[g]), rtol=1e-12, atol=1e-300)


def test_parallel_driver_identical():
    rng = np.random.default_rng(9)
    q, k_ctx, k_new = _rand_head(rng, 3, 200, 8, 16)
    S, lse = oracle.head_scores(q, k_ctx, k_new, 0.25)
    S2, lse2 = oracle.head_scores_parallel(q, k_ctx, k_new, 0.25, workers=2, row_block=37)
    np.testing.assert_allclose(S2, S, rtol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-15)


def test_row_lse_single_row():
    rng = np.random.default_rng(10)
    q, k_ctx, k_new = _rand_head(rng, 2, 30, 4, 8)
    _, lse = oracle.head_scores(q, k_ctx, k_new, 0.3)
    for g, i in [(0, 0), (1, 33), (0, 17)]:
        assert oracle.row_lse(q[g, i], i, k_ctx, k_new, 0.3) == pytest.approx(lse[g, i], rel=1e-14)


# ---------------------------------------------------------------------------
# selection and compaction
# ---------------------------------------------------------------------------
def test_keep_count_rule():
    assert [oracle.keep_count(n, r) for n, r in
            [(512, 0.3), (8192, 0.3), (32768, 0.25), (131072, 0.3), (16384, 0.1),
             (8 * 16384, 0.1), (10, 1.0), (10, 0.05), (3, 0.999)]] == \
        [153, 2457, 8192, 39321, 1638, 13107, 10, 1, 2]
    for bad in (0.0, -0.1, 1.0000001, float("nan")):
        with pytest.raises(ValueError):
            oracle.keep_count(10, bad)


@pytest.mark.parametrize("seed", range(10))
def test_topk_brute_subsets(seed):
    rng = np.random.default_rng(200 + seed)
    n = 6 + seed % 7
    # few distinct levels -> many exact ties straddling the threshold
    s = rng.integers(0, 4, size=n).astype(np.float64) / 4.0
    for k in range(1, n + 1):
        assert oracle.topk_ascending(s, k).tolist() == brute_topk(list(s), k)


def test_topk_identity_and_argmax():
    rng = np.random.default_rng(11)
    s = rng.random((2, 3, 50))
    off, idx = oracle.select(s, 1.0, 0)
    assert off.tolist() == [50 * t for t in range(7)]
    assert idx.tolist() == list(range(50)) * 6
    s[0, 0, 7] = s[0, 0, 9] = 2.0
    off, idx = oracle.select(s, 0.01, 0)           # 0.5 keys -> 1
    assert idx[0] == 7
    off, idx = oracle.select(s, 1.0, 1)
    assert idx.tolist() == list(range(50)) * 6


@pytest.mark.parametrize("seed", range(6))
def test_layer_budget_brute(seed):
    rng = np.random.default_rng(300 + seed)
    L, H, n_c = 2, 3, 4
    s = rng.integers(0, 3, size=(L, H, n_c)).astype(np.float64)
    r = [0.25, 0.34, 0.5, 0.67, 0.1, 0.9][seed]
    off, idx = oracle.select(s, r, 1)
    kl = oracle.keep_count(H * n_c, r)
    for l in range(L):
        flat = brute_topk(list(s[l].reshape(-1)), kl)
        got = []
        for h in range(H):
            lh = l * H + h
            got += [h * n_c + j for j in idx[off[lh]:off[lh + 1]]]
        assert got == flat
    assert off[-1] == L * kl


@pytest.mark.parametrize("seed", range(6))
def test_model_budget_brute(seed):
    # mode 2: one budget over every head of every layer (KVzip section 4.1)
    rng = np.random.default_rng(400 + seed)
    L, H, n_c = 2, 2, 4
    s = rng.integers(0, 3, size=(L, H, n_c)).astype(np.float64) / 2.0
    r = [0.25, 0.34, 0.5, 0.67, 0.1, 0.9][seed]
    off, idx = oracle.select(s, r, 2)
    k = oracle.keep_count(L * H * n_c, r)
    want = brute_topk(list(s.reshape(-1)), k)
    got = []
    for lh in range(L * H):
        got += [lh * n_c + j for j in idx[off[lh]:off[lh + 1]]]
    assert got == want
    assert off[-1] == k and off[0] == 0


def test_model_budget_reduces_to_other_modes():
    rng = np.random.default_rng(13)
    s = rng.random((1, 3, 40))
    for r in (0.05, 0.3, 0.77, 1.0):
        a, b = oracle.select(s, r, 2), oracle.select(s, r, 1)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    s = rng.random((1, 1, 40))
    for r in (0.05, 0.3, 1.0):
        a, b = oracle.select(s, r, 2), oracle.select(s, r, 0)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # a head whose scores all exceed another's takes its whole share first
    s = np.stack([rng.random(30) + 2.0, rng.random(30)])[None]
    off, idx = oracle.select(s, 0.5, 2)
    assert off.tolist() == [0, 30, 30] and idx.tolist() == list(range(30))


def test_head_level_scores():
    # KVzip section 4.2: the head score is the max along the sequence
    with pytest.raises(ValueError):
        oracle.head_level_scores(np.zeros((2, 2, 0)))
    # zero queries: every row is uniform, row 0 sees n_c + 1 keys, so the
    # head score is 1 / (n_c + 1)
    for n_c, n_p in [(1, 0), (5, 3), (17, 2)]:
        q = np.zeros((2, n_p + n_c, 4))
        S, _ = oracle.head_scores(q, np.ones((n_c, 4)), np.ones((n_p + n_c, 4)), 0.5)
        hs = oracle.head_level_scores(S[None, None])
        assert hs.shape == (1, 1) and abs(hs[0, 0] - 1.0 / (n_c + 1)) < 1e-15
    # brute force: the largest attention weight any cached key gets anywhere
    rng = np.random.default_rng(14)
    for _ in range(5):
        G, n_c, n_p, d = 2, 5, 2, 3
        q = rng.normal(size=(G, n_p + n_c, d))
        kc, kn = rng.normal(size=(n_c, d)), rng.normal(size=(n_p + n_c, d))
        _, _, A = brute_scores(q.tolist(), kc.tolist(), kn.tolist(), 0.7)
        want = max(A[g][i][j] for g in range(G) for i in range(n_p + n_c)
                   for j in range(n_c))
        S, _ = oracle.head_scores(q, kc, kn, 0.7)
        assert abs(oracle.head_level_scores(S[None, None])[0, 0] - want) < 1e-13


def test_compact_rows_are_kept_rows():
    rng = np.random.default_rng(12)
    L, H, n_c, d = 2, 2, 20, 4
    k = rng.integers(0, 2 ** 16, size=(L, H, n_c, d), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(L, H, n_c, d), dtype=np.uint16)
    s = rng.random((L, H, n_c))
    for mode in (0, 1, 2):
        off, idx = oracle.select(s, 0.35, mode)
        ko, vo = oracle.compact(k, v, off, idx)
        assert ko.shape == (off[-1], d)
        for lh in range(L * H):
            l, h = divmod(lh, H)
            for t in range(off[lh], off[lh + 1]):
                assert np.array_equal(ko[t], k[l, h, idx[t]])
                assert np.array_equal(vo[t], v[l, h, idx[t]])
    off, idx = oracle.select(s, 1.0, 0)
    ko, vo = oracle.compact(k, v, off, idx)
    assert np.array_equal(ko, k.reshape(-1, d)) and np.array_equal(vo, v.reshape(-1, d))


def test_bf16_conversion_exact():
    bits = np.array([0x3F80, 0xBFC0, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], dtype=np.uint16)
    want = [1.0, -1.5, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41, 3.140625]
    got = oracle.bf16_to_f64(bits)
    assert got.tolist() == want


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by a pin above
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("mutant", [
    lambda n_c, i: n_c + i,        # diagonal key dropped
    lambda n_c, i: n_c + i + 2,    # one future key leaked
    lambda n_c, i: n_c,            # normalised over cached keys only
])
def test_planted_mask_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(OK, "visible_keys", mutant)
    caught = 0
    try:
        test_zero_queries_closed_form(2, 7, 3, 5)
    except (AssertionError, ValueError, IndexError):
        caught += 1
    try:
        test_golden_worked_example()
    except (AssertionError, ValueError, IndexError):
        caught += 1
    assert caught == 2


# ---------------------------------------------------------------------------
# chunked scoring (KVzip page, section 3.4)
# ---------------------------------------------------------------------------
def _pack_chunks(rng, G, n_c, n_prompt, d, chunk, amp=1.0):
    k_ctx = amp * rng.standard_normal((n_c, d))
    qs, kns = [], []
    for _, m in OK.chunk_bounds(n_c, chunk):
        qs.append(amp * rng.standard_normal((G * (n_prompt + m), d)))
        kns.append(amp * rng.standard_normal((n_prompt + m, d)))
    return np.concatenate(qs), k_ctx, np.concatenate(kns)


def test_chunk_bounds():
    assert OK.chunk_bounds(10, 4) == [(0, 4), (4, 4), (8, 2)]
    assert OK.chunk_bounds(8, 4) == [(0, 4), (4, 4)]
    assert OK.chunk_bounds(3, 10) == [(0, 3)]
    assert OK.chunk_bounds(5, 1) == [(j, 1) for j in range(5)]


def test_chunked_whole_context_is_unchunked():
    rng = np.random.default_rng(20)
    G, n_c, n_p, d = 3, 40, 4, 8
    q, kc, kn = _rand_head(rng, G, n_c, n_p, d)
    S, lse = oracle.head_scores(q, kc, kn, 0.3)
    for chunk in (n_c, n_c + 1, 10 ** 6):
        S2, l2 = oracle.chunked_head_scores(q.reshape(-1, d), kc, kn, 0.3, n_p, chunk, G)
        np.testing.assert_array_equal(S2, S)
        np.testing.assert_array_equal(l2, lse.reshape(-1))


def test_chunked_zero_queries_closed_form():
    rng = np.random.default_rng(21)
    G, n_c, n_p, d, chunk = 2, 23, 3, 5, 7
    q, kc, kn = _pack_chunks(rng, G, n_c, n_p, d, chunk, amp=2.0)
    q[:] = 0.0
    S, lse = oracle.chunked_head_scores(q, kc, kn, 0.5, n_p, chunk, G)
    off = 0
    for start, m in OK.chunk_bounds(n_c, chunk):
        # each chunk is its own uniform attention over m + i + 1 keys
        np.testing.assert_allclose(S[start:start + m], 1.0 / (m + 1), rtol=1e-14)
        want = np.tile(np.log(m + np.arange(n_p + m) + 1.0), G)
        np.testing.assert_allclose(lse[off:off + G * (n_p + m)], want, atol=1e-13)
        off += G * (n_p + m)


def test_chunked_single_key_chunks_are_logistic():
    # chunk = 1, n_prompt = 0: chunk j holds cached key j and one new key,
    # so S_j = max_g logistic(scale * q_gj . (k_ctx[j] - k_new[j]))
    rng = np.random.default_rng(22)
    G, n_c, d, scale = 3, 9, 4, 0.7
    q, kc, kn = _pack_chunks(rng, G, n_c, 0, d, 1, amp=1.5)
    S, _ = oracle.chunked_head_scores(q, kc, kn, scale, 0, 1, G)
    for j in range(n_c):
        qj = q[G * j:G * (j + 1)]
        want = scipy.special.expit(scale * qj @ (kc[j] - kn[j])).max()
        assert S[j] == pytest.approx(want, rel=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_chunked_brute_force(seed):
    rng = np.random.default_rng(400 + seed)
    G, n_c, n_p, d = 1 + seed % 3, 5 + seed, seed % 3, 1 + seed % 3
    chunk = 1 + seed % 4
    q, kc, kn = _pack_chunks(rng, G, n_c, n_p, d, chunk)
    S, lse = oracle.chunked_head_scores(q, kc, kn, 0.6, n_p, chunk, G)
    qo = ko = 0
    for start, m in OK.chunk_bounds(n_c, chunk):
        n_in = n_p + m
        qc = q[qo:qo + G * n_in].reshape(G, n_in, d)
        Sb, lb, _ = brute_scores(qc.tolist(), kc[start:start + m].tolist(),
                                 kn[ko:ko + n_in].tolist(), 0.6)
        np.testing.assert_allclose(S[start:start + m], Sb, rtol=1e-12)
        np.testing.assert_allclose(lse[qo:qo + G * n_in], np.ravel(lb), rtol=1e-12, atol=1e-12)
        qo += G * n_in
        ko += n_in


def test_select_signed_zero_equals_zero():
    """-0.0 and +0.0 are the same score: with zeros at the cut, the kept
    zeros are the lowest positions, whatever their sign bits (KVzip section
    4.1 ranks by score value; ties go to the lower index)."""
    s = np.array([[[0.5, -0.0, 0.0, -0.0, 0.25, 0.0]]], dtype=np.float32)
    # keep 4 of 6: 0.5, 0.25, then the two lowest-position zeros (1 and 2)
    off, idx = oracle.select(s, 4 / 6 + 1e-9, 0)
    assert off.tolist() == [0, 4] and idx.tolist() == [0, 1, 2, 4]
    assert oracle.epikv.select_tokens(s.reshape(-1), 4).tolist() == [0, 1, 2, 4]
    s2 = np.abs(s)
    assert np.array_equal(oracle.select(s2, 4 / 6 + 1e-9, 0)[1], idx)

