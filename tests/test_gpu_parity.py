"""GPU parity: libkvq (through its C ABI) against the float64 oracle.

Scores and lse within the tolerances of parity_util; top-k on oracle scores
and compaction bit-exact; top-k on GPU scores exact outside the near-tie band.
Definitions: KVzip page ("KVzip: Query-Agnostic KV Cache Compression with
Context Reconstruction"), section 3.2 (score), section 4.1 (budget).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import query_agnostic_eviction_amd as kvq
from parity_util import (check_lse, check_scores, check_topk_band, check_valid_topk,
                         dev_bf16_bits, flat_kept, head_kept, oracle_head, to_dev_bf16)

pytestmark = pytest.mark.gpu

WORKERS = min(16, synth.default_workers())


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    kvq.api._lib.load()
    yield
    torch.cuda.synchronize()


def _upload(gen):
    return {k: to_dev_bf16(v) for k, v in gen.items()}


def _run(w, dev, mode=0):
    lse = kvq.kvscore_lse(dev["q"], dev["k_ctx"], dev["k_new"], scale=float(w.scale))
    sc = kvq.kvscore_colmax(dev["q"], dev["k_ctx"], lse, scale=float(w.scale))
    off, idx = kvq.kv_topk_select(sc, w.keep_ratio, mode)
    ko, vo = kvq.kv_compact(dev["k_ctx"], dev["v_ctx"], off, idx)
    torch.cuda.synchronize()
    return dict(lse=lse, scores=sc, offsets=off, idx=idx, k_out=ko, v_out=vo)


def _full_check(w, gen, out, heads=None, mode=0):
    """Oracle on every head listed (default: all) of a fully generated input."""
    L, H = w.L, w.H
    heads = heads or [(l, h) for l in range(L) for h in range(H)]
    lse_g = out["lse"].cpu().numpy()
    sc_g = out["scores"].cpu().numpy()
    S_ref = np.zeros((L, H, w.n_c))
    for (l, h) in heads:
        hg = {k: gen[k][l, h] for k in ("q", "k_ctx", "k_new")}
        S, lse = oracle_head(hg, float(w.scale), workers=WORKERS if w.n_c > 2000 else 1)
        check_lse(lse_g[l, h], lse, f"lse[{l},{h}]")
        check_scores(sc_g[l, h], S, f"scores[{l},{h}]")
        S_ref[l, h] = S
    return S_ref


def _select_checks(w, gen, out, S_ref, heads, mode):
    off = out["offsets"].cpu().numpy()
    idx = out["idx"].cpu().numpy()
    if mode == 0:
        k = oracle.keep_count(w.n_c, w.keep_ratio)
        assert np.array_equal(off, np.arange(w.L * w.H + 1) * k)
        for (l, h) in heads:
            check_topk_band(head_kept(off, idx, l * w.H + h), S_ref[l, h], k)
    # top-k of the oracle's own scores (rounded to fp32) must be bit-exact
    s32 = torch.from_numpy(S_ref.astype(np.float32)).cuda()
    o2, i2 = kvq.kv_topk_select(s32, w.keep_ratio, mode)
    ro, ri = oracle.select(S_ref.astype(np.float32), w.keep_ratio, mode)
    assert np.array_equal(o2.cpu().numpy(), ro)
    assert np.array_equal(i2.cpu().numpy(), ri)
    # compaction of the oracle's kept set must be bit-exact
    ko, vo = kvq.kv_compact(to_dev_bf16(gen["k_ctx"]), to_dev_bf16(gen["v_ctx"]),
                            torch.from_numpy(ro).cuda(), torch.from_numpy(ri).cuda())
    rko, rvo = oracle.compact(gen["k_ctx"], gen["v_ctx"], ro, ri)
    assert np.array_equal(dev_bf16_bits(ko), rko)
    assert np.array_equal(dev_bf16_bits(vo), rvo)


# ---------------------------------------------------------------------------
def test_tiny_end_to_end():
    w = synth.TINY
    _say("case: tiny", w)
    gen = synth.generate_workload(w, workers=1)
    out = _run(w, _upload(gen))
    S_ref = _full_check(w, gen, out)
    _select_checks(w, gen, out, S_ref, [(0, 0)], 0)
    # compacted rows are the kept rows of the input
    idx = out["idx"].cpu().numpy()
    assert np.array_equal(dev_bf16_bits(out["k_out"]), gen["k_ctx"][0, 0][idx])
    assert np.array_equal(dev_bf16_bits(out["v_out"]), gen["v_ctx"][0, 0][idx])


RAGGED = [
    # (base, G, d, n_c, n_prompt, L, H)
    ("llama3.1-8b-8k", 1, 64, 1, 0, 1, 1),
    ("llama3.1-8b-8k", 1, 64, 1000, 3, 1, 2),
    ("gemma3-12b-16k", 2, 256, 300, 32, 2, 1),
    ("llama3.1-8b-8k", 3, 128, 777, 5, 1, 1),
    ("qwen2.5-14b-32k", 5, 128, 200, 32, 1, 2),
    ("llama3.1-8b-8k", 8, 64, 129, 7, 1, 1),
    ("llama3.1-8b-8k", 4, 128, 64, 0, 1, 1),
    ("gemma3-12b-16k", 7, 256, 45, 1, 1, 1),
    ("llama3.1-8b-128k", 4, 128, 4300, 32, 1, 1),
    ("tiny", 6, 64, 2049, 17, 1, 1),
]


@pytest.mark.parametrize("case", RAGGED, ids=[f"G{c[1]}-d{c[2]}-nc{c[3]}-np{c[4]}" for c in RAGGED])
def test_ragged_shapes(case):
    base, G, d, n_c, n_p, L, H = case
    w = synth.BY_NAME[base].shrink(G=G, d=d, n_c=n_c, n_prompt=n_p, L=L, H=H,
                                   rank=min(synth.BY_NAME[base].rank, d))
    _say("case:", case)
    gen = synth.generate_workload(w, workers=1)
    for mode in (0, 1, 2):
        out = _run(w, _upload(gen), mode)
        S_ref = _full_check(w, gen, out)
        _select_checks(w, gen, out, S_ref, [(l, h) for l in range(L) for h in range(H)], mode)


def _tile_boundary_cases():
    """G = 1 shapes whose row count G * n_in and key count sit on either side
    of one and two 32 KB tiles (16384 / d rows or keys): pass 2's last row
    tile is shifted back to end at the last row (rows seen twice), or clamped
    when all rows fit in one tile; pass 1's key tiles end ragged or exact."""
    out = []
    for d in (64, 128, 256):
        qt = 16384 // d
        for rows in (qt - 1, qt, qt + 1, 2 * qt - 1, 2 * qt + 1):
            out.append((d, rows - 3, 3))       # n_in = rows, n_c = rows - 3
    return out


@pytest.mark.parametrize("case", _tile_boundary_cases(),
                         ids=[f"d{c[0]}-nc{c[1]}" for c in _tile_boundary_cases()])
def test_tile_boundaries(case):
    d, n_c, n_p = case
    w = synth.LLAMA8B_8K.shrink(G=1, d=d, n_c=n_c, n_prompt=n_p, L=1, H=2,
                                rank=min(synth.LLAMA8B_8K.rank, d))
    _say("case: tile boundary", case)
    gen = synth.generate_workload(w, workers=1)
    out = _run(w, _upload(gen), 0)
    S_ref = _full_check(w, gen, out)
    _select_checks(w, gen, out, S_ref, [(0, 0), (0, 1)], 0)


EXTREME = [
    # (G, d, n_c, n_prompt, H)
    (2, 64, 300, 5, 2),
    (4, 128, 1000, 32, 1),
    (2, 256, 500, 8, 1),
]


@pytest.mark.parametrize("profile", synth.EXTREME_PROFILES)
@pytest.mark.parametrize("case", EXTREME, ids=[f"G{c[0]}-d{c[1]}-nc{c[2]}" for c in EXTREME])
def test_extreme_logit_ranges(case, profile):
    """Cached-key norms rising or falling 150-fold along the context, or a few
    keys 40-120x above the rest: logits span hundreds of natural-log units, so
    pass 1 raises its running max many times mid-sweep (rising, spikes) or
    sums mostly underflowing terms (falling), and pass 2 subtracts lse values
    near 750 from logits of the same size."""
    G, d, n_c, n_p, H = case
    _say("case: extreme", profile, case)
    w = synth.LLAMA8B_8K.shrink(G=G, d=d, n_c=n_c, n_prompt=n_p, L=1, H=H, rank=8)
    gen = synth.generate_extreme_workload(profile, 1, H, G, d, n_c, n_p)
    out = _run(w, _upload(gen))
    assert np.all(np.isfinite(out["lse"].cpu().numpy()))
    sc = out["scores"].cpu().numpy()
    assert np.all((sc >= 0) & (sc <= 1))
    S_ref = _full_check(w, gen, out)
    _select_checks(w, gen, out, S_ref, [(0, h) for h in range(H)], 0)


def test_zero_queries_closed_form():
    w = synth.LLAMA8B_8K.shrink(n_c=1500, n_prompt=9, L=1, H=2)
    gen = synth.generate_workload(w, workers=1)
    gen["q"][:] = 0
    out = _run(w, _upload(gen))
    n_in = w.n_in
    lse = out["lse"].cpu().numpy()
    want = np.log(w.n_c + np.arange(n_in) + 1.0)
    for l in range(w.L):
        for h in range(w.H):
            for g in range(w.G):
                check_lse(lse[l, h, g], want)
    check_scores(out["scores"].cpu().numpy(), np.full((1, 2, w.n_c), 1.0 / (w.n_c + 1)))


def test_keep_all_is_identity():
    w = synth.TINY.shrink(keep_ratio=1.0, L=2, H=2, n_c=300)
    gen = synth.generate_workload(w, workers=1)
    for mode in (0, 1, 2):
        out = _run(w, _upload(gen), mode)
        assert np.array_equal(out["idx"].cpu().numpy(), np.tile(np.arange(300), 4))
        assert np.array_equal(out["offsets"].cpu().numpy(), np.arange(5) * 300)
        assert np.array_equal(dev_bf16_bits(out["k_out"]), gen["k_ctx"].reshape(-1, w.d))
        assert np.array_equal(dev_bf16_bits(out["v_out"]), gen["v_ctx"].reshape(-1, w.d))


# the last four sit at the LDS-staging limit of 32,768 scores per segment:
# mode 0 segments of 32,768 and 32,769, mode 1 segments (H * n_c) likewise
@pytest.mark.parametrize("n_c,L,H", [(5000, 2, 3), (20000, 1, 2), (8193, 2, 1), (1, 3, 2), (7, 1, 4),
                                     (32768, 1, 2), (32769, 1, 1), (8192, 2, 4), (10923, 1, 3)])
def test_select_ties_bit_exact(n_c, L, H):
    rng = np.random.default_rng(n_c + L + H)
    # few distinct values: long runs of exact ties across chunk boundaries
    s = (rng.integers(0, 6, size=(L, H, n_c)).astype(np.float32) / 8.0)
    s[0, 0, :min(n_c, 3)] = 0.0
    dev = torch.from_numpy(s).cuda()
    for mode in (0, 1, 2):
        for r in (0.01, 0.1, 0.3, 0.5, 0.77, 1.0):
            o, i = kvq.kv_topk_select(dev, r, mode)
            ro, ri = oracle.select(s, r, mode)
            assert np.array_equal(o.cpu().numpy(), ro), (mode, r)
            assert np.array_equal(i.cpu().numpy(), ri), (mode, r)


@pytest.mark.parametrize("n_c,L,H", [(5000, 2, 3), (8193, 1, 2), (9, 2, 2)])
def test_select_signed_zero_ties_with_zero(n_c, L, H):
    """A -0.0 score equals +0.0: it ties with the zeros by position instead of
    ranking above every positive score (its sign bit would otherwise put it
    first in the bit-pattern order)."""
    rng = np.random.default_rng(31 + n_c)
    s = (rng.integers(0, 4, size=(L, H, n_c)).astype(np.float32) / 4.0)
    zeros = s == 0.0
    flip = zeros & (rng.random(s.shape) < 0.5)
    s[flip] = -0.0
    assert np.signbit(s).any() and (s == 0).sum() > np.signbit(s).sum()
    dev = torch.from_numpy(s).cuda()
    for mode in (0, 1, 2):
        for r in (0.1, 0.6, 0.9, 1.0):
            o, i = kvq.kv_topk_select(dev, r, mode)
            ro, ri = oracle.select(s, r, mode)
            assert np.array_equal(o.cpu().numpy(), ro), (mode, r)
            assert np.array_equal(i.cpu().numpy(), ri), (mode, r)
    # the signed token select folds -0.0 the same way
    flat = torch.from_numpy(s.reshape(-1)).cuda()
    k = max(1, s.size * 3 // 4)
    got = kvq.kv_select_tokens(flat, k).cpu().numpy()
    want = oracle.epikv.select_tokens(s.reshape(-1).astype(np.float64), k)
    assert np.array_equal(got, want)


def test_select_distinct_bit_patterns():
    # scores spanning many exponents, including exact zeros and 1.0
    rng = np.random.default_rng(5)
    s = np.exp(rng.uniform(-80, 0, size=(3, 2, 3000))).astype(np.float32)
    s[1, 1, 100:200] = 0.0
    s[2, 0, 5] = 1.0
    dev = torch.from_numpy(s).cuda()
    for mode in (0, 1, 2):
        for r in (0.001, 0.25, 0.9):
            o, i = kvq.kv_topk_select(dev, r, mode)
            ro, ri = oracle.select(s, r, mode)
            assert np.array_equal(o.cpu().numpy(), ro)
            assert np.array_equal(i.cpu().numpy(), ri)


# model-wide budget (mode 2) at the full score-array sizes of the workloads
MODEL_BUDGET = [(32, 8, 8192, 0.3), (48, 8, 16384, 0.1), (32, 8, 131072, 0.3),
                (3, 5, 2999, 0.5), (1, 1, 4097, 0.001)]


@pytest.mark.parametrize("L,H,n_c,r", MODEL_BUDGET,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}" for c in MODEL_BUDGET])
def test_model_budget_bit_exact(L, H, n_c, r):
    _say("case: model budget", L, H, n_c, r)
    rng = np.random.default_rng(L * H + n_c)
    # quantised scores: long runs of exact ties across blocks and heads, with
    # per-head offsets so that heads get very different counts
    s = rng.integers(0, 64, size=(L, H, n_c)).astype(np.float32) / 256.0
    s += (rng.integers(0, 4, size=(L, H, 1)) / 16.0).astype(np.float32)
    dev = torch.from_numpy(s).cuda()
    ws = torch.empty(kvq.kv_topk_workspace_bytes(L, H, n_c, 2), dtype=torch.uint8,
                     device="cuda")
    for rr in (r, 1.0):
        o, i = kvq.kv_topk_select(dev, rr, 2, workspace=ws)
        ro, ri = oracle.select(s, rr, 2)
        assert np.array_equal(o.cpu().numpy(), ro), rr
        assert np.array_equal(i.cpu().numpy(), ri), rr
    # head-level scores and a ranking of the heads by them
    hs = kvq.kv_head_scores(dev)
    ref = oracle.head_level_scores(s)
    assert np.array_equal(hs.cpu().numpy(), ref)
    o, i = kvq.kv_topk_select(hs.reshape(1, 1, L * H), 0.5, 0)
    ro, ri = oracle.select(ref.reshape(1, 1, L * H), 0.5, 0)
    assert np.array_equal(i.cpu().numpy(), ri)


def test_head_scores_shapes():
    rng = np.random.default_rng(21)
    for (L, H, n_c) in [(1, 1, 1), (2, 3, 5), (5, 1, 1000), (1, 7, 64), (2, 2, 131073)]:
        s = rng.random((L, H, n_c)).astype(np.float32)
        s[0, 0, -1] = 1.0
        if n_c > 1:
            s[-1, -1, :] = 0.0
        got = kvq.kv_head_scores(torch.from_numpy(s).cuda()).cpu().numpy()
        assert np.array_equal(got, oracle.head_level_scores(s)), (L, H, n_c)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_compact_given_indices(d):
    rng = np.random.default_rng(d)
    L, H, n_c = 3, 2, 700
    k = rng.integers(0, 2 ** 16, size=(L, H, n_c, d), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(L, H, n_c, d), dtype=np.uint16)
    counts = rng.integers(0, 200, size=L * H)
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    idx = np.concatenate([np.sort(rng.choice(n_c, size=c, replace=False)) for c in counts]).astype(np.int32)
    ko, vo = kvq.kv_compact(to_dev_bf16(k), to_dev_bf16(v), torch.from_numpy(off).cuda(),
                            torch.from_numpy(idx).cuda())
    rko, rvo = oracle.compact(k, v, off, idx)
    assert np.array_equal(dev_bf16_bits(ko), rko)
    assert np.array_equal(dev_bf16_bits(vo), rvo)
    # indices outside [0, n_c) give zero rows (documented), never a stray read
    bad = idx.copy()
    bad[:: 7] = -1
    bad[3:: 11] = n_c
    ko, vo = kvq.kv_compact(to_dev_bf16(k), to_dev_bf16(v), torch.from_numpy(off).cuda(),
                            torch.from_numpy(bad).cuda())
    got = dev_bf16_bits(ko)
    zero = (bad < 0) | (bad >= n_c)
    assert np.all(got[zero] == 0)
    assert np.array_equal(got[~zero], rko[~zero])


def test_deterministic_reruns():
    w = synth.LLAMA8B_8K.shrink(n_c=3000, n_prompt=32, L=2, H=2)
    gen = synth.generate_workload(w, workers=1)
    dev = _upload(gen)
    a = _run(w, dev)
    b = _run(w, dev)
    for k in a:
        assert torch.equal(a[k], b[k]), k


# ---------------------------------------------------------------------------
# full-size workloads, launched exactly as the benchmark launches them
# ---------------------------------------------------------------------------
def _sampled_select_checks(w, out, S_ref, heads):
    """Band rule on the GPU-score selection, and bit-exact selection of the
    oracle's own (fp32-rounded) scores, for each sampled head."""
    off = out["offsets"].cpu().numpy()
    idx = out["idx"].cpu().numpy()
    k = oracle.keep_count(w.n_c, w.keep_ratio)
    for (l, h) in heads:
        band = check_topk_band(head_kept(off, idx, l * w.H + h), S_ref[l, h], k)
        _say(f"head ({l},{h}): near-tie band holds {band} keys")
        s32 = S_ref[l, h].astype(np.float32)[None, None]
        o2, i2 = kvq.kv_topk_select(torch.from_numpy(s32).cuda(), w.keep_ratio, 0)
        ro, ri = oracle.select(s32, w.keep_ratio, 0)
        assert np.array_equal(o2.cpu().numpy(), ro) and np.array_equal(i2.cpu().numpy(), ri)


def test_llama8b_8k_full_size():
    w = synth.LLAMA8B_8K
    _say("case: full", w.name)
    gen = synth.generate_workload(w, workers=WORKERS)
    out = _run(w, _upload(gen))
    heads = [(0, 0), (31, 7), (13, 5)]
    S_ref = _full_check(w, gen, out, heads)
    _sampled_select_checks(w, out, S_ref, heads)
    # every head: k ascending positions in range; compacted rows are the kept rows
    off = out["offsets"].cpu().numpy()
    idx = out["idx"].cpu().numpy()
    k = oracle.keep_count(w.n_c, w.keep_ratio)
    assert np.array_equal(off, np.arange(w.heads + 1) * k)
    per = idx.reshape(w.heads, k)
    assert np.all(np.diff(per, axis=1) > 0) and per.min() >= 0 and per.max() < w.n_c
    ko = dev_bf16_bits(out["k_out"]).reshape(w.heads, k, w.d)
    vo = dev_bf16_bits(out["v_out"]).reshape(w.heads, k, w.d)
    kc = gen["k_ctx"].reshape(w.heads, w.n_c, w.d)
    vc = gen["v_ctx"].reshape(w.heads, w.n_c, w.d)
    for lh in (0, 77, 255):
        assert np.array_equal(ko[lh], kc[lh][per[lh]])
        assert np.array_equal(vo[lh], vc[lh][per[lh]])
    # full-size compaction of an index set the oracle made, bit-exact
    rng = np.random.default_rng(7)
    ridx = np.concatenate([np.sort(rng.choice(w.n_c, size=k, replace=False))
                           for _ in range(w.heads)]).astype(np.int32)
    roff = (np.arange(w.heads + 1) * k).astype(np.int64)
    ko2, vo2 = kvq.kv_compact(to_dev_bf16(gen["k_ctx"]), to_dev_bf16(gen["v_ctx"]),
                              torch.from_numpy(roff).cuda(), torch.from_numpy(ridx).cuda())
    rko, rvo = oracle.compact(gen["k_ctx"], gen["v_ctx"], roff, ridx)
    assert np.array_equal(dev_bf16_bits(ko2), rko)
    assert np.array_equal(dev_bf16_bits(vo2), rvo)


def _full_size_inputs(w, true_heads, seed=1234):
    """Device inputs at the workload's full shape: the heads in `true_heads`
    carry the seeded generator's values, the others cheap seeded GPU noise
    (same launch configuration; only the listed heads are checked)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    shapes = {"q": (w.G, w.n_in, w.d), "k_ctx": (w.n_c, w.d),
              "k_new": (w.n_in, w.d), "v_ctx": (w.n_c, w.d)}
    dev = {}
    for k, shp in shapes.items():
        t = torch.empty((w.L, w.H) + shp, dtype=torch.bfloat16, device="cuda")
        for l in range(w.L):
            t[l] = torch.randn((w.H,) + shp, generator=g, device="cuda").to(torch.bfloat16)
        dev[k] = t
    gens = {}
    for (l, h) in true_heads:
        gh = synth.generate_head(w, l, h)
        gens[(l, h)] = gh
        for k in shapes:
            dev[k][l, h] = to_dev_bf16(gh[k])
    torch.cuda.synchronize()
    return dev, gens


def _check_heads(w, out, gens, heads):
    lse_g, sc_g = out["lse"], out["scores"]
    S_ref = {}
    for (l, h) in heads:
        _say(f"oracle head ({l},{h}) of {w.name}")
        S, lse = oracle_head({k: gens[(l, h)][k] for k in ("q", "k_ctx", "k_new")},
                             float(w.scale), workers=WORKERS)
        check_lse(lse_g[l, h].cpu().numpy(), lse, f"lse[{l},{h}]")
        check_scores(sc_g[l, h].cpu().numpy(), S, f"scores[{l},{h}]")
        S_ref[(l, h)] = S
    return S_ref


def test_qwen14b_32k_full_size():
    w = synth.QWEN14B_32K
    heads = [(0, 0), (47, 7)]
    _say("case: full", w.name)
    dev, gens = _full_size_inputs(w, heads)
    out = _run(w, dev)
    S_ref = _check_heads(w, out, gens, heads)
    off = out["offsets"].cpu().numpy()
    idx = out["idx"].cpu().numpy()
    k = oracle.keep_count(w.n_c, w.keep_ratio)
    assert np.array_equal(off, np.arange(w.heads + 1) * k)
    for (l, h) in heads:
        lh = l * w.H + h
        band = check_topk_band(head_kept(off, idx, lh), S_ref[(l, h)], k)
        _say(f"head ({l},{h}): near-tie band holds {band} keys")
        s32 = S_ref[(l, h)].astype(np.float32)[None, None]
        o2, i2 = kvq.kv_topk_select(torch.from_numpy(s32).cuda(), w.keep_ratio, 0)
        ro, ri = oracle.select(s32, w.keep_ratio, 0)
        assert np.array_equal(i2.cpu().numpy(), ri)
        kept = head_kept(off, idx, lh)
        assert np.array_equal(dev_bf16_bits(out["k_out"][off[lh]:off[lh + 1]]),
                              gens[(l, h)]["k_ctx"][kept])


def test_gemma12b_16k_full_size_both_modes():
    w = synth.GEMMA12B_16K
    layer = w.L - 1
    heads = [(0, 0)] + [(layer, h) for h in range(w.H)]
    _say("case: full", w.name)
    dev, gens = _full_size_inputs(w, heads)
    out0 = _run(w, dev, 0)
    S_ref = _check_heads(w, out0, gens, heads)
    k = oracle.keep_count(w.n_c, w.keep_ratio)
    off = out0["offsets"].cpu().numpy()
    idx = out0["idx"].cpu().numpy()
    for (l, h) in heads:
        check_topk_band(head_kept(off, idx, l * w.H + h), S_ref[(l, h)], k)
    # mode 1: one budget over the layer's H * n_c scores
    sc = out0["scores"]
    off1, idx1 = kvq.kv_topk_select(sc, w.keep_ratio, 1)
    off1 = off1.cpu().numpy()
    idx1 = idx1.cpu().numpy()
    kl = oracle.keep_count(w.H * w.n_c, w.keep_ratio)
    assert off1[-1] == w.L * kl
    lay = np.stack([S_ref[(layer, h)] for h in range(w.H)])        # (H, n_c)
    flat_kept = np.concatenate([head_kept(off1, idx1, layer * w.H + h) + h * w.n_c
                                for h in range(w.H)])
    band = check_topk_band(flat_kept, lay.reshape(-1), kl)
    _say(f"layer {layer} budget: near-tie band holds {band} keys")
    # mode 1 on the oracle's own scores: bit-exact
    s32 = lay.astype(np.float32)[None]
    o2, i2 = kvq.kv_topk_select(torch.from_numpy(s32).cuda(), w.keep_ratio, 1)
    ro, ri = oracle.select(s32, w.keep_ratio, 1)
    assert np.array_equal(o2.cpu().numpy(), ro) and np.array_equal(i2.cpu().numpy(), ri)
    # mode 2 (one budget over the model) on the GPU scores: a valid top-k of
    # those scores, and compaction of it equal to the kept input rows
    _model_budget_checks(w, dev, sc, heads, S_ref)


def _model_budget_checks(w, dev, sc, heads, S_ref):
    off2, idx2 = kvq.kv_topk_select(sc, w.keep_ratio, 2)
    ko, vo = kvq.kv_compact(dev["k_ctx"], dev["v_ctx"], off2, idx2)
    off2 = off2.cpu().numpy()
    idx2 = idx2.cpu().numpy()
    km = oracle.keep_count(w.L * w.H * w.n_c, w.keep_ratio)
    assert off2[0] == 0 and off2[-1] == km and np.all(np.diff(off2) >= 0)
    sc_np = sc.cpu().numpy()
    check_valid_topk(sc_np, flat_kept(off2, idx2, w.n_c), km)
    _say(f"model budget: {km} kept, per-head counts "
         f"{np.diff(off2).min()}..{np.diff(off2).max()}")
    hs = kvq.kv_head_scores(sc).cpu().numpy()
    assert np.array_equal(hs, sc_np.max(axis=2))
    for (l, h) in heads:
        lh = l * w.H + h
        rows = idx2[off2[lh]:off2[lh + 1]]
        assert np.array_equal(dev_bf16_bits(ko[off2[lh]:off2[lh + 1]]),
                              dev_bf16_bits(dev["k_ctx"][l, h])[rows])
        assert np.array_equal(dev_bf16_bits(vo[off2[lh]:off2[lh + 1]]),
                              dev_bf16_bits(dev["v_ctx"][l, h])[rows])
        if S_ref is not None:   # head-level score against the oracle's
            check_scores(hs[l, h:h + 1], np.array([S_ref[(l, h)].max()]),
                         f"head score ({l},{h})")


def _golden_128k(l, h):
    """The float64 oracle's stored values of one whole head of the 128K
    workload (written by tests/golden/make_llama128k_head.py)."""
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        f"llama3.1-8b-128k_head{l}-{h}.npz")


def test_llama8b_128k_full_size_sampled():
    w = synth.LLAMA8B_128K
    l, h = 0, 0
    gl, gh_ = w.L - 1, w.H - 1
    _say("case: full", w.name)
    dev, gens = _full_size_inputs(w, [(l, h), (gl, gh_)])
    out = _run(w, dev)
    # whole-head parity of the first and the last head against the float64
    # oracle's stored values: every score, the lse of every 16th row, and the
    # kept set outside the near-tie band
    k = oracle.keep_count(w.n_c, w.keep_ratio)
    for (hl, hh) in ((l, h), (gl, gh_)):
        gold = np.load(_golden_128k(hl, hh))
        assert (int(gold["layer"]), int(gold["head"])) == (hl, hh)
        S_gold = gold["scores"].astype(np.float64)
        check_scores(out["scores"][hl, hh].cpu().numpy(), S_gold, f"scores[{hl},{hh}]")
        check_lse(out["lse"][hl, hh].cpu().numpy()[:, ::16],
                  gold["lse_rows16"].astype(np.float64), f"lse[{hl},{hh}] every 16th row")
        band = check_topk_band(head_kept(out["offsets"].cpu().numpy(), out["idx"].cpu().numpy(),
                                         hl * w.H + hh), S_gold, k)
        _say(f"head ({hl},{hh}): whole head within tolerance, near-tie band holds {band} keys")
    gh = gens[(l, h)]
    q, kc, kn = oracle.workload_head_inputs(gh)
    lse_g = out["lse"][l, h].cpu().numpy()
    sc_g = out["scores"][l, h].cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(3)
    rows = [(g, i) for g in range(w.G) for i in (0, 1, w.n_prompt, w.n_in - 1)]
    rows += [(int(rng.integers(w.G)), int(rng.integers(w.n_in))) for _ in range(24)]
    k_all = np.concatenate([kc, kn])
    for (g, i) in rows:
        want = oracle.row_lse(q[g, i], i, kc, kn, float(w.scale))
        check_lse(np.array([lse_g[g, i]]), np.array([want]), f"lse[{g},{i}]")
        # every score is at least the probability this row gives the key
        a, _ = oracle.attention_rows(q[g, i][None], np.array([i]), k_all, w.n_c, float(w.scale))
        p = a[0, :w.n_c]
        assert np.all(sc_g >= p * (1 - 2e-3) - 1e-6), f"score below row ({g},{i})"
    assert np.all(sc_g >= 0) and np.all(sc_g <= 1)
    # exact copies of a key (the repeated spans) receive identical logits in
    # every row, hence identical scores
    span = np.arange(64, 128)
    for kk in (1, 7, 31):
        assert np.array_equal(sc_g[4096 * kk + span], sc_g[span])
    # selection: k keys, ascending; the kept set is a valid top-k of the GPU
    # scores with ties broken toward the lower index
    off = out["offsets"].cpu().numpy()
    kept = head_kept(off, out["idx"].cpu().numpy(), 0)
    k = oracle.keep_count(w.n_c, w.keep_ratio)
    assert kept.size == k and np.all(np.diff(kept) > 0)
    s32 = out["scores"][l, h].cpu().numpy()
    thr = s32[kept].min()
    dropped = np.setdiff1d(np.arange(w.n_c), kept)
    assert s32[dropped].max() <= thr, "a dropped key outscored a kept one"
    eq = np.flatnonzero(s32 == thr)
    kept_eq = np.intersect1d(kept, eq)
    assert np.array_equal(kept_eq, eq[:kept_eq.size]), "ties must go to the lower index"
    # one budget over the whole model's 33.5M scores
    _model_budget_checks(w, dev, out["scores"], [(l, h)], None)


# ---------------------------------------------------------------------------
# chunked scoring (KVzip page, section 3.4)
# ---------------------------------------------------------------------------
def _chunked_inputs(w, chunk, heads=None):
    rows = synth.chunk_rows(w, chunk)
    gens = {}
    q = np.zeros((w.L, w.H, rows * w.G, w.d), np.uint16)
    kn = np.zeros((w.L, w.H, rows, w.d), np.uint16)
    kc = np.zeros((w.L, w.H, w.n_c, w.d), np.uint16)
    for l in range(w.L):
        for h in range(w.H):
            if heads is not None and (l, h) not in heads:
                continue
            g = synth.generate_chunked_head(w, l, h, chunk, ("q", "k_ctx", "k_new"))
            gens[(l, h)] = g
            q[l, h], kn[l, h], kc[l, h] = g["q"], g["k_new"], g["k_ctx"]
    return gens, {"q": to_dev_bf16(q), "k_new": to_dev_bf16(kn), "k_ctx": to_dev_bf16(kc)}


CHUNKED = [
    # (base, G, d, n_c, n_prompt, chunk, L, H)
    ("tiny", 4, 64, 512, 16, 128, 1, 1),
    ("tiny", 4, 64, 512, 16, 200, 1, 2),
    ("llama3.1-8b-8k", 4, 128, 1000, 32, 300, 2, 1),
    ("gemma3-12b-16k", 2, 256, 300, 5, 64, 1, 2),
    ("qwen2.5-14b-32k", 5, 128, 77, 0, 1, 1, 1),
    ("llama3.1-8b-8k", 3, 128, 70, 3, 1000, 1, 1),
    # several chunks per workgroup in pass 1, in groups of up to four chunks
    # of one head: 5 full chunks per head (groups of 4 and 1) over 2 x 2
    # heads, and 6 per head (4 and 2) over 3 heads at d = 256
    ("llama3.1-8b-8k", 4, 128, 700, 8, 128, 2, 2),
    ("gemma3-12b-16k", 2, 256, 384, 4, 64, 1, 3),
]


@pytest.mark.parametrize("case", CHUNKED, ids=[f"d{c[2]}-nc{c[3]}-m{c[5]}" for c in CHUNKED])
def test_chunked_parity(case):
    base, G, d, n_c, n_p, chunk, L, H = case
    w = synth.BY_NAME[base].shrink(G=G, d=d, n_c=n_c, n_prompt=n_p, L=L, H=H,
                                   rank=min(synth.BY_NAME[base].rank, d))
    _say("case:", case)
    gens, dev = _chunked_inputs(w, chunk)
    sc, lse = kvq.score_chunked(dev["q"], dev["k_ctx"], dev["k_new"], G, n_p, chunk,
                                scale=float(w.scale))
    torch.cuda.synchronize()
    for (l, h), g in gens.items():
        S, l_ref = oracle.chunked_head_scores(
            oracle.bf16_to_f64(g["q"]), oracle.bf16_to_f64(g["k_ctx"]),
            oracle.bf16_to_f64(g["k_new"]), float(w.scale), n_p, chunk, G)
        check_lse(lse[l, h].cpu().numpy(), l_ref, f"lse[{l},{h}]")
        check_scores(sc[l, h].cpu().numpy(), S, f"scores[{l},{h}]")


def test_chunked_whole_context_equals_unchunked():
    w = synth.LLAMA8B_8K.shrink(n_c=777, n_prompt=9, L=1, H=2)
    gen = synth.generate_workload(w, workers=1)
    dev = _upload(gen)
    sc0 = kvq.kvscore_colmax(dev["q"], dev["k_ctx"],
                             kvq.kvscore_lse(dev["q"], dev["k_ctx"], dev["k_new"], scale=float(w.scale)),
                             scale=float(w.scale))
    q = dev["q"].reshape(w.L, w.H, w.G * w.n_in, w.d)
    for chunk in (w.n_c, 5000):
        sc1, _ = kvq.score_chunked(q, dev["k_ctx"], dev["k_new"], w.G, w.n_prompt, chunk,
                                   scale=float(w.scale))
        assert torch.equal(sc0, sc1)


def test_llama8b_128k_chunked_full_size():
    w = synth.LLAMA8B_128K
    chunk = 2048
    heads = [(0, 0), (31, 7)]
    _say("case: chunked full", w.name, chunk)
    rows = synth.chunk_rows(w, chunk)
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    q = torch.randn((w.L, w.H, rows * w.G, w.d), generator=g, device="cuda").to(torch.bfloat16)
    kn = torch.randn((w.L, w.H, rows, w.d), generator=g, device="cuda").to(torch.bfloat16)
    kc = torch.randn((w.L, w.H, w.n_c, w.d), generator=g, device="cuda").to(torch.bfloat16)
    gens = {}
    for (l, h) in heads:
        gh = synth.generate_chunked_head(w, l, h, chunk, ("q", "k_ctx", "k_new"))
        gens[(l, h)] = gh
        q[l, h], kn[l, h], kc[l, h] = to_dev_bf16(gh["q"]), to_dev_bf16(gh["k_new"]), to_dev_bf16(gh["k_ctx"])
    sc, lse = kvq.score_chunked(q, kc, kn, w.G, w.n_prompt, chunk, scale=float(w.scale))
    torch.cuda.synchronize()
    for (l, h) in heads:
        gh = gens[(l, h)]
        S, l_ref = oracle.chunked_head_scores(
            oracle.bf16_to_f64(gh["q"]), oracle.bf16_to_f64(gh["k_ctx"]),
            oracle.bf16_to_f64(gh["k_new"]), float(w.scale), w.n_prompt, chunk, w.G,
            workers=WORKERS)
        check_lse(lse[l, h].cpu().numpy(), l_ref, f"lse[{l},{h}]")
        check_scores(sc[l, h].cpu().numpy(), S, f"scores[{l},{h}]")


def test_one_million_key_head():
    # the largest context here: one head of 2^20 cached keys (8x the 128K
    # workload), G = 2, from the seeded generator; sampled rows against the
    # oracle's row definition, every score against the rows' lower bounds,
    # and the selection as a valid top-k of the GPU scores
    w = synth.LLAMA8B_8K.shrink(n_c=1 << 20, n_prompt=32, L=1, H=1, G=2, structure="none")
    _say("case: one head of", w.n_c, "keys")
    gen = synth.generate_workload(w, workers=WORKERS)
    dev = _upload(gen)
    out = _run(w, dev)
    q, kc, kn = oracle.workload_head_inputs({k: gen[k][0, 0] for k in ("q", "k_ctx", "k_new")})
    lse_g = out["lse"][0, 0].cpu().numpy()
    sc_g = out["scores"][0, 0].cpu().numpy().astype(np.float64)
    k_all = np.concatenate([kc, kn])
    rng = np.random.default_rng(4)
    rows = [(g, i) for g in range(w.G) for i in (0, w.n_prompt, w.n_in - 1)]
    rows += [(int(rng.integers(w.G)), int(rng.integers(w.n_in))) for _ in range(6)]
    for (g, i) in rows:
        a, l = oracle.attention_rows(q[g, i][None], np.array([i]), k_all[: w.n_c + i + 1],
                                     w.n_c, float(w.scale))
        check_lse(np.array([lse_g[g, i]]), l, f"lse[{g},{i}]")
        assert np.all(sc_g >= a[0, :w.n_c] * (1 - 2e-3) - 1e-6), f"score below row ({g},{i})"
    assert np.all(sc_g >= 0) and np.all(sc_g <= 1)
    k = oracle.keep_count(w.n_c, w.keep_ratio)
    kept = head_kept(out["offsets"].cpu().numpy(), out["idx"].cpu().numpy(), 0)
    check_valid_topk(out["scores"][0, 0].cpu().numpy(), kept, k)
    assert np.array_equal(dev_bf16_bits(out["k_out"]), gen["k_ctx"][0, 0][kept])
    # the model-wide budget over the same 2^20 scores equals mode 0 here
    o2, i2 = kvq.kv_topk_select(out["scores"], w.keep_ratio, 2)
    assert torch.equal(i2, out["idx"]) and torch.equal(o2, out["offsets"])


# the compaction's head search over many heads, empty heads among them
@pytest.mark.parametrize("L,H", [(1, 1), (16, 128), (1, 2049), (3, 1000)])
def test_compact_many_heads(L, H):
    _say("case: compact heads", L, H)
    rng = np.random.default_rng(L * H)
    n_c, d = 9, 64
    k = rng.integers(0, 2 ** 16, size=(L, H, n_c, d), dtype=np.uint16)
    v = rng.integers(0, 2 ** 16, size=(L, H, n_c, d), dtype=np.uint16)
    counts = rng.integers(0, n_c + 1, size=L * H)       # empty heads included
    counts[0] = n_c
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    idx = np.concatenate([np.sort(rng.choice(n_c, size=c, replace=False)) for c in counts]).astype(np.int32)
    ko, vo = kvq.kv_compact(to_dev_bf16(k), to_dev_bf16(v), torch.from_numpy(off).cuda(),
                            torch.from_numpy(idx).cuda())
    rko, rvo = oracle.compact(k, v, off, idx)
    assert np.array_equal(dev_bf16_bits(ko), rko)
    assert np.array_equal(dev_bf16_bits(vo), rvo)
