"""GPU parity of the attention-free EpiKV path (EpiKV page, section 3.2,
equations 1-3; section 3.1 budget) through libkvq's C ABI, against the
float64 oracle in oracle.epikv.

Tolerances (derived from the arithmetic, see epi_tolerances):
  g: relative 1e-5 (fp32 differences of bf16 inputs, fp32 fma sums of at
     most 8 * 16 terms per lane plus a 6-level butterfly, fp32 sqrt);
  scores: first-order propagation of that relative error through the window
     mean and deviation (fp64 on both sides), plus the final fp32 rounding.
Selection on the oracle's scores and compaction are bit-exact; selection on
the GPU's own scores must hold every key that the tolerance cannot move
across the threshold.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import query_agnostic_eviction_amd as kvq
from oracle import epikv as E
from parity_util import dev_bf16_bits, to_dev_bf16

pytestmark = pytest.mark.gpu

G_RTOL = 1e-5


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    kvq.api._lib.load()
    yield
    torch.cuda.synchronize()


def _windows(x, w):
    """Per position t >= 1: (count, max |x|, population std) over the window
    max(1, t-w+1)..t (position 0: zeros).  Test-side helper for tolerances."""
    n = x.shape[0]
    cnt = np.zeros(n)
    mx = np.zeros(n)
    sd = np.zeros(n)
    for t in range(1, n):
        win = x[max(1, t - w + 1):t + 1]
        cnt[t] = win.size
        mx[t] = np.abs(win).max()
        sd[t] = win.std()
    return cnt, mx, sd


def epi_tolerances(g_ref, n_a, w, eps, detrend):
    """Per-position bound on |score_gpu - score_ref|."""
    nl, n = g_ref.shape
    tol = np.zeros(n)
    for l in range(nl):
        _, mx, sd = _windows(g_ref[l], w)
        per = 1.0 / (n_a if l < n_a else nl - n_a)
        if detrend:
            z = E.rolling_zscore(g_ref[l], w, eps)
            tol += per * (2.0 + np.abs(z)) * G_RTOL * mx / (sd + eps)
        else:
            tol += per * G_RTOL * mx
    return 1.5 * tol + 1e-12


def oracle_path(hbits, n_a, w, eps, detrend):
    g = np.stack([E.hidden_deltas(oracle.bf16_to_f64(hbits[l])) for l in range(hbits.shape[0])])
    s = E.token_scores(list(g[:n_a]), list(g[n_a:]), w, eps, detrend)
    return g, s


def check_g(g_gpu, g_ref):
    err = np.abs(g_gpu - g_ref)
    bad = err > G_RTOL * np.abs(g_ref) + 1e-30
    assert not bad.any(), (f"g mismatch at {np.argwhere(bad)[:5].tolist()}: "
                           f"gpu {g_gpu[bad][:5]} ref {g_ref[bad][:5]}")


def check_scores(s_gpu, s_ref, tol):
    err = np.abs(s_gpu.astype(np.float64) - s_ref)
    bad = err > tol + 2.0 ** -23 * np.abs(s_ref)
    assert not bad.any(), (f"score mismatch at {np.flatnonzero(bad)[:5].tolist()}: "
                           f"gpu {s_gpu[bad][:5]} ref {s_ref[bad][:5]} tol {tol[bad][:5]}")


def check_select_band(kept, s_ref, tol, k):
    """Keys that no score within tolerance can move across the k-th place."""
    kept = np.asarray(kept)
    assert kept.size == k and np.all(np.diff(kept) > 0)
    hi, lo = s_ref + tol, s_ref - tol
    h_k = np.sort(hi)[::-1][k - 1]
    l_k = np.sort(lo)[::-1][k - 1]
    mask = np.zeros(s_ref.size, bool)
    mask[kept] = True
    assert mask[lo > h_k].all(), "a key certainly in the top-k was dropped"
    assert not mask[hi < l_k].any(), "a key certainly outside the top-k was kept"
    return int(np.count_nonzero((lo <= h_k) & (hi >= l_k)))


def run_and_check(w, hbits, n_a, detrend=True, kv=None):
    _say("case:", w.name, "n", w.n, "D", w.D, "layers", hbits.shape[0], "n_a", n_a,
         "window", w.window, "detrend", detrend)
    h_dev = to_dev_bf16(hbits)
    g_gpu = kvq.kv_epi_deltas(h_dev)
    s_gpu = kvq.kv_epi_scores(g_gpu, n_a, w.window, w.eps, detrend)
    torch.cuda.synchronize()
    g_ref, s_ref = oracle_path(hbits, n_a, w.window, w.eps, detrend)
    g_np = g_gpu.cpu().numpy().astype(np.float64)
    check_g(g_np, g_ref)
    assert np.all(g_np[:, 0] == 0.0)
    tol = epi_tolerances(g_ref, n_a, w.window, w.eps, detrend)
    s_np = s_gpu.cpu().numpy()
    check_scores(s_np, s_ref, tol)
    assert s_np[0] == 0.0
    k = min(w.budget, w.n)
    idx = kvq.kv_select_tokens(s_gpu, k).cpu().numpy()
    band = check_select_band(idx, s_ref, tol, k)
    _say(f"  select on GPU scores: {band} keys inside the tolerance band")
    # selection of the oracle's own scores (fp32) is bit-exact
    s32 = s_ref.astype(np.float32)
    got = kvq.kv_select_tokens(torch.from_numpy(s32).cuda(), k).cpu().numpy()
    assert np.array_equal(got, E.select_tokens(s32, k))
    return idx


# ---------------------------------------------------------------------------
def test_tiny_end_to_end():
    w = synth.EPIKV_TINY
    hbits = synth.generate_hidden(w)
    kc, vc = synth.generate_kv(w)
    for detrend in (True, False):
        idx = run_and_check(w, hbits, len(w.band_a), detrend)
    ko, vo, idx2, _, _ = kvq.epikv_evict(to_dev_bf16(hbits), len(w.band_a), to_dev_bf16(kc),
                                         to_dev_bf16(vc), w.budget, w.window, w.eps)
    ref_idx = kvq.kv_select_tokens(kvq.kv_epi_scores(kvq.kv_epi_deltas(to_dev_bf16(hbits)),
                                                     len(w.band_a), w.window, w.eps), w.budget)
    assert torch.equal(idx2, ref_idx)
    rk, rv = E.compact_tokens(kc, vc, idx2.cpu().numpy())
    assert np.array_equal(dev_bf16_bits(ko), rk)
    assert np.array_equal(dev_bf16_bits(vo), rv)


RAGGED = [
    # (n, D, n_a, n_b, window)
    (1, 8, 1, 1, 64),
    (2, 56, 1, 1, 1),
    (33, 512, 2, 1, 2),
    (1000, 3584, 1, 1, 64),
    (777, 4104, 1, 2, 64),
    (300, 8192, 1, 1, 1024),
    (5000, 4096, 3, 2, 100),
    (4097, 1024, 1, 1, 64),
]


@pytest.mark.parametrize("case", RAGGED, ids=[f"n{c[0]}-D{c[1]}-a{c[2]}b{c[3]}-w{c[4]}"
                                              for c in RAGGED])
def test_ragged_shapes(case):
    n, D, n_a, n_b, win = case
    w = synth.EPIKV_TINY.shrink(n=n, D=D, window=win, budget=max(1, n // 3),
                                band_a=tuple(range(1, 1 + n_a)),
                                band_b=tuple(range(10, 10 + n_b)))
    hbits = synth.generate_hidden(w)
    for detrend in (True, False):
        run_and_check(w, hbits, n_a, detrend)


def test_constant_and_ramp_hidden_states():
    # h(t) = t * u: every delta is |u|, so every window is constant: z = 0
    # and the raw band difference is |u_A| - |u_B|
    n, D = 500, 256
    u_a = np.zeros(D); u_a[:4] = [1.0, 2.0, 2.0, 0.0]          # |u| = 3
    u_b = np.zeros(D); u_b[5:7] = [0.5, 0.0]                   # |u| = 0.5
    h = np.stack([np.outer(np.arange(n) * 1.0, u_a), np.outer(np.arange(n) * 1.0, u_b)])
    hb = synth.generate.f64_to_bf16_bits(h)
    g = kvq.kv_epi_deltas(to_dev_bf16(hb))
    gg = g.cpu().numpy()
    # bf16 holds these integers exactly up to 256; beyond that rounding moves
    # single rows, so check the exact prefix
    assert gg[0, 0] == 0.0 and gg[1, 0] == 0.0
    assert np.allclose(gg[0, 1:200], 3.0, rtol=2 ** -22, atol=0)
    assert np.allclose(gg[1, 1:200], 0.5, rtol=2 ** -22, atol=0)
    assert np.unique(gg[0, 1:200]).size == 1 and np.unique(gg[1, 1:200]).size == 1
    z = kvq.kv_epi_scores(g[:, :200].contiguous(), 1, 64, 1e-6, True).cpu().numpy()
    assert np.all(z == 0.0)        # a constant window: mean exact, deviation 0
    raw = kvq.kv_epi_scores(g[:, :200].contiguous(), 1, 64, 1e-6, False).cpu().numpy()
    assert raw[0] == 0.0 and np.allclose(raw[1:], 2.5, rtol=1e-6, atol=0)


@pytest.mark.parametrize("n", [1, 7, 1024, 4097, 65536, 1 << 20])
def test_select_tokens_bit_exact(n):
    rng = np.random.default_rng(n)
    s = (rng.integers(-8, 8, size=n) / 4.0).astype(np.float32)
    s[rng.random(n) < 0.1] = -0.0
    s[rng.random(n) < 0.05] = np.float32(rng.normal()) * 1e-30
    dev = torch.from_numpy(s).cuda()
    for k in sorted({1, max(1, n // 10), max(1, n // 2), n}):
        got = kvq.kv_select_tokens(dev, k).cpu().numpy()
        assert np.array_equal(got, E.select_tokens(s, k)), (n, k)


def test_compact_tokens_edges():
    rng = np.random.default_rng(9)
    L, H, n, d = 2, 3, 300, 128
    kc = rng.integers(0, 2 ** 16, size=(L, H, n, d), dtype=np.uint16)
    vc = rng.integers(0, 2 ** 16, size=(L, H, n, d), dtype=np.uint16)
    idx = np.sort(rng.choice(n, size=77, replace=False)).astype(np.int32)
    ko, vo = kvq.kv_compact_tokens(to_dev_bf16(kc), to_dev_bf16(vc), torch.from_numpy(idx).cuda())
    rk, rv = E.compact_tokens(kc, vc, idx)
    assert np.array_equal(dev_bf16_bits(ko), rk) and np.array_equal(dev_bf16_bits(vo), rv)
    bad = idx.copy()
    bad[::5] = -3
    bad[1::7] = n
    ko, _ = kvq.kv_compact_tokens(to_dev_bf16(kc), to_dev_bf16(vc), torch.from_numpy(bad).cuda())
    got = dev_bf16_bits(ko)
    zero = (bad < 0) | (bad >= n)
    assert np.all(got[:, :, zero] == 0)
    assert np.array_equal(got[:, :, ~zero], rk[:, :, ~zero])


def test_epikv_r1_8b_64k_full_size():
    w = synth.EPIKV_R1_8B_64K
    _say("case: full", w.name)
    hbits = synth.generate_hidden(w)
    idx = run_and_check(w, hbits, len(w.band_a), True)
    # token compaction of the full 32 x 8 x 65536 x 128 caches, launched as
    # the benchmark launches it; random bit patterns made on the device
    gen = torch.Generator(device="cuda").manual_seed(7)
    shape = (w.L, w.H, w.n, w.d)
    kc = torch.randint(-32768, 32767, shape, dtype=torch.int16, device="cuda",
                       generator=gen).view(torch.bfloat16)
    vc = torch.randint(-32768, 32767, shape, dtype=torch.int16, device="cuda",
                       generator=gen).view(torch.bfloat16)
    idx_dev = torch.from_numpy(idx).cuda()
    ko, vo = kvq.kv_compact_tokens(kc, vc, idx_dev)
    torch.cuda.synchronize()
    for (l, h) in [(0, 0), (w.L - 1, w.H - 1), (13, 5)]:
        assert torch.equal(ko[l, h].view(torch.int16), kc[l, h][idx_dev.long()].view(torch.int16))
        assert torch.equal(vo[l, h].view(torch.int16), vc[l, h][idx_dev.long()].view(torch.int16))


@pytest.mark.parametrize("i", range(40))
def test_random_shapes(i):
    rng = np.random.default_rng(7000 + i)
    n = int(rng.choice([1, 2, 63, 64, 65, int(rng.integers(2, 5000))]))
    D = int(8 * rng.integers(1, 1025))
    n_a, n_b = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    win = int(rng.choice([1, 2, 64, int(rng.integers(1, 1025))]))
    eps = float(rng.choice([1e-6, 1e-3, 1.0]))
    w = synth.EPIKV_TINY.shrink(n=n, D=D, window=win, eps=eps, seed=i,
                                budget=int(rng.integers(1, n + 1)),
                                band_a=tuple(range(1, 1 + n_a)),
                                band_b=tuple(range(10, 10 + n_b)))
    hbits = synth.generate_hidden(w)
    run_and_check(w, hbits, n_a, bool(rng.integers(2)))
