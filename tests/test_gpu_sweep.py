"""Seeded random sweep of small shapes through the whole KVzip path (scores,
lse, all three budgets, compaction, chunked scoring) against the float64
oracle, to the tolerances of parity_util.  Shapes are drawn so that tile
tails, single-key contexts, prompt-free passes, G up to 8 and every head
dimension occur."""
import numpy as np
import pytest
import torch

import oracle
import synth
import query_agnostic_eviction_amd as kvq
from parity_util import (check_lse, check_scores, check_topk_band, dev_bf16_bits,
                         head_kept, to_dev_bf16)

pytestmark = pytest.mark.gpu

N_CASES = 160


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    kvq.api._lib.load()
    yield
    torch.cuda.synchronize()


def _draw(i):
    rng = np.random.default_rng(9000 + i)
    base = synth.ALL[int(rng.integers(len(synth.ALL)))]
    d = int(rng.choice([64, 128, 256]))
    G = int(rng.integers(1, 9))
    n_c = int(rng.choice([1, 2, 31, 32, 33, int(rng.integers(1, 3000))]))
    n_p = int(rng.choice([0, 1, int(rng.integers(0, 40))]))
    L, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
    r = float(rng.choice([0.01, 0.1, 0.3, 0.5, 0.99, 1.0]))
    chunk = int(rng.choice([0, 1, 7, 64, int(rng.integers(1, 4000))]))
    w = base.shrink(G=G, d=d, n_c=n_c, n_prompt=n_p, L=L, H=H, keep_ratio=r,
                    rank=min(base.rank, d), seed=i)
    return w, chunk


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    w, chunk = _draw(i)
    _say(f"case {i}: {w.name} L{w.L} H{w.H} G{w.G} d{w.d} n_c{w.n_c} n_p{w.n_prompt} "
         f"r{w.keep_ratio} chunk{chunk}")
    gen = synth.generate_workload(w, workers=1)
    dev = {k: to_dev_bf16(v) for k, v in gen.items()}
    scale = float(w.scale)
    lse = kvq.kvscore_lse(dev["q"], dev["k_ctx"], dev["k_new"], scale=scale)
    sc = kvq.kvscore_colmax(dev["q"], dev["k_ctx"], lse, scale=scale)
    torch.cuda.synchronize()
    lse_g, sc_g = lse.cpu().numpy(), sc.cpu().numpy()
    S_ref = np.zeros((w.L, w.H, w.n_c))
    for l in range(w.L):
        for h in range(w.H):
            q, kc, kn = oracle.workload_head_inputs({k: gen[k][l, h] for k in ("q", "k_ctx", "k_new")})
            S, ls = oracle.head_scores(q, kc, kn, scale)
            check_lse(lse_g[l, h], ls, f"lse[{l},{h}]")
            check_scores(sc_g[l, h], S, f"scores[{l},{h}]")
            S_ref[l, h] = S
    s32 = S_ref.astype(np.float32)
    for mode in (0, 1, 2):
        o, x = kvq.kv_topk_select(torch.from_numpy(s32).cuda(), w.keep_ratio, mode)
        ro, rx = oracle.select(s32, w.keep_ratio, mode)
        assert np.array_equal(o.cpu().numpy(), ro) and np.array_equal(x.cpu().numpy(), rx), mode
        ko, vo = kvq.kv_compact(dev["k_ctx"], dev["v_ctx"], o, x)
        rko, rvo = oracle.compact(gen["k_ctx"], gen["v_ctx"], ro, rx)
        assert np.array_equal(dev_bf16_bits(ko), rko) and np.array_equal(dev_bf16_bits(vo), rvo)
    # selection of the GPU's own scores: exact outside the near-tie band
    off, idx = kvq.kv_topk_select(sc, w.keep_ratio, 0)
    k = oracle.keep_count(w.n_c, w.keep_ratio)
    for l in range(w.L):
        for h in range(w.H):
            check_topk_band(head_kept(off.cpu().numpy(), idx.cpu().numpy(), l * w.H + h),
                            S_ref[l, h], k)
    hs = kvq.kv_head_scores(torch.from_numpy(s32).cuda()).cpu().numpy()
    assert np.array_equal(hs, oracle.head_level_scores(s32))
    if chunk:
        cgen = synth.generate_chunked_workload(w, chunk, workers=1)
        cdev = {k: to_dev_bf16(v) for k, v in cgen.items()}
        clse = kvq.kvscore_chunked_lse(cdev["q"], cdev["k_ctx"], cdev["k_new"], w.G,
                                       w.n_prompt, chunk, scale=scale)
        csc = kvq.kvscore_chunked_colmax(cdev["q"], cdev["k_ctx"], clse, w.G, w.n_prompt,
                                         chunk, scale=scale).cpu().numpy()
        for l in range(w.L):
            for h in range(w.H):
                q, kc, kn = oracle.workload_head_inputs(
                    {k: cgen[k][l, h] for k in ("q", "k_ctx", "k_new")})
                S, _ = oracle.chunked_head_scores(q, kc, kn, scale, w.n_prompt, chunk, w.G)
                check_scores(csc[l, h], S, f"chunked scores[{l},{h}]")
