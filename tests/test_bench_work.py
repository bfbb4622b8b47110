"""bench.py's algorithmic work (the numerator of its roofline figures) equals
the number of attention entries the method defines, counted on the oracle's
own materialised rows: pass 1 evaluates every logit a row sees, pass 2 every
logit of a cached-key column; chunked scoring counts each chunk's pass."""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import oracle  # noqa: E402
import synth  # noqa: E402


def _counted_logits(G, n_c, n_prompt, d, rng):
    """(pass-1 logits, pass-2 logits) of one (layer, KV head), counted as the
    nonzero entries of the oracle's attention rows on random inputs."""
    n_in = n_prompt + n_c
    q = rng.standard_normal((G, n_in, d))
    k_all = rng.standard_normal((n_c + n_in, d))
    seen = cached = 0
    for g in range(G):
        a, _ = oracle.attention_rows(q[g], np.arange(n_in), k_all, n_c, 0.1)
        seen += int(np.count_nonzero(a))
        cached += int(np.count_nonzero(a[:, :n_c]))
    return seen, cached


@pytest.mark.parametrize("G,d,n_c,n_prompt,chunk",
                         [(2, 8, 7, 3, None), (3, 16, 12, 0, None), (1, 8, 10, 2, 4),
                          (2, 8, 9, 1, 9), (2, 8, 9, 1, 20)])
def test_algorithmic_work_counts_the_defined_logits(G, d, n_c, n_prompt, chunk):
    rng = np.random.default_rng(5)
    w = synth.TINY.shrink(L=2, H=3, G=G, d=d, n_c=n_c, n_prompt=n_prompt)
    seen = cached = 0
    spans = oracle.chunk_bounds(n_c, chunk) if chunk else [(0, n_c)]
    for _start, m in spans:
        s1, s2 = _counted_logits(G, m, n_prompt, d, rng)
        seen += s1
        cached += s2
    work = bench.algorithmic_work(w, 0, chunk)
    heads = w.L * w.H
    assert work["lse_exps"] == seen * heads
    assert work["lse_flops"] == 2.0 * d * seen * heads
    assert work["colmax_flops"] == 2.0 * d * cached * heads
    # compaction moves each kept K and V row once each way, plus its index
    k = oracle.keep_count(n_c, w.keep_ratio)
    assert work["kept_rows"] == heads * k
    assert work["compact_bytes"] == heads * k * (2 * 2 * 2 * d + 4)


def _stage_limit():
    """The per-segment LDS staging limit of the top-k kernel, read from its
    source so that bench.py's byte count follows the kernel."""
    import re
    src = open(os.path.join(ROOT, "query_agnostic_eviction_amd", "csrc", "kv_topk.hip")).read()
    return int(re.search(r"constexpr int kTkStage = (\d+);", src).group(1))


@pytest.mark.parametrize("mode,H,n_c", [(0, 3, 8192), (0, 2, 40000), (1, 8, 4096), (1, 8, 4097),
                                        (2, 4, 100)])
def test_select_bytes_follow_the_staging_limit(mode, H, n_c):
    # a segment (a head in mode 0, a layer's H * n_c scores in mode 1) that
    # fits the LDS stage is read once; longer ones four times; the grid-wide
    # model budget (mode 2) five times
    lim = _stage_limit()
    w = synth.TINY.shrink(L=2, H=H, n_c=n_c)
    seg = n_c if mode == 0 else H * n_c
    reads = 5 if mode == 2 else (1 if seg <= lim else 4)
    heads = w.L * H
    total = bench.synth_total(w, mode)
    work = bench.algorithmic_work(w, mode)
    assert work["select_bytes"] == 4.0 * reads * heads * n_c + 4.0 * total + 8.0 * (heads + 1)
    if mode == 1:
        assert (seg <= lim) == (n_c == 4096)   # the two cases straddle the limit
