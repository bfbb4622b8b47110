"""The stored whole-head oracle values of the 128K workload (CPU only):
tests/golden/llama3.1-8b-128k_head{l}-{h}.npz, written by
tests/golden/make_llama128k_head.py from the seeded inputs and the float64
oracle (KVzip page, "KVzip: Query-Agnostic KV Cache Compression with Context
Reconstruction", section 3.2), and used by the GPU full-size parity test."""
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("l,h", [(0, 0), (31, 7)])
def test_golden_128k_heads_rederived(l, h):
    """The stored whole-head values of the 128K workload (first and last head)
    are the oracle's: sampled rows' lse re-derived from the seeded inputs with
    the scalar-row oracle, and the stored scores obey what a score must (in
    (0, 1]; exact copies of a key, the repeated spans, score identically)."""
    w = synth.LLAMA8B_128K
    gold = np.load(os.path.join(GOLDEN, f"llama3.1-8b-128k_head{l}-{h}.npz"))
    assert (int(gold["layer"]), int(gold["head"]), str(gold["workload"])) == (l, h, w.name)
    q, kc, kn = oracle.workload_head_inputs(synth.generate_head(w, l, h))
    rng = np.random.default_rng(l * 8 + h)
    rows = [(0, 0), (w.G - 1, 16 * ((w.n_in - 1) // 16))]
    rows += [(int(rng.integers(w.G)), 16 * int(rng.integers(w.n_in // 16))) for _ in range(4)]
    for (g, i) in rows:
        want = oracle.row_lse(q[g, i], i, kc, kn, float(w.scale))
        got = float(gold["lse_rows16"][g, i // 16])
        assert abs(got - want) <= 4e-7 * abs(want), (g, i, got, want)
    S = gold["scores"].astype(np.float64)
    assert S.shape == (w.n_c,) and np.all(S > 0) and np.all(S <= 1)
    span = np.arange(64, 128)
    for kk in (1, 15, 31):
        assert np.array_equal(S[4096 * kk + span], S[span])
