"""GPU: kv_topk_select_noalloc (the allocation-free selection, for callers
that cannot allocate device memory) against kv_topk_select on the same
scores, through the C ABI.  Index work, so bit-exact: offsets and kept
positions must be identical.  Two calls in a row, the second on a smaller
input, so that state the first call left in the library's device array
cannot leak into the second; and the float64 oracle's selection (KVzip page,
"KVzip: Query-Agnostic KV Cache Compression with Context Reconstruction",
section 4.1) as a third witness on the smaller case.
"""
import numpy as np
import pytest
import torch

import oracle
import query_agnostic_eviction_amd as kvq

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _scores(L, H, n_c, seed, ties):
    """Seeded non-negative scores; with ties, values on a coarse grid so that
    many scores are equal and the lower-index rule decides."""
    rng = np.random.default_rng(seed)
    s = rng.random((L, H, n_c), dtype=np.float32)
    if ties:
        s = np.floor(s * 64.0).astype(np.float32) / 64.0
    return s


def _both(s_host, keep, mode):
    L, H, n_c = s_host.shape
    sc = torch.from_numpy(s_host).cuda()
    total = kvq.kv_topk_total(L, H, n_c, keep, mode)
    off_a, idx_a = kvq.kv_topk_select(sc, keep, mode)
    off_b = torch.full((L * H + 1,), -7, dtype=torch.int64, device="cuda")
    idx_b = torch.full((total,), -7, dtype=torch.int32, device="cuda")
    kvq.kv_topk_select_noalloc(sc, keep, mode, off_b, idx_b)
    torch.cuda.synchronize()
    return (off_a.cpu().numpy(), idx_a.cpu().numpy(), off_b.cpu().numpy(),
            idx_b.cpu().numpy())


@pytest.mark.parametrize("mode", [2, 1, 0])
@pytest.mark.parametrize("ties", [False, True])
def test_noalloc_matches_select_twice(mode, ties):
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    # first a larger input (many workgroups of the grid-wide select), then a
    # smaller one with a different keep ratio
    for (L, H, n_c, keep, seed) in ((4, 8, 8192, 0.3, 11), (2, 3, 1000, 0.05, 12)):
        _say(f"noalloc select: mode {mode} ties {ties} L={L} H={H} n_c={n_c} keep={keep}")
        s = _scores(L, H, n_c, seed, ties)
        off_a, idx_a, off_b, idx_b = _both(s, keep, mode)
        assert np.array_equal(off_a, off_b)
        assert np.array_equal(idx_a, idx_b)
    # the smaller case against the oracle's selection on the same fp32 scores
    off_o, idx_o = oracle.select(s.astype(np.float64), keep, mode)
    assert np.array_equal(off_b, off_o)
    assert np.array_equal(idx_b, idx_o)


def test_noalloc_capacity_error_writes_nothing():
    L, H, n_c, keep = 1, 2, 512, 0.5
    sc = torch.from_numpy(_scores(L, H, n_c, 3, False)).cuda()
    total = kvq.kv_topk_total(L, H, n_c, keep, 2)
    off = torch.full((L * H + 1,), -7, dtype=torch.int64, device="cuda")
    idx = torch.full((total - 1,), -7, dtype=torch.int32, device="cuda")
    with pytest.raises(kvq.KvqError, match="KV_ERR_CAPACITY"):
        kvq.kv_topk_select_noalloc(sc, keep, 2, off, idx)
    torch.cuda.synchronize()
    assert bool((off == -7).all()) and bool((idx == -7).all())
