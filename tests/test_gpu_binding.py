"""The binding refuses caller-supplied outputs that are too small for what
the kernels write, before anything is enqueued (a short buffer would
otherwise be written past its end)."""
import pytest
import torch

import query_agnostic_eviction_amd as kvq

pytestmark = pytest.mark.gpu


def test_undersized_outputs_are_rejected():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print("undersized-output checks", flush=True)
    dev = "cuda"
    L, H, G, d, n_c, n_p = 1, 2, 2, 64, 40, 3
    n_in = n_c + n_p
    q = torch.zeros((L, H, G, n_in, d), dtype=torch.bfloat16, device=dev)
    kc = torch.zeros((L, H, n_c, d), dtype=torch.bfloat16, device=dev)
    kn = torch.zeros((L, H, n_in, d), dtype=torch.bfloat16, device=dev)
    f32 = lambda n: torch.zeros(n, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="lse"):
        kvq.kvscore_lse(q, kc, kn, lse=f32(L * H * G * n_in - 1))
    lse = kvq.kvscore_lse(q, kc, kn)
    with pytest.raises(ValueError, match="scores"):
        kvq.kvscore_colmax(q, kc, lse, scores=f32(L * H * n_c - 1))
    scores = kvq.kvscore_colmax(q, kc, lse)
    # chunked layout, chunk 16: three chunks of 16, 16 and 8 keys
    n_ch, rows = kvq.kv_chunk_layout(n_c, n_p, 16)
    qc = torch.zeros((L, H, rows * G, d), dtype=torch.bfloat16, device=dev)
    knc = torch.zeros((L, H, rows, d), dtype=torch.bfloat16, device=dev)
    lsec = kvq.kvscore_chunked_lse(qc, kc, knc, G, n_p, 16)
    with pytest.raises(ValueError, match="scores"):
        kvq.kvscore_chunked_colmax(qc, kc, lsec, G, n_p, 16, scores=f32(L * H * n_c - 1))
    with pytest.raises(ValueError, match="offsets"):
        kvq.kv_topk_select(scores, 0.5, 0,
                           offsets=torch.zeros(L * H, dtype=torch.int64, device=dev))
    offsets, idx = kvq.kv_topk_select(scores, 0.5, 0)
    total = idx.numel()
    vc = torch.zeros_like(kc)
    narrow = torch.zeros((total, d // 2), dtype=torch.bfloat16, device=dev)  # rows ok, too few elements
    with pytest.raises(ValueError, match="k_out"):
        kvq.kv_compact(kc, vc, offsets, idx, k_out=narrow)
    with pytest.raises(ValueError, match="v_out"):
        kvq.kv_compact(kc, vc, offsets, idx, v_out=narrow)
    # properly sized outputs still work
    ko, vo = kvq.kv_compact(kc, vc, offsets, idx)
    torch.cuda.synchronize()
    assert ko.shape == (total, d) and vo.shape == (total, d)


def test_empty_kept_sets():
    """An empty kept set is a valid request: the calls return empty outputs
    (empty tensors may carry a null data pointer) and enqueue nothing."""
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print("empty kept sets", flush=True)
    dev = "cuda"
    L, H, n_c, d = 2, 3, 50, 128
    kc = torch.randn((L, H, n_c, d), device=dev).to(torch.bfloat16)
    vc = torch.randn((L, H, n_c, d), device=dev).to(torch.bfloat16)
    offsets = torch.zeros(L * H + 1, dtype=torch.int64, device=dev)
    idx = torch.empty(0, dtype=torch.int32, device=dev)
    ko, vo = kvq.kv_compact(kc, vc, offsets, idx)
    assert ko.shape == (0, d) and vo.shape == (0, d)
    src_offsets = torch.zeros(1, dtype=torch.int64, device=dev)
    ko, vo, gate, mass = kvq.kv_merge_compact(kc, vc, offsets, idx, src_offsets, idx)
    assert ko.shape == (0, d) and gate.numel() == 0 and mass.numel() == 0
    ko, vo = kvq.kv_compact_tokens(kc, vc, idx)
    assert ko.shape == (L, H, 0, d) and vo.shape == (L, H, 0, d)
    # the library's state is untouched: a real compaction right after still matches
    keep = torch.tensor([0, 7, 49], dtype=torch.int32, device=dev)
    ko, vo = kvq.kv_compact_tokens(kc, vc, keep)
    torch.cuda.synchronize()
    assert torch.equal(ko, kc[:, :, keep.long()]) and torch.equal(vo, vc[:, :, keep.long()])


def test_compact_with_spare_capacity():
    """idx and the outputs may hold more rows than the kept set: the kept rows
    are gathered bit for bit and the rows past offsets[L*H] stay untouched
    (KVzip page, section 2.1: KV_p is a subset of KV_c)."""
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print("compaction with spare capacity", flush=True)
    dev = "cuda"
    L, H, n_c, d, keep = 2, 3, 300, 128, 0.2
    g = torch.Generator(device=dev).manual_seed(5)
    kc = torch.randn((L, H, n_c, d), device=dev, generator=g).to(torch.bfloat16)
    vc = torch.randn((L, H, n_c, d), device=dev, generator=g).to(torch.bfloat16)
    scores = torch.rand((L, H, n_c), device=dev, generator=g)
    total = kvq.kv_topk_total(L, H, n_c, keep, 1)
    spare = 37
    offsets = torch.empty(L * H + 1, dtype=torch.int64, device=dev)
    idx = torch.full((total + spare,), 12345, dtype=torch.int32, device=dev)  # garbage past the set
    kvq.kv_topk_select(scores, keep, 1, offsets, idx[:total])
    sentinel = torch.full((total + spare, d), -3.0, dtype=torch.bfloat16, device=dev)
    ko, vo = sentinel.clone(), sentinel.clone()
    kvq.kv_compact(kc, vc, offsets, idx, ko, vo)
    torch.cuda.synchronize()
    off = offsets.cpu().tolist()
    assert off[-1] == total
    ix = idx.cpu()
    for lh in range(L * H):
        l, h = divmod(lh, H)
        rows = ix[off[lh]:off[lh + 1]].long()
        assert torch.equal(ko[off[lh]:off[lh + 1]], kc[l, h][rows.to(dev)])
        assert torch.equal(vo[off[lh]:off[lh + 1]], vc[l, h][rows.to(dev)])
    assert torch.equal(ko[total:], sentinel[total:]) and torch.equal(vo[total:], sentinel[total:])


def test_default_scale_is_float32_inverse_sqrt_d():
    """scale omitted (0 at the C ABI) equals passing float32(1 / sqrt(d))."""
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print("default scale", flush=True)
    import numpy as np
    dev = "cuda"
    for d in (64, 128, 256):
        L, H, G, n_c, n_p = 1, 2, 2, 200, 5
        g = torch.Generator(device=dev).manual_seed(d)
        q = torch.randn((L, H, G, n_c + n_p, d), device=dev, generator=g).to(torch.bfloat16)
        kc = torch.randn((L, H, n_c, d), device=dev, generator=g).to(torch.bfloat16)
        kn = torch.randn((L, H, n_c + n_p, d), device=dev, generator=g).to(torch.bfloat16)
        s_def, l_def = kvq.score(q, kc, kn)
        s_exp, l_exp = kvq.score(q, kc, kn, scale=float(np.float32(1.0 / np.sqrt(d))))
        torch.cuda.synchronize()
        assert torch.equal(s_def, s_exp) and torch.equal(l_def, l_exp)
