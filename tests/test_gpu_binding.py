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
