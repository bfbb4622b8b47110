"""Reentrancy: two different workloads run at the same time on two streams
(each with its own buffers and its own model-wide select workspace) give
exactly the results of running them one after the other.  The library keeps
no state between calls beyond what the caller's buffers hold, so concurrent
calls on different buffers cannot interfere."""
import pytest
import torch

import synth
import query_agnostic_eviction_amd as kvq
from parity_util import to_dev_bf16

pytestmark = pytest.mark.gpu


def _inputs(w):
    gen = synth.generate_workload(w, workers=1)
    return {k: to_dev_bf16(v) for k, v in gen.items()}


def _path(dev, r, stream):
    """Score, every budget mode, compaction and gated merge on `stream`;
    returns the outputs (all allocated on that stream)."""
    with torch.cuda.stream(stream):
        scores, lse = kvq.score(dev["q"], dev["k_ctx"], dev["k_new"], stream=stream)
        out = [lse, scores]
        for mode in (0, 1, 2):
            off, idx = kvq.kv_topk_select(scores, r, mode, stream=stream)
            ko, vo = kvq.kv_compact(dev["k_ctx"], dev["v_ctx"], off, idx, stream=stream)
            out += [off, idx, ko, vo]
        # token-level select of the flattened scores (signed path, own workspace)
        tok = kvq.kv_select_tokens(scores.reshape(-1) - 0.5, max(1, scores.numel() // 5),
                                   stream=stream)
        out.append(tok)
        hs = kvq.kv_head_scores(scores, stream=stream)
        out.append(hs)
    return out


def test_two_streams_match_sequential():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print("two-stream reentrancy", flush=True)
    wa = synth.TINY.shrink(L=2, H=3, n_c=3000, n_prompt=17, G=4, d=128, seed=11)
    wb = synth.TINY.shrink(L=3, H=2, n_c=2100, n_prompt=5, G=2, d=64, seed=12)
    da, db = _inputs(wa), _inputs(wb)
    s0 = torch.cuda.current_stream()
    seq_a = [t.clone() for t in _path(da, 0.3, s0)]
    seq_b = [t.clone() for t in _path(db, 0.15, s0)]
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(s0)
    sb.wait_stream(s0)
    for rep in range(3):
        par_a = _path(da, 0.3, sa)
        par_b = _path(db, 0.15, sb)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(seq_a, par_a)):
            assert torch.equal(x, y), (rep, "a", i)
        for i, (x, y) in enumerate(zip(seq_b, par_b)):
            assert torch.equal(x, y), (rep, "b", i)


def _chunked_path(dev, w, chunk, routes, stream):
    """Chunked scoring, per-(l, h) budget and the gated merge on `stream`."""
    with torch.cuda.stream(stream):
        scores, lse = kvq.score_chunked(dev["q"], dev["k_ctx"], dev["k_new"], w.G,
                                        w.n_prompt, chunk, stream=stream)
        off, idx = kvq.kv_topk_select(scores, w.keep_ratio, 0, stream=stream)
        so, si = routes
        ko, vo, gate, mass = kvq.kv_merge_compact(dev["k_ctx"], dev["v_ctx"], off, idx, so, si,
                                                  stream=stream)
    return [lse, scores, off, idx, ko, vo, gate, mass]


def test_two_streams_chunked_and_merge():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    print("two-stream reentrancy: chunked scoring and gated merge", flush=True)
    wa = synth.LLAMA8B_8K.shrink(L=2, H=2, n_c=2500, n_prompt=32, seed=21)
    wb = synth.LLAMA8B_8K.shrink(L=1, H=3, n_c=1800, n_prompt=7, G=2, d=64, rank=4, seed=22)
    ca, cb = 1024, 512
    da = {k: to_dev_bf16(v) for k, v in synth.generate_chunked_workload(wa, ca, workers=1).items()}
    db = {k: to_dev_bf16(v) for k, v in synth.generate_chunked_workload(wb, cb, workers=1).items()}
    s0 = torch.cuda.current_stream()
    routes = []
    for d_, w_, c_ in ((da, wa, ca), (db, wb, cb)):   # routing from the (deterministic) kept set
        sc, _ = kvq.score_chunked(d_["q"], d_["k_ctx"], d_["k_new"], w_.G, w_.n_prompt, c_)
        off, idx = kvq.kv_topk_select(sc, w_.keep_ratio, 0)
        so, si = synth.nearest_position_routes(off.cpu().numpy(), idx.cpu().numpy(), w_.n_c)
        routes.append((torch.from_numpy(so).cuda(), torch.from_numpy(si).cuda()))
    seq_a = [t.clone() for t in _chunked_path(da, wa, ca, routes[0], s0)]
    seq_b = [t.clone() for t in _chunked_path(db, wb, cb, routes[1], s0)]
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(s0)
    sb.wait_stream(s0)
    for rep in range(3):
        par_a = _chunked_path(da, wa, ca, routes[0], sa)
        par_b = _chunked_path(db, wb, cb, routes[1], sb)
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(seq_a, par_a)):
            assert torch.equal(x, y), (rep, "a", i)
        for i, (x, y) in enumerate(zip(seq_b, par_b)):
            assert torch.equal(x, y), (rep, "b", i)
