"""The path under HIP graph capture: one captured step of each path, replayed
several times with eager work and synchronisations between replays, every
replay bit-identical to the eager result.  No kernel of the library records a
memset (workspaces are cleared by its own kernels), so capture needs nothing
special beyond preallocated buffers."""
import numpy as np
import pytest
import torch

import synth
import query_agnostic_eviction_amd as kvq
from parity_util import to_dev_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    kvq.api._lib.load()
    yield
    torch.cuda.synchronize()


def _replay_and_check(step, outputs, reps=3):
    """Capture step() on a side stream, then replay it `reps` times, each
    after eager work that overwrites the outputs; compare with the eager run."""
    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        step()
    for r in range(reps):
        for o in outputs:            # eager work between replays
            o.zero_() if o.dtype != torch.bfloat16 else o.view(torch.int16).fill_(r + 1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, eager):
            a = o.view(torch.int16) if o.dtype == torch.bfloat16 else o
            b = e.view(torch.int16) if e.dtype == torch.bfloat16 else e
            assert torch.equal(a, b), f"replay {r} differs"


@pytest.mark.parametrize("mode", [0, 2])
def test_kvzip_path_graph_replay(mode):
    w = synth.LLAMA8B_8K.shrink(L=2, H=2, n_c=3000, n_prompt=32)
    gen = synth.generate_workload(w, workers=1)
    q, kc, kn, vc = (to_dev_bf16(gen[k]) for k in ("q", "k_ctx", "k_new", "v_ctx"))
    scale = float(w.scale)
    total = kvq.kv_topk_total(w.L, w.H, w.n_c, w.keep_ratio, mode)
    lse = torch.empty((w.L, w.H, w.G, w.n_in), dtype=torch.float32, device="cuda")
    sc = torch.empty((w.L, w.H, w.n_c), dtype=torch.float32, device="cuda")
    off = torch.empty(w.L * w.H + 1, dtype=torch.int64, device="cuda")
    idx = torch.empty(total, dtype=torch.int32, device="cuda")
    ko = torch.empty((total, w.d), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    ws = torch.empty(max(kvq.kv_topk_workspace_bytes(w.L, w.H, w.n_c, mode), 1),
                     dtype=torch.uint8, device="cuda")

    def step():
        st = torch.cuda.current_stream()
        kvq.kvscore_lse(q, kc, kn, lse, scale, st)
        kvq.kvscore_colmax(q, kc, lse, sc, scale, st)
        kvq.kv_topk_select(sc, w.keep_ratio, mode, off, idx, st, ws)
        kvq.kv_compact(kc, vc, off, idx, ko, vo, st)

    _replay_and_check(step, [lse, sc, off, idx, ko, vo])


def test_epikv_path_graph_replay():
    w = synth.EPIKV_TINY.shrink(n=3000, D=1024)
    hb = synth.generate_hidden(w)
    kb, vb = synth.generate_kv(w)
    h, kc, vc = to_dev_bf16(hb), to_dev_bf16(kb), to_dev_bf16(vb)
    g = torch.empty((2, w.n), dtype=torch.float32, device="cuda")
    sc = torch.empty(w.n, dtype=torch.float32, device="cuda")
    idx = torch.empty(w.budget, dtype=torch.int32, device="cuda")
    ws = torch.empty(kvq.kv_select_tokens_workspace_bytes(w.n), dtype=torch.uint8, device="cuda")
    ko = torch.empty((w.L, w.H, w.budget, w.d), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)

    def step():
        st = torch.cuda.current_stream()
        kvq.kv_epi_deltas(h, g, st)
        kvq.kv_epi_scores(g, 1, w.window, w.eps, True, sc, st)
        kvq.kv_select_tokens(sc, w.budget, idx, st, ws)
        kvq.kv_compact_tokens(kc, vc, idx, ko, vo, st)

    _replay_and_check(step, [g, sc, idx, ko, vo])


def test_chunked_and_merge_graph_replay():
    """Chunked scoring (two launches per pass: full chunks and the shorter
    last one), the per-(l, h) budget and the gated merge with routing built
    once on the host, captured as one step."""
    w = synth.LLAMA8B_8K.shrink(L=2, H=2, n_c=2500, n_prompt=32)
    chunk = 1024                       # chunks of 1024, 1024 and 452 keys
    gen = synth.generate_chunked_workload(w, chunk, workers=1)
    q, kc, kn, vc = (to_dev_bf16(gen[k]) for k in ("q", "k_ctx", "k_new", "v_ctx"))
    scale = float(w.scale)
    n_ch, rows = kvq.kv_chunk_layout(w.n_c, w.n_prompt, chunk)
    lse = torch.empty((w.L, w.H, rows * w.G), dtype=torch.float32, device="cuda")
    sc = torch.empty((w.L, w.H, w.n_c), dtype=torch.float32, device="cuda")
    total = kvq.kv_topk_total(w.L, w.H, w.n_c, w.keep_ratio, 0)
    off = torch.empty(w.L * w.H + 1, dtype=torch.int64, device="cuda")
    idx = torch.empty(total, dtype=torch.int32, device="cuda")
    # the kept set is deterministic: build the routing from one eager run
    kvq.kvscore_chunked_lse(q, kc, kn, w.G, w.n_prompt, chunk, lse, scale)
    kvq.kvscore_chunked_colmax(q, kc, lse, w.G, w.n_prompt, chunk, sc, scale)
    kvq.kv_topk_select(sc, w.keep_ratio, 0, off, idx)
    torch.cuda.synchronize()
    so_np, si_np = synth.nearest_position_routes(off.cpu().numpy(), idx.cpu().numpy(), w.n_c)
    so, si = torch.from_numpy(so_np).cuda(), torch.from_numpy(si_np).cuda()
    ko = torch.empty((total, w.d), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    gate = torch.empty(si.numel(), dtype=torch.float32, device="cuda")
    mass = torch.empty(total, dtype=torch.float32, device="cuda")

    def step():
        st = torch.cuda.current_stream()
        kvq.kvscore_chunked_lse(q, kc, kn, w.G, w.n_prompt, chunk, lse, scale, st)
        kvq.kvscore_chunked_colmax(q, kc, lse, w.G, w.n_prompt, chunk, sc, scale, st)
        kvq.kv_topk_select(sc, w.keep_ratio, 0, off, idx, st)
        kvq.kv_merge_compact(kc, vc, off, idx, so, si, ko, vo, gate, mass, st)

    _replay_and_check(step, [lse, sc, off, idx, ko, vo, gate, mass])
