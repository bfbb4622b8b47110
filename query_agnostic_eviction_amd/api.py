"""Python binding of libkvq: the C entry points under the same names, taking
torch tensors.  Argument marshalling only - every step runs in the HIP
kernels of libkvq.so; torch supplies device memory and the current stream.

Shapes follow the KVzip page's notation ("KVzip: Query-Agnostic KV Cache
Compression with Context Reconstruction", sections 2.1 and 3.2):
    q      bf16 [L, H, G, n_in, d]     k_ctx, v_ctx  bf16 [L, H, n_c, d]
    k_new  bf16 [L, H, n_in, d]        lse  fp32 [L, H, G, n_in]
    scores fp32 [L, H, n_c]            offsets int64 [L*H + 1], idx int32
"""
from __future__ import annotations

import ctypes
from typing import Optional, Tuple

import torch

from . import _lib


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        lib = _lib.load()
        name = lib.kv_status_string(status).decode()
        extra = ""
        if status == _lib.KV_ERR_HIP:
            extra = f" (hipError {lib.kv_last_hip_error()})"
        super().__init__(f"{fn} failed: {name}{extra}")
        self.status = status


def _check(fn: str, status: int) -> None:
    if status != _lib.KV_OK:
        raise KvqError(fn, status)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _size(t: torch.Tensor, n: int, name: str) -> None:
    """A caller-supplied output must hold at least the n elements the kernel
    writes (checked before anything is enqueued)."""
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, {n} needed")


def _dev(t: torch.Tensor, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------------------
# host helpers
# ---------------------------------------------------------------------------
def kv_status_string(status: int) -> str:
    return _lib.load().kv_status_string(status).decode()


def kv_keep_count(n: int, keep_ratio: float) -> int:
    out = ctypes.c_int64()
    _check("kv_keep_count", _lib.load().kv_keep_count(n, keep_ratio, ctypes.byref(out)))
    return out.value


def kv_topk_total(L: int, H: int, n_c: int, keep_ratio: float, mode: int) -> int:
    out = ctypes.c_int64()
    _check("kv_topk_total",
           _lib.load().kv_topk_total(L, H, n_c, keep_ratio, mode, ctypes.byref(out)))
    return out.value


def kv_topk_workspace_bytes(L: int, H: int, n_c: int, mode: int) -> int:
    return int(_lib.load().kv_topk_workspace_bytes(L, H, n_c, mode))


# ---------------------------------------------------------------------------
# device entry points
# ---------------------------------------------------------------------------
def _score_dims(q, k_ctx):
    if q.dim() != 5 or k_ctx.dim() != 4:
        raise ValueError("q must be [L,H,G,n_in,d] and k_ctx [L,H,n_c,d]")
    L, H, G, n_in, d = q.shape
    n_c = k_ctx.shape[2]
    if tuple(k_ctx.shape) != (L, H, n_c, d) or n_in < n_c:
        raise ValueError("q / k_ctx shapes disagree")
    return L, H, G, d, n_c, n_in - n_c


def kvscore_lse(q: torch.Tensor, k_ctx: torch.Tensor, k_new: torch.Tensor,
                lse: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                stream=None) -> torch.Tensor:
    """Pass 1: lse[l,h,g,i] over cached keys and causal new keys."""
    _dev(q, torch.bfloat16, "q")
    _dev(k_ctx, torch.bfloat16, "k_ctx")
    _dev(k_new, torch.bfloat16, "k_new")
    L, H, G, d, n_c, n_prompt = _score_dims(q, k_ctx)
    if tuple(k_new.shape) != (L, H, n_c + n_prompt, d):
        raise ValueError("k_new must be [L,H,n_in,d]")
    if lse is None:
        lse = torch.empty((L, H, G, n_c + n_prompt), dtype=torch.float32, device=q.device)
    _dev(lse, torch.float32, "lse")
    _size(lse, L * H * G * (n_c + n_prompt), "lse")
    if scale is None:
        scale = 0.0   # the library's default, float32(1 / sqrt(d))
    _check("kvscore_lse", _lib.load().kvscore_lse(
        _ptr(q), _ptr(k_ctx), _ptr(k_new), _ptr(lse), L, H, G, d, n_c, n_prompt,
        float(scale), _stream(stream)))
    return lse


def kvscore_colmax(q: torch.Tensor, k_ctx: torch.Tensor, lse: torch.Tensor,
                   scores: Optional[torch.Tensor] = None,
                   scale: Optional[float] = None, stream=None) -> torch.Tensor:
    """Pass 2: scores[l,h,j] = max_{g,i} exp(scale q.k_j - lse)."""
    _dev(q, torch.bfloat16, "q")
    _dev(k_ctx, torch.bfloat16, "k_ctx")
    _dev(lse, torch.float32, "lse")
    L, H, G, d, n_c, n_prompt = _score_dims(q, k_ctx)
    if tuple(lse.shape) != (L, H, G, n_c + n_prompt):
        raise ValueError("lse must be [L,H,G,n_in]")
    if scores is None:
        scores = torch.empty((L, H, n_c), dtype=torch.float32, device=q.device)
    _dev(scores, torch.float32, "scores")
    _size(scores, L * H * n_c, "scores")
    if scale is None:
        scale = 0.0   # the library's default, float32(1 / sqrt(d))
    _check("kvscore_colmax", _lib.load().kvscore_colmax(
        _ptr(q), _ptr(k_ctx), _ptr(lse), _ptr(scores), L, H, G, d, n_c, n_prompt,
        float(scale), _stream(stream)))
    return scores


def kv_chunk_layout(n_c: int, n_prompt: int, chunk: int) -> Tuple[int, int]:
    """(n_chunks, rows per (l, h)) of the packed chunked layouts."""
    nch, rows = ctypes.c_int64(), ctypes.c_int64()
    _check("kv_chunk_layout", _lib.load().kv_chunk_layout(
        n_c, n_prompt, chunk, ctypes.byref(nch), ctypes.byref(rows)))
    return nch.value, rows.value


def _chunked_dims(q, k_ctx, k_new, G, n_prompt, chunk):
    if q.dim() != 4 or k_ctx.dim() != 4 or k_new.dim() != 4:
        raise ValueError("q [L,H,rows*G,d], k_ctx [L,H,n_c,d], k_new [L,H,rows,d]")
    L, H, n_c, d = k_ctx.shape
    _, rows = kv_chunk_layout(n_c, n_prompt, chunk)
    if tuple(q.shape) != (L, H, rows * G, d) or tuple(k_new.shape) != (L, H, rows, d):
        raise ValueError("chunked q / k_new shapes disagree with the chunk layout")
    return L, H, d, n_c, rows


def kvscore_chunked_lse(q, k_ctx, k_new, G: int, n_prompt: int, chunk: int,
                        lse=None, scale=None, stream=None):
    """Pass 1 of chunked scoring (packed chunk layout, see kvq.h)."""
    for t, n in ((q, "q"), (k_ctx, "k_ctx"), (k_new, "k_new")):
        _dev(t, torch.bfloat16, n)
    L, H, d, n_c, rows = _chunked_dims(q, k_ctx, k_new, G, n_prompt, chunk)
    if lse is None:
        lse = torch.empty((L, H, rows * G), dtype=torch.float32, device=q.device)
    _dev(lse, torch.float32, "lse")
    if tuple(lse.shape) != (L, H, rows * G):
        raise ValueError("lse must be [L,H,rows*G]")
    if scale is None:
        scale = 0.0   # the library's default, float32(1 / sqrt(d))
    _check("kvscore_chunked_lse", _lib.load().kvscore_chunked_lse(
        _ptr(q), _ptr(k_ctx), _ptr(k_new), _ptr(lse), L, H, G, d, n_c, n_prompt,
        chunk, float(scale), _stream(stream)))
    return lse


def kvscore_chunked_colmax(q, k_ctx, lse, G: int, n_prompt: int, chunk: int,
                           scores=None, scale=None, stream=None):
    """Pass 2 of chunked scoring; scores come out as [L,H,n_c]."""
    _dev(q, torch.bfloat16, "q")
    _dev(k_ctx, torch.bfloat16, "k_ctx")
    _dev(lse, torch.float32, "lse")
    L, H, n_c, d = k_ctx.shape
    _, rows = kv_chunk_layout(n_c, n_prompt, chunk)
    if tuple(q.shape) != (L, H, rows * G, d) or tuple(lse.shape) != (L, H, rows * G):
        raise ValueError("chunked q / lse shapes disagree with the chunk layout")
    if scores is None:
        scores = torch.empty((L, H, n_c), dtype=torch.float32, device=q.device)
    _dev(scores, torch.float32, "scores")
    _size(scores, L * H * n_c, "scores")
    if scale is None:
        scale = 0.0   # the library's default, float32(1 / sqrt(d))
    _check("kvscore_chunked_colmax", _lib.load().kvscore_chunked_colmax(
        _ptr(q), _ptr(k_ctx), _ptr(lse), _ptr(scores), L, H, G, d, n_c, n_prompt,
        chunk, float(scale), _stream(stream)))
    return scores


def kv_topk_select(scores: torch.Tensor, keep_ratio: float, mode: int = 0,
                   offsets: Optional[torch.Tensor] = None,
                   idx: Optional[torch.Tensor] = None,
                   stream=None,
                   workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Kept positions, CSR form: budget per head (mode 0), per layer (mode 1)
    or over the whole model (mode 2)."""
    _dev(scores, torch.float32, "scores")
    if scores.dim() != 3:
        raise ValueError("scores must be [L,H,n_c]")
    L, H, n_c = scores.shape
    total = kv_topk_total(L, H, n_c, keep_ratio, mode)
    if offsets is None:
        offsets = torch.empty(L * H + 1, dtype=torch.int64, device=scores.device)
    if idx is None:
        idx = torch.empty(total, dtype=torch.int32, device=scores.device)
    _dev(offsets, torch.int64, "offsets")
    _dev(idx, torch.int32, "idx")
    _size(offsets, L * H + 1, "offsets")
    ws_bytes = kv_topk_workspace_bytes(L, H, n_c, mode)
    ws = None
    if ws_bytes:
        if workspace is not None:
            _dev(workspace, torch.uint8, "workspace")
            if workspace.numel() < ws_bytes:
                raise ValueError("workspace too small")
            ws = workspace
        else:
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=scores.device)
    _check("kv_topk_select", _lib.load().kv_topk_select(
        _ptr(scores), L, H, n_c, float(keep_ratio), mode, _ptr(offsets), _ptr(idx),
        idx.numel(), _ptr(ws), ws_bytes, _stream(stream)))
    return offsets, idx


def kv_topk_select_noalloc(scores: torch.Tensor, keep_ratio: float, mode: int,
                           offsets: torch.Tensor, idx: torch.Tensor,
                           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """kv_topk_select without a workspace and without allocating: the caller
    passes the outputs; mode 2 uses the library's own per-GPU device array."""
    _dev(scores, torch.float32, "scores")
    if scores.dim() != 3:
        raise ValueError("scores must be [L,H,n_c]")
    L, H, n_c = scores.shape
    _dev(offsets, torch.int64, "offsets")
    _dev(idx, torch.int32, "idx")
    _size(offsets, L * H + 1, "offsets")
    _check("kv_topk_select_noalloc", _lib.load().kv_topk_select_noalloc(
        _ptr(scores), L, H, n_c, float(keep_ratio), mode, _ptr(offsets), _ptr(idx),
        idx.numel(), _stream(stream)))
    return offsets, idx


def kv_head_scores(scores: torch.Tensor, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Head-level static score (KVzip section 4.2): max of each head's scores."""
    _dev(scores, torch.float32, "scores")
    if scores.dim() != 3:
        raise ValueError("scores must be [L,H,n_c]")
    L, H, n_c = scores.shape
    if out is None:
        out = torch.empty((L, H), dtype=torch.float32, device=scores.device)
    _dev(out, torch.float32, "out")
    if out.numel() != L * H:
        raise ValueError("out must hold L*H entries")
    _check("kv_head_scores", _lib.load().kv_head_scores(
        _ptr(scores), L, H, n_c, _ptr(out), _stream(stream)))
    return out


def kv_compact(k_ctx: torch.Tensor, v_ctx: torch.Tensor, offsets: torch.Tensor,
               idx: torch.Tensor, k_out: Optional[torch.Tensor] = None,
               v_out: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gather the kept rows of K and V (bit copies)."""
    _dev(k_ctx, torch.bfloat16, "k_ctx")
    _dev(v_ctx, torch.bfloat16, "v_ctx")
    _dev(offsets, torch.int64, "offsets")
    _dev(idx, torch.int32, "idx")
    if k_ctx.dim() != 4 or v_ctx.shape != k_ctx.shape:
        raise ValueError("k_ctx / v_ctx must both be [L,H,n_c,d]")
    L, H, n_c, d = k_ctx.shape
    if offsets.numel() != L * H + 1:
        raise ValueError("offsets must hold L*H+1 entries")
    # the rows idx and the outputs hold: the kept count offsets[L*H] (on the
    # device) or more; the library writes only the kept rows
    total = idx.numel()
    if k_out is None:
        k_out = torch.empty((total, d), dtype=torch.bfloat16, device=k_ctx.device)
    if v_out is None:
        v_out = torch.empty((total, d), dtype=torch.bfloat16, device=k_ctx.device)
    _dev(k_out, torch.bfloat16, "k_out")
    _dev(v_out, torch.bfloat16, "v_out")
    _size(k_out, total * d, "k_out")
    _size(v_out, total * d, "v_out")
    _check("kv_compact", _lib.load().kv_compact(
        _ptr(k_ctx), _ptr(v_ctx), _ptr(offsets), _ptr(idx), _ptr(k_out), _ptr(v_out),
        L, H, d, n_c, total, _stream(stream)))
    return k_out, v_out


def kv_copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> torch.Tensor:
    """Plain streaming copy of src's bytes into dst (the HBM reference the
    compaction is read against)."""
    for t, n in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{n} must be a contiguous GPU tensor")
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    _check("kv_copy", _lib.load().kv_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))
    return dst


def kv_merge_compact(k_ctx: torch.Tensor, v_ctx: torch.Tensor, offsets: torch.Tensor,
                     idx: torch.Tensor, src_offsets: torch.Tensor, src_idx: torch.Tensor,
                     k_out: Optional[torch.Tensor] = None,
                     v_out: Optional[torch.Tensor] = None,
                     gate: Optional[torch.Tensor] = None,
                     mass: Optional[torch.Tensor] = None, stream=None):
    """SelKV soft cosine gate and gated merge of routed tokens into the kept
    rows: returns (k_out, v_out, gate, mass)."""
    _dev(k_ctx, torch.bfloat16, "k_ctx")
    _dev(v_ctx, torch.bfloat16, "v_ctx")
    for t, name, dt in ((offsets, "offsets", torch.int64), (idx, "idx", torch.int32),
                        (src_offsets, "src_offsets", torch.int64),
                        (src_idx, "src_idx", torch.int32)):
        _dev(t, dt, name)
    if k_ctx.dim() != 4 or v_ctx.shape != k_ctx.shape:
        raise ValueError("k_ctx / v_ctx must both be [L,H,n_c,d]")
    L, H, n_c, d = k_ctx.shape
    total, n_src = idx.numel(), src_idx.numel()
    if offsets.numel() != L * H + 1 or src_offsets.numel() != total + 1:
        raise ValueError("offsets must hold L*H+1 and src_offsets total+1 entries")
    dev = k_ctx.device
    k_out = torch.empty((total, d), dtype=torch.bfloat16, device=dev) if k_out is None else k_out
    v_out = torch.empty((total, d), dtype=torch.bfloat16, device=dev) if v_out is None else v_out
    gate = torch.empty(n_src, dtype=torch.float32, device=dev) if gate is None else gate
    mass = torch.empty(total, dtype=torch.float32, device=dev) if mass is None else mass
    for t, name, dt, n in ((k_out, "k_out", torch.bfloat16, total * d),
                           (v_out, "v_out", torch.bfloat16, total * d),
                           (gate, "gate", torch.float32, n_src),
                           (mass, "mass", torch.float32, total)):
        _dev(t, dt, name)
        if t.numel() < n:
            raise ValueError(f"{name} too small")
    _check("kv_merge_compact", _lib.load().kv_merge_compact(
        _ptr(k_ctx), _ptr(v_ctx), _ptr(offsets), _ptr(idx), _ptr(src_offsets), _ptr(src_idx),
        _ptr(k_out), _ptr(v_out), _ptr(gate), _ptr(mass), L, H, d, n_c, total, n_src,
        _stream(stream)))
    return k_out, v_out, gate, mass


# ---------------------------------------------------------------------------
# attention-free token score (EpiKV page, section 3.2)
# ---------------------------------------------------------------------------
def kv_epi_deltas(h: torch.Tensor, g: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Eq. 1: g[l][t] = ||h[l][t] - h[l][t-1]||_2 (g[l][0] = 0); h bf16 [n_layers,n,D]."""
    _dev(h, torch.bfloat16, "h")
    if h.dim() != 3:
        raise ValueError("h must be [n_layers, n, D]")
    nl, n, D = h.shape
    if g is None:
        g = torch.empty((nl, n), dtype=torch.float32, device=h.device)
    _dev(g, torch.float32, "g")
    if g.numel() != nl * n:
        raise ValueError("g must hold n_layers*n entries")
    _check("kv_epi_deltas", _lib.load().kv_epi_deltas(_ptr(h), nl, n, D, _ptr(g),
                                                      _stream(stream)))
    return g


def kv_epi_scores(g: torch.Tensor, n_a: int, window: int = 64, eps: float = 1e-6,
                  detrend: bool = True, scores: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Eq. 3 (detrend) or eq. 2: band A (rows 0..n_a-1 of g) minus band B."""
    _dev(g, torch.float32, "g")
    if g.dim() != 2 or not 1 <= n_a < g.shape[0]:
        raise ValueError("g must be [n_a + n_b, n] with both bands non-empty")
    nl, n = g.shape
    if scores is None:
        scores = torch.empty(n, dtype=torch.float32, device=g.device)
    _dev(scores, torch.float32, "scores")
    if scores.numel() != n:
        raise ValueError("scores must hold n entries")
    _check("kv_epi_scores", _lib.load().kv_epi_scores(
        _ptr(g), n_a, nl - n_a, n, window, float(eps), int(bool(detrend)), _ptr(scores),
        _stream(stream)))
    return scores


def kv_select_tokens_workspace_bytes(n: int) -> int:
    return int(_lib.load().kv_select_tokens_workspace_bytes(n))


def kv_select_tokens(scores: torch.Tensor, k: int, idx: Optional[torch.Tensor] = None,
                     stream=None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The k highest of n signed scores, ties to the lower position, ascending."""
    _dev(scores, torch.float32, "scores")
    n = scores.numel()
    if idx is None:
        idx = torch.empty(k, dtype=torch.int32, device=scores.device)
    _dev(idx, torch.int32, "idx")
    if idx.numel() < k:
        raise ValueError("idx too small")
    ws_bytes = kv_select_tokens_workspace_bytes(n)
    if workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=scores.device)
    _dev(workspace, torch.uint8, "workspace")
    if workspace.numel() < ws_bytes:
        raise ValueError("workspace too small")
    _check("kv_select_tokens", _lib.load().kv_select_tokens(
        _ptr(scores), n, k, _ptr(idx), _ptr(workspace), workspace.numel(), _stream(stream)))
    return idx


def kv_compact_tokens(k_cache: torch.Tensor, v_cache: torch.Tensor, idx: torch.Tensor,
                      k_out: Optional[torch.Tensor] = None,
                      v_out: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """The same kept positions in every (layer, head): [L,H,n,d] -> [L,H,k,d]."""
    _dev(k_cache, torch.bfloat16, "k_cache")
    _dev(v_cache, torch.bfloat16, "v_cache")
    _dev(idx, torch.int32, "idx")
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must both be [L,H,n,d]")
    L, H, n, d = k_cache.shape
    k = idx.numel()
    shape = (L, H, k, d)
    if k_out is None:
        k_out = torch.empty(shape, dtype=torch.bfloat16, device=k_cache.device)
    if v_out is None:
        v_out = torch.empty(shape, dtype=torch.bfloat16, device=k_cache.device)
    _dev(k_out, torch.bfloat16, "k_out")
    _dev(v_out, torch.bfloat16, "v_out")
    if k_out.numel() < L * H * k * d or v_out.numel() < L * H * k * d:
        raise ValueError("k_out / v_out too small")
    _check("kv_compact_tokens", _lib.load().kv_compact_tokens(
        _ptr(k_cache), _ptr(v_cache), _ptr(idx), _ptr(k_out), _ptr(v_out), L, H, d, n, k,
        _stream(stream)))
    return k_out, v_out


def epikv_evict(h: torch.Tensor, n_a: int, k_cache: torch.Tensor, v_cache: torch.Tensor,
                budget: int, window: int = 64, eps: float = 1e-6, detrend: bool = True,
                stream=None):
    """Hidden-state deltas, band scores, top-`budget` tokens, token compaction:
    returns (k_out, v_out, idx, scores, g)."""
    g = kv_epi_deltas(h, stream=stream)
    scores = kv_epi_scores(g, n_a, window, eps, detrend, stream=stream)
    idx = kv_select_tokens(scores, budget, stream=stream)
    k_out, v_out = kv_compact_tokens(k_cache, v_cache, idx, stream=stream)
    return k_out, v_out, idx, scores, g


# ---------------------------------------------------------------------------
# the whole path
# ---------------------------------------------------------------------------
def score(q, k_ctx, k_new, scale=None, stream=None):
    """(scores, lse) of every cached key: pass 1 then pass 2."""
    lse = kvscore_lse(q, k_ctx, k_new, scale=scale, stream=stream)
    scores = kvscore_colmax(q, k_ctx, lse, scale=scale, stream=stream)
    return scores, lse


def score_chunked(q, k_ctx, k_new, G, n_prompt, chunk, scale=None, stream=None):
    """(scores, lse) of chunked scoring (KVzip section 3.4)."""
    lse = kvscore_chunked_lse(q, k_ctx, k_new, G, n_prompt, chunk, scale=scale, stream=stream)
    scores = kvscore_chunked_colmax(q, k_ctx, lse, G, n_prompt, chunk, scale=scale,
                                    stream=stream)
    return scores, lse


def select(scores, keep_ratio, mode=0, stream=None):
    """(offsets, idx) of the kept pairs (kv_topk_select)."""
    return kv_topk_select(scores, keep_ratio, mode, stream=stream)


def compact(k_ctx, v_ctx, offsets, idx, stream=None):
    """(k_out, v_out): the kept rows (kv_compact)."""
    return kv_compact(k_ctx, v_ctx, offsets, idx, stream=stream)


def evict(q, k_ctx, k_new, v_ctx, keep_ratio, mode=0, scale=None, stream=None):
    """Score, select and compact: returns (k_out, v_out, offsets, idx, scores)."""
    scores, _ = score(q, k_ctx, k_new, scale=scale, stream=stream)
    offsets, idx = kv_topk_select(scores, keep_ratio, mode, stream=stream)
    k_out, v_out = kv_compact(k_ctx, v_ctx, offsets, idx, stream=stream)
    return k_out, v_out, offsets, idx, scores
