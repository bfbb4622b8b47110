"""Float64 CPU oracle for query-agnostic KV scoring, selection and compaction.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The library's product
path never calls it, and it shares no code with the GPU kernels.

What it computes, in the notation of the KVzip page ("KVzip: Query-Agnostic KV
Cache Compression with Context Reconstruction"):

* Section 2.1 (notation): L layers, H KV heads, G query heads per KV head;
  prefilling a context of n_c tokens caches L x H x n_c KV pairs (KV_c); the
  goal is a subset KV_p of KV_c.
* Section 3.2 (KV importance scoring): the input is the repeat prompt
  (n_prompt tokens) followed by the context, n_in = n_prompt + n_c positions,
  processed teacher-forced in one forward pass with KV_c as the prefix cache.
  For layer l and KV head h this yields grouped queries Q in R^{G x n_in x d}
  and keys K in R^{(n_c + n_in) x d} (the cached keys, then the n_in new
  keys).  A = Softmax(Q K^T) is G x n_in x (n_c + n_in); its slice to the
  n_c cached-key columns is A-bar; the score of cached key j is the maximum of
  A-bar[g, i, j] over all g and all n_in rows i (the displayed equation of
  that section).
* Section 3.4 (chunk-based scoring): each chunk of m context tokens is
  scored from its own repeat pass (prompt + that chunk), on an
  n_in x (m + n_in) attention over the chunk's cached keys and new keys.
* Section 4.1 (eviction structure): keep the r% highest-scoring KV pairs.

Readings taken where the page is silent:
  - the softmax logits carry the model's 1/sqrt(d) temperature; it is passed
    in as `scale` (the same float32 value the GPU receives);
  - the pass is causal over the new tokens: query row i (0-based) sees every
    cached key and new keys 0..i, its own key included;
  - every one of the n_in rows counts, prompt rows included;
  - the softmax is normalised over all keys a row sees (cached and new), and
    only then sliced to the cached columns;
  - the kept count is k = clamp(floor(r * n), 1, n) in IEEE double (the
    floor rule m = floor(rho * n) of the SelKV page, section 3.1);
  - ties go to the lower index (the flattened h * n_c + j across heads), and
    kept indices are returned in ascending position order;
  - the "across all heads" budget of section 4.1 is read per layer (mode 1)
    and over the whole model (mode 2); mode 0 keeps the same count in every
    (layer, KV head);
  - section 4.2's head-level score of a head is the largest of its pair
    scores along the sequence.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

ROW_SUM_TOL = 1e-12


# ----------------------------------------------------------------------------
# input conversion
# ----------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32)
    return (b << 16).view(np.float32).astype(np.float64)


# ----------------------------------------------------------------------------
# KVzip section 3.2: attention rows of the repeat pass, lse and max score
# ----------------------------------------------------------------------------
def visible_keys(n_c: int, i: int) -> int:
    """Number of keys query row i sees: all n_c cached keys plus new keys
    0..i (teacher-forced, causal over the new tokens, diagonal included)."""
    return n_c + i + 1


def attention_rows(q_rows: np.ndarray, pos: np.ndarray, k_all: np.ndarray,
                   n_c: int, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Materialise rows of A = Softmax(scale * Q K^T) for the given query rows.

    q_rows : (B, d) float64, one query vector per row
    pos    : (B,) int, the position i of each row in the n_in-long input
    k_all  : (n_c + n_in, d) float64, cached keys then new keys
    returns (A_rows (B, n_c + n_in) with zeros at keys a row does not see,
             lse (B,) natural-log normaliser of each row)
    """
    x = scale * (q_rows @ k_all.T)                         # logits
    ncols = k_all.shape[0]
    col = np.arange(ncols)[None, :]
    seen = col < np.array([visible_keys(n_c, int(i)) for i in pos])[:, None]
    x = np.where(seen, x, -np.inf)
    m = x.max(axis=1, keepdims=True)
    lse = (m + np.log(np.exp(x - m).sum(axis=1, keepdims=True)))[:, 0]
    a = np.exp(x - lse[:, None])                            # exp(-inf) = 0
    err = np.abs(a.sum(axis=1) - 1.0).max()
    if not err <= ROW_SUM_TOL:
        raise AssertionError(f"attention row sums off by {err}")
    return a, lse


def head_scores(q: np.ndarray, k_ctx: np.ndarray, k_new: np.ndarray,
                scale: float, row_block: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Score of every cached key of one (layer, KV head).

    q     : (G, n_in, d) float64 grouped queries
    k_ctx : (n_c, d) float64 cached keys (KV_c)
    k_new : (n_in, d) float64 keys of the repeat pass
    returns (S (n_c,) in (0, 1], lse (G, n_in))
    """
    G, n_in, d = q.shape
    n_c = k_ctx.shape[0]
    if k_new.shape != (n_in, d) or k_ctx.shape[1] != d:
        raise ValueError("shape mismatch")
    k_all = np.concatenate([k_ctx, k_new], axis=0)
    S = np.zeros(n_c)
    lse = np.empty((G, n_in))
    for g in range(G):
        for i0 in range(0, n_in, row_block):
            i1 = min(n_in, i0 + row_block)
            pos = np.arange(i0, i1)
            a, l = attention_rows(q[g, i0:i1], pos, k_all, n_c, scale)
            lse[g, i0:i1] = l
            # slice to the cached-key columns, then max over g and i
            np.maximum(S, a[:, :n_c].max(axis=0), out=S)
    return S, lse


def row_lse(q_row: np.ndarray, i: int, k_ctx: np.ndarray, k_new: np.ndarray,
            scale: float) -> float:
    """lse of a single query row at position i (for sampled checks)."""
    k_all = np.concatenate([k_ctx, k_new[: i + 1]], axis=0)
    _, l = attention_rows(q_row[None, :], np.array([i]), k_all, k_ctx.shape[0], scale)
    return float(l[0])


# ----------------------------------------------------------------------------
# parallel runner over row blocks of one head (threads, one BLAS thread each)
# ----------------------------------------------------------------------------
def head_scores_parallel(q, k_ctx, k_new, scale, workers: int,
                         row_block: int = 128):
    """Same result as head_scores, split by row blocks over a thread pool
    (NumPy and BLAS release the GIL; nothing is forked).  The max-combine is
    exact and order-free, so the result is identical."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    G, n_in, _ = q.shape
    n_c = k_ctx.shape[0]
    k_all = np.concatenate([k_ctx, k_new], axis=0)
    jobs = [(g, i0, min(n_in, i0 + row_block))
            for g in range(G) for i0 in range(0, n_in, row_block)]
    lse = np.empty((G, n_in))
    S = np.zeros(n_c)

    def block(job):
        g, i0, i1 = job
        a, l = attention_rows(q[g, i0:i1], np.arange(i0, i1), k_all, n_c, scale)
        lse[g, i0:i1] = l
        return a[:, :n_c].max(axis=0)

    with threadpool_limits(limits=1), ThreadPoolExecutor(max(1, workers)) as ex:
        for smax in ex.map(block, jobs):
            np.maximum(S, smax, out=S)
    return S, lse


# ----------------------------------------------------------------------------
# KVzip section 3.4: chunked scoring
# ----------------------------------------------------------------------------
def chunk_bounds(n_c: int, chunk: int):
    """(first key, length) of every chunk: fixed length `chunk`, the last one
    shorter when chunk does not divide n_c."""
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    return [(s, min(chunk, n_c - s)) for s in range(0, n_c, chunk)]


def chunked_head_scores(q_packed: np.ndarray, k_ctx: np.ndarray,
                        k_new_packed: np.ndarray, scale: float, n_prompt: int,
                        chunk: int, G: int, workers: int = 1
                        ) -> Tuple[np.ndarray, np.ndarray]:
    """Chunk-based scoring of one (layer, KV head).

    Each chunk of m_c context tokens is reconstructed on its own: the repeat
    prompt followed by the chunk gives n_in_c = n_prompt + m_c queries per
    query head and n_in_c new keys, and the chunk's m_c cached keys plus those
    new keys form an n_in_c x (m_c + n_in_c) attention; the chunk's keys are
    scored from it exactly as in section 3.2.

    q_packed     : (rows * G, d) - chunk blocks [G][n_in_c][d] back to back
    k_new_packed : (rows, d)     - chunk blocks [n_in_c][d] back to back
    returns (S (n_c,), lse_packed (rows * G,))
    """
    n_c, d = k_ctx.shape
    S = np.zeros(n_c)
    lse_parts = []
    qo = ko = 0
    for start, m in chunk_bounds(n_c, chunk):
        n_in = n_prompt + m
        qc = q_packed[qo:qo + G * n_in].reshape(G, n_in, d)
        kn = k_new_packed[ko:ko + n_in]
        kc = k_ctx[start:start + m]
        if workers > 1:
            Sc, lc = head_scores_parallel(qc, kc, kn, scale, workers=workers)
        else:
            Sc, lc = head_scores(qc, kc, kn, scale)
        S[start:start + m] = Sc
        lse_parts.append(lc.reshape(-1))
        qo += G * n_in
        ko += n_in
    if qo != q_packed.shape[0] or ko != k_new_packed.shape[0]:
        raise ValueError("packed chunk layout does not match n_c, n_prompt, chunk")
    return S, np.concatenate(lse_parts)


# ----------------------------------------------------------------------------
# KVzip section 4.1: keep the r% highest-scoring pairs
# ----------------------------------------------------------------------------
def keep_count(n: int, keep_ratio: float) -> int:
    """k = clamp(floor(r * n), 1, n), r in (0, 1], computed in IEEE double."""
    if not (0.0 < keep_ratio <= 1.0) or n < 1:
        raise ValueError("keep_ratio must be in (0, 1] and n >= 1")
    return int(min(max(math.floor(keep_ratio * float(n)), 1), n))


def topk_ascending(scores: np.ndarray, k: int) -> np.ndarray:
    """The k entries that come first in the order (higher score, then lower
    index), returned as ascending indices."""
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -np.asarray(scores, dtype=np.float64)))
    return np.sort(order[:k])


def select(scores: np.ndarray, keep_ratio: float, mode: int
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Kept index sets in CSR form.

    scores : (L, H, n_c) array (float32 or float64)
    mode 0 : per (l, h), k = keep_count(n_c, r) in every head
    mode 1 : per layer, one top-k_L over the H * n_c flattened scores,
             k_L = keep_count(H * n_c, r); heads end up with different counts
    mode 2 : one top-k over all L * H * n_c scores of the model (the budget
             shared across every head of every layer), k = keep_count(L * H *
             n_c, r); equal scores go to the lower flattened index
             (l * H + h) * n_c + j
    returns offsets int64 (L*H + 1,), idx int32 (total,) - idx holds positions
    j in [0, n_c), ascending within each (l, h), heads in (l, h) order.
    """
    L, H, n_c = scores.shape
    per_head = []
    if mode == 0:
        k = keep_count(n_c, keep_ratio)
        for l in range(L):
            for h in range(H):
                per_head.append(topk_ascending(scores[l, h], k))
    elif mode == 1:
        kl = keep_count(H * n_c, keep_ratio)
        for l in range(L):
            flat = topk_ascending(scores[l].reshape(-1), kl)
            for h in range(H):
                sel = flat[(flat >= h * n_c) & (flat < (h + 1) * n_c)]
                per_head.append(sel - h * n_c)
    elif mode == 2:
        flat = topk_ascending(scores.reshape(-1), keep_count(L * H * n_c, keep_ratio))
        for lh in range(L * H):
            sel = flat[(flat >= lh * n_c) & (flat < (lh + 1) * n_c)]
            per_head.append(sel - lh * n_c)
    else:
        raise ValueError("mode must be 0, 1 or 2")
    counts = np.array([len(x) for x in per_head], dtype=np.int64)
    offsets = np.zeros(L * H + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    idx = (np.concatenate(per_head) if per_head else np.zeros(0)).astype(np.int32)
    return offsets, idx


# ----------------------------------------------------------------------------
# KVzip section 4.2: head-level (context-independent) score
# ----------------------------------------------------------------------------
def head_level_scores(scores: np.ndarray) -> np.ndarray:
    """One static score per (l, h): the largest pair score of the head along
    the sequence.  scores: (L, H, n_c) -> (L, H)."""
    scores = np.asarray(scores)
    if scores.ndim != 3 or scores.shape[2] < 1:
        raise ValueError("scores must be (L, H, n_c) with n_c >= 1")
    return scores.max(axis=2)


# ----------------------------------------------------------------------------
# KVzip section 2.1: KV_p is a subset of KV_c (gather the kept rows)
# ----------------------------------------------------------------------------
def compact(k_ctx: np.ndarray, v_ctx: np.ndarray, offsets: np.ndarray,
            idx: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """k_ctx, v_ctx: (L, H, n_c, d) arrays of any dtype (bit copies).
    returns (k_out, v_out) of shape (total, d), rows grouped in (l, h) order."""
    L, H, n_c, d = k_ctx.shape
    ks, vs = [], []
    for lh in range(L * H):
        l, h = divmod(lh, H)
        sel = idx[offsets[lh]:offsets[lh + 1]]
        ks.append(np.take(k_ctx[l, h], sel, axis=0))
        vs.append(np.take(v_ctx[l, h], sel, axis=0))
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


# ----------------------------------------------------------------------------
# whole-workload convenience (tests and the benchmark's CPU leg)
# ----------------------------------------------------------------------------
def workload_head_inputs(gen_head: dict) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """bf16 bit arrays of one head -> float64 (q, k_ctx, k_new)."""
    return (bf16_to_f64(gen_head["q"]), bf16_to_f64(gen_head["k_ctx"]),
            bf16_to_f64(gen_head["k_new"]))
