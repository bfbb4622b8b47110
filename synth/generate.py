"""Seeded synthetic inputs for the scoring / eviction path.

Both the float64 oracle and the GPU path read the values made here; nothing in
this module computes any part of the method.  Every (layer, KV head) slice is
drawn from its own counter-keyed stream
    numpy PCG64(SeedSequence([seed, cfg_id, l, h, stream]))
so any head can be regenerated on its own, on any machine, bit for bit.

Recipe for one (l, h) slice, in the shapes of the KVzip page's section 3.2
(Q in R^{G x n_in x d}; keys of the pass are the n_c cached keys followed by
the n_in new keys):
  * a basis B (rank x d) with orthonormal rows, from the QR factors of a
    Gaussian matrix (stream 0);
  * every row x of Q (stream 1), K_ctx (stream 2) and K_new (stream 3) is
    x = z + alpha * (c @ B) with z ~ N(0, I_d) and c ~ N(0, I_rank);
  * V_ctx ~ N(0, I_d) (stream 4), plus alpha * (c @ B) for the tiny workload;
  * sink rows of K_ctx are multiplied by sink_scale;
  * structure (stream 5):
      near_dup    - floor(0.1 n_c) rows p drawn without replacement from
                    [5, n_c) become K_base[q] + 0.01 N(0, I_d), q ~ U[4, p);
      span_repeat - K_ctx and V_ctx rows [4096 k + 64, 4096 k + 128) become
                    exact copies of rows [64, 128) for every k >= 1 that fits;
      student_t   - every K_ctx and K_new row is multiplied by |t|, t drawn
                    from a Student-t law with 3 degrees of freedom;
  * every value is rounded float64 -> float32 -> bfloat16, each step to
    nearest-even.  The returned arrays hold the bfloat16 bit patterns
    (uint16); consumers must read those rounded values, never the unrounded
    draws.
"""
from __future__ import annotations

import os
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np

from . import configs as C
from .configs import Workload

(STREAM_BASIS, STREAM_Q, STREAM_KCTX, STREAM_KNEW, STREAM_V, STREAM_STRUCT,
 STREAM_Q_CHUNKS, STREAM_KNEW_CHUNKS, STREAM_STRUCT_CHUNKS) = range(9)


def _rng(w: Workload, l: int, h: int, stream: int) -> np.random.Generator:
    ss = np.random.SeedSequence([w.seed, w.cfg_id, l, h, stream])
    return np.random.Generator(np.random.PCG64(ss))


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (nearest-even) -> bfloat16 bits (nearest-even)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 values."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


def _basis(w: Workload, l: int, h: int) -> np.ndarray:
    g = _rng(w, l, h, STREAM_BASIS).standard_normal((w.d, w.rank))
    qf, _ = np.linalg.qr(g)              # d x rank, orthonormal columns
    return np.ascontiguousarray(qf.T)    # rank x d, orthonormal rows


def _rows(rng: np.random.Generator, n: int, w: Workload, basis: np.ndarray,
          lowrank: bool = True) -> np.ndarray:
    z = rng.standard_normal((n, w.d))
    if lowrank:
        c = rng.standard_normal((n, w.rank))
        z += w.alpha * (c @ basis)
    return z


def generate_head(w: Workload, l: int, h: int,
                  parts: Iterable[str] = ("q", "k_ctx", "k_new", "v_ctx")
                  ) -> Dict[str, np.ndarray]:
    """bf16 bit patterns of one (l, h) slice.

    Returns a dict with any of
      q      uint16 [G][n_in][d]
      k_ctx  uint16 [n_c][d]
      k_new  uint16 [n_in][d]
      v_ctx  uint16 [n_c][d]
    """
    parts = tuple(parts)
    basis = _basis(w, l, h)
    out: Dict[str, np.ndarray] = {}
    srng = None
    need_k = ("k_ctx" in parts) or ("v_ctx" in parts and w.structure == "span_repeat")

    k_ctx = k_new = None
    if need_k or "k_new" in parts:
        k_ctx = _rows(_rng(w, l, h, STREAM_KCTX), w.n_c, w, basis)
        for r in w.sink_rows:
            if r < w.n_c:
                k_ctx[r] *= w.sink_scale
    if "k_new" in parts or w.structure == "student_t":
        k_new = _rows(_rng(w, l, h, STREAM_KNEW), w.n_in, w, basis)

    v_ctx = None
    if "v_ctx" in parts:
        v_ctx = _rows(_rng(w, l, h, STREAM_V), w.n_c, w, basis, lowrank=w.v_lowrank)

    if w.structure != "none":
        srng = _rng(w, l, h, STREAM_STRUCT)
    if w.structure == "near_dup" and k_ctx is not None:
        n_copy = int(np.floor(C.NEAR_DUP_FRACTION * w.n_c))
        lo = C.NEAR_DUP_MIN_DST
        if w.n_c - lo > 0 and n_copy > 0:
            n_copy = min(n_copy, w.n_c - lo)
            dst = lo + srng.choice(w.n_c - lo, size=n_copy, replace=False)
            src = srng.integers(C.NEAR_DUP_MIN_SRC, dst)      # q ~ U[4, p)
            noise = srng.standard_normal((n_copy, w.d)) * C.NEAR_DUP_NOISE_STD
            base = k_ctx.copy()
            k_ctx[dst] = base[src] + noise
    elif w.structure == "span_repeat":
        s0, s1 = C.SPAN_SRC, C.SPAN_SRC + C.SPAN_LEN
        k = 1
        while C.SPAN_PERIOD * k + s1 <= w.n_c:
            a = C.SPAN_PERIOD * k + s0
            if k_ctx is not None:
                k_ctx[a:a + C.SPAN_LEN] = k_ctx[s0:s1]
            if v_ctx is not None:
                v_ctx[a:a + C.SPAN_LEN] = v_ctx[s0:s1]
            k += 1
    elif w.structure == "student_t":
        t_ctx = np.abs(srng.standard_t(C.STUDENT_T_NU, size=w.n_c))
        t_new = np.abs(srng.standard_t(C.STUDENT_T_NU, size=w.n_in))
        if k_ctx is not None:
            k_ctx *= t_ctx[:, None]
        if k_new is not None:
            k_new *= t_new[:, None]

    if "q" in parts:
        q = _rows(_rng(w, l, h, STREAM_Q), w.G * w.n_in, w, basis)
        out["q"] = f64_to_bf16_bits(q).reshape(w.G, w.n_in, w.d)
    if "k_ctx" in parts:
        out["k_ctx"] = f64_to_bf16_bits(k_ctx)
    if "k_new" in parts:
        out["k_new"] = f64_to_bf16_bits(k_new)
    if "v_ctx" in parts:
        out["v_ctx"] = f64_to_bf16_bits(v_ctx)
    return out


def chunk_rows(w: Workload, chunk: int) -> int:
    """Query positions per (l, h) over all chunks of the packed layout."""
    n_chunks = -(-w.n_c // min(chunk, w.n_c))
    return n_chunks * w.n_prompt + w.n_c


def generate_chunked_head(w: Workload, l: int, h: int, chunk: int,
                          parts: Iterable[str] = ("q", "k_ctx", "k_new", "v_ctx")
                          ) -> Dict[str, np.ndarray]:
    """Inputs of chunk-based scoring for one (l, h): every chunk has its own
    repeat pass, so its queries and new keys are fresh draws of the same
    recipe (streams 6 and 7; the Student-t key multipliers of the new keys
    from stream 8).  The cached keys and values are those of generate_head.

      q      uint16 [rows * G][d]   chunk blocks [G][n_prompt + m_c][d]
      k_new  uint16 [rows][d]       chunk blocks [n_prompt + m_c][d]
      k_ctx, v_ctx as generate_head
    """
    parts = tuple(parts)
    out = generate_head(w, l, h, [p for p in parts if p in ("k_ctx", "v_ctx")])
    basis = _basis(w, l, h)
    m = min(chunk, w.n_c)
    bounds = [(s0, min(m, w.n_c - s0)) for s0 in range(0, w.n_c, m)]
    if "q" in parts:
        rng = _rng(w, l, h, STREAM_Q_CHUNKS)
        blocks = [_rows(rng, w.G * (w.n_prompt + mc), w, basis) for _, mc in bounds]
        out["q"] = f64_to_bf16_bits(np.concatenate(blocks))
    if "k_new" in parts:
        rng = _rng(w, l, h, STREAM_KNEW_CHUNKS)
        blocks = [_rows(rng, w.n_prompt + mc, w, basis) for _, mc in bounds]
        kn = np.concatenate(blocks)
        if w.structure == "student_t":
            t = np.abs(_rng(w, l, h, STREAM_STRUCT_CHUNKS).standard_t(C.STUDENT_T_NU,
                                                                       size=kn.shape[0]))
            kn *= t[:, None]
        out["k_new"] = f64_to_bf16_bits(kn)
    return out


def _head_job(args):
    w, l, h, parts = args
    return l, h, generate_head(w, l, h, parts)


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def generate_workload(w: Workload,
                      heads: Optional[Sequence[Tuple[int, int]]] = None,
                      parts: Iterable[str] = ("q", "k_ctx", "k_new", "v_ctx"),
                      workers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Full [L][H]-indexed bf16 bit arrays for the listed heads.

    Heads not listed stay zero.  Uses a thread pool when workers > 1.
    """
    parts = tuple(parts)
    if heads is None:
        heads = [(l, h) for l in range(w.L) for h in range(w.H)]
    shapes = {
        "q": (w.L, w.H, w.G, w.n_in, w.d),
        "k_ctx": (w.L, w.H, w.n_c, w.d),
        "k_new": (w.L, w.H, w.n_in, w.d),
        "v_ctx": (w.L, w.H, w.n_c, w.d),
    }
    out = {p: np.zeros(shapes[p], dtype=np.uint16) for p in parts}
    jobs = [(w, l, h, parts) for (l, h) in heads]
    workers = default_workers() if workers is None else workers

    def run(job):
        l, h, d = _head_job(job)
        for p in parts:
            out[p][l, h] = d[p]

    if workers <= 1 or len(jobs) <= 1:
        for job in jobs:
            run(job)
    else:
        # threads, not processes: NumPy's random fills, BLAS and ufunc loops
        # release the GIL, and nothing is forked (safe after GPU start-up)
        from concurrent.futures import ThreadPoolExecutor
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1), ThreadPoolExecutor(min(workers, len(jobs))) as ex:
            list(ex.map(run, jobs))
    return out


def generate_chunked_workload(w: Workload, chunk: int,
                              workers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """generate_chunked_head for every (l, h), as [L][H]-indexed arrays:
    q [L][H][rows*G][d], k_new [L][H][rows][d], k_ctx / v_ctx [L][H][n_c][d]."""
    rows = chunk_rows(w, chunk)
    out = {"q": np.zeros((w.L, w.H, rows * w.G, w.d), np.uint16),
           "k_new": np.zeros((w.L, w.H, rows, w.d), np.uint16),
           "k_ctx": np.zeros((w.L, w.H, w.n_c, w.d), np.uint16),
           "v_ctx": np.zeros((w.L, w.H, w.n_c, w.d), np.uint16)}

    def run(lh):
        l, h = lh
        g = generate_chunked_head(w, l, h, chunk)
        for p in out:
            out[p][l, h] = g[p]

    heads = [(l, h) for l in range(w.L) for h in range(w.H)]
    workers = default_workers() if workers is None else workers
    if workers <= 1:
        for lh in heads:
            run(lh)
    else:
        from concurrent.futures import ThreadPoolExecutor
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1), ThreadPoolExecutor(workers) as ex:
            list(ex.map(run, heads))
    return out
