"""MI355X-native query-agnostic KV cache scoring and eviction.

KVzip-style maximum cross-attention scoring (pass 1: row lse; pass 2:
cached-key column max), per-head or per-layer top-k selection and K/V
compaction, as hand-written gfx950 HIP kernels in libkvq.so behind a C ABI
(include/kvq.h).  This package is the Python binding of that library; it
fails loudly when the library has not been built.
"""
from .api import (KvqError, epikv_evict, evict, kv_chunk_layout, kv_compact,
                  kv_compact_tokens, kv_copy, kv_epi_deltas, kv_epi_scores, kv_keep_count,
                  kv_head_scores, kv_merge_compact, kv_select_tokens,
                  kv_select_tokens_workspace_bytes, kv_status_string, kv_topk_select,
                  kv_topk_select_noalloc, kv_topk_total,
                  kv_topk_workspace_bytes, kvscore_chunked_colmax,
                  kvscore_chunked_lse, kvscore_colmax, kvscore_lse, score,
                  score_chunked, select, compact)
