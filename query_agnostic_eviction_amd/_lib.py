"""ctypes view of libkvq.so (declarations mirror include/kvq.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KV_OK = 0
KV_ERR_INVALID_ARG = -1
KV_ERR_UNSUPPORTED = -2
KV_ERR_ALIGNMENT = -3
KV_ERR_CAPACITY = -4
KV_ERR_HIP = -5

# every symbol declared in include/kvq.h
EXPORTS = (
    "kv_status_string", "kv_last_hip_error", "kv_keep_count", "kvscore_lse",
    "kvscore_colmax", "kv_chunk_layout", "kvscore_chunked_lse",
    "kvscore_chunked_colmax", "kv_topk_total", "kv_topk_workspace_bytes",
    "kv_topk_select", "kv_topk_select_noalloc", "kv_head_scores", "kv_compact", "kv_copy", "kv_epi_deltas",
    "kv_epi_scores", "kv_select_tokens_workspace_bytes", "kv_select_tokens",
    "kv_compact_tokens", "kv_merge_compact",
)

_lib = None


def _check_stamp() -> None:
    """Refuse a library built from other sources than the ones in the tree."""
    from .build import STAMP, source_digest
    want = source_digest()
    try:
        with open(STAMP) as fh:
            have = fh.read().strip()
    except OSError:
        have = None
    if have != want:
        raise ImportError(
            f"{LIB_PATH} does not match the sources in the tree (stale build): "
            "rebuild with python -m query_agnostic_eviction_amd.build")


def load() -> ctypes.CDLL:
    """Load libkvq.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -m query_agnostic_eviction_amd.build)")
    _check_stamp()
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                  ctypes.c_float, ctypes.c_double, ctypes.c_size_t)
    sig = {
        "kv_status_string": (ctypes.c_char_p, [i32]),
        "kv_last_hip_error": (i32, []),
        "kv_keep_count": (i32, [i64, f64, ctypes.POINTER(i64)]),
        "kvscore_lse": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, i64, i64, f32, vp]),
        "kvscore_colmax": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, i64, i64, f32, vp]),
        "kv_chunk_layout": (i32, [i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "kvscore_chunked_lse": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, i64, i64, i64, f32, vp]),
        "kvscore_chunked_colmax": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, i64, i64, i64, f32, vp]),
        "kv_topk_total": (i32, [i32, i32, i64, f64, i32, ctypes.POINTER(i64)]),
        "kv_topk_workspace_bytes": (sz, [i32, i32, i64, i32]),
        "kv_topk_select": (i32, [vp, i32, i32, i64, f64, i32, vp, vp, i64, vp, sz, vp]),
        "kv_topk_select_noalloc": (i32, [vp, i32, i32, i64, f64, i32, vp, vp, i64, vp]),
        "kv_head_scores": (i32, [vp, i32, i32, i64, vp, vp]),
        "kv_compact": (i32, [vp, vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, vp]),
        "kv_copy": (i32, [vp, vp, i64, vp]),
        "kv_epi_deltas": (i32, [vp, i32, i64, i32, vp, vp]),
        "kv_epi_scores": (i32, [vp, i32, i32, i64, i32, f64, i32, vp, vp]),
        "kv_select_tokens_workspace_bytes": (sz, [i64]),
        "kv_select_tokens": (i32, [vp, i64, i64, vp, vp, sz, vp]),
        "kv_compact_tokens": (i32, [vp, vp, vp, vp, vp, i32, i32, i32, i64, i64, vp]),
        "kv_merge_compact": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32,
                                   i64, i64, i64, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
