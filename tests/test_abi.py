"""C ABI of libkvq on the host (no GPU): exported symbols and argument checks.

Every call here fails validation before any HIP call is made, so nothing is
launched; fake but well-aligned pointer values stand in for device buffers.
"""
import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
from query_agnostic_eviction_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

OK, INV, UNS, ALN, CAP = 0, -1, -2, -3, -4
P = ctypes.c_void_p(0x10000)      # aligned fake pointer
P2 = ctypes.c_void_p(0x10002)     # 2-byte aligned only
P4 = ctypes.c_void_p(0x10004)     # 4-byte aligned only
NUL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kv\w*)\s*\(", text)))


def test_header_symbols_exported(lib):
    declared = _declared()
    assert set(declared) == set(_lib.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", out, flags=re.M))
    missing = [s for s in declared if s not in exported]
    assert not missing, missing
    for s in declared:
        assert hasattr(lib, s)


def test_status_strings(lib):
    names = {0: b"KV_OK", -1: b"KV_ERR_INVALID_ARG", -2: b"KV_ERR_UNSUPPORTED",
             -3: b"KV_ERR_ALIGNMENT", -4: b"KV_ERR_CAPACITY", -5: b"KV_ERR_HIP"}
    for k, v in names.items():
        assert lib.kv_status_string(k) == v
    assert lib.kv_status_string(42) == b"KV_ERR_UNKNOWN"
    assert lib.kv_last_hip_error() == 0


def test_keep_count_matches_oracle(lib):
    rng = np.random.default_rng(0)
    out = ctypes.c_int64()
    cases = [(512, 0.3), (8192, 0.3), (32768, 0.25), (131072, 0.3), (16384, 0.1),
             (131072, 0.1), (1, 1.0), (7, 0.999999), (10, 0.05)]
    cases += [(int(rng.integers(1, 10 ** 7)), float(rng.uniform(1e-6, 1.0))) for _ in range(500)]
    for n, r in cases:
        assert lib.kv_keep_count(n, r, ctypes.byref(out)) == OK
        assert out.value == oracle.keep_count(n, r), (n, r)
    for bad in (0.0, -1.0, 1.5, math.nan, math.inf):
        assert lib.kv_keep_count(10, bad, ctypes.byref(out)) == INV
    assert lib.kv_keep_count(0, 0.5, ctypes.byref(out)) == INV
    assert lib.kv_keep_count(10, 0.5, None) == INV


def test_topk_total(lib):
    out = ctypes.c_int64()
    assert lib.kv_topk_total(32, 8, 8192, 0.3, 0, ctypes.byref(out)) == OK
    assert out.value == 256 * 2457
    assert lib.kv_topk_total(48, 8, 16384, 0.1, 1, ctypes.byref(out)) == OK
    assert out.value == 48 * 13107
    assert lib.kv_topk_total(48, 8, 16384, 0.1, 2, ctypes.byref(out)) == OK
    assert out.value == oracle.keep_count(48 * 8 * 16384, 0.1)
    assert lib.kv_topk_total(48, 8, 16384, 0.1, 3, ctypes.byref(out)) == UNS
    assert lib.kv_topk_total(0, 8, 16384, 0.1, 0, ctypes.byref(out)) == INV
    # mode 2 is limited to 2^40 scores in all; modes 0 and 1 are not
    assert lib.kv_topk_total(2 ** 20, 1, 2 ** 20, 0.1, 2, ctypes.byref(out)) == INV
    assert lib.kv_topk_total(2 ** 20, 1, 2 ** 20 - 1, 0.1, 2, ctypes.byref(out)) == OK
    assert lib.kv_topk_total(2 ** 20, 1, 2 ** 20, 0.1, 0, ctypes.byref(out)) == OK
    assert lib.kv_topk_workspace_bytes(32, 8, 8192, 0) == 0
    assert lib.kv_topk_workspace_bytes(32, 8, 8192, 1) == 0
    ws = lib.kv_topk_workspace_bytes(32, 8, 8192, 2)
    assert 16384 <= ws <= 16384 + 16 * 1024 + 1024
    assert lib.kv_topk_workspace_bytes(1, 1, 1, 2) >= 16384


def _lse(lib, q=P, kc=P, kn=P, lse=P, L=1, H=1, G=4, d=128, n_c=16, n_p=2, scale=0.1):
    return lib.kvscore_lse(q, kc, kn, lse, L, H, G, d, n_c, n_p, scale, NUL)


def _col(lib, q=P, kc=P, lse=P, sc=P, L=1, H=1, G=4, d=128, n_c=16, n_p=2, scale=0.1):
    return lib.kvscore_colmax(q, kc, lse, sc, L, H, G, d, n_c, n_p, scale, NUL)


@pytest.mark.parametrize("fn", [_lse, _col])
def test_score_validation(lib, fn):
    assert fn(lib, q=NUL) == INV
    assert fn(lib, kc=NUL) == INV
    assert fn(lib, L=0) == INV
    assert fn(lib, H=-1) == INV
    assert fn(lib, n_c=0) == INV
    assert fn(lib, n_p=-1) == INV
    for s in (-0.5, -0.0 - 1e-30, math.nan, math.inf, 2.4e8, 2e-39):
        assert fn(lib, scale=s) == INV
    # accepted scales pass on to the pointer checks (a misaligned pointer
    # then reports KV_ERR_ALIGNMENT without touching a device): 0 selects
    # float32(1 / sqrt(d)); the range ends where 1e30 * scale * log2(e) or
    # 1 / scale stops being finite in fp32
    for s in (0.0, 0.1, 2.3e8, 3e-39):
        assert fn(lib, scale=s, q=P2) == ALN
    for d in (0, 32, 96, 512):
        assert fn(lib, d=d) == UNS
    for g in (0, 9, -1):
        assert fn(lib, G=g) == UNS
    assert fn(lib, G=8, n_c=2 ** 28, n_p=0) == INV       # G * n_in >= 2^31
    assert fn(lib, n_c=2 ** 31, G=1, n_p=0) == INV
    assert fn(lib, q=P2) == ALN
    assert fn(lib, kc=P4) == ALN


def test_score_validation_specific(lib):
    assert _lse(lib, kn=NUL) == INV
    assert _lse(lib, lse=NUL) == INV
    assert _lse(lib, kn=P4) == ALN
    assert _lse(lib, lse=P2) == ALN
    assert _col(lib, lse=NUL) == INV
    assert _col(lib, sc=NUL) == INV
    assert _col(lib, sc=P2) == ALN


def _sel(lib, sc=P, L=2, H=2, n_c=100, r=0.3, mode=0, off=P, idx=P, cap=1000,
         ws=NUL, wsb=0):
    return lib.kv_topk_select(sc, L, H, n_c, r, mode, off, idx, cap, ws, wsb, NUL)


def test_select_validation(lib):
    assert _sel(lib, sc=NUL) == INV
    assert _sel(lib, off=NUL) == INV
    assert _sel(lib, idx=NUL) == INV
    for r in (0.0, 1.01, -0.2, math.nan):
        assert _sel(lib, r=r) == INV
    assert _sel(lib, mode=3) == UNS
    assert _sel(lib, mode=-1) == UNS
    wsb = lib.kv_topk_workspace_bytes(2, 2, 100, 2)
    assert _sel(lib, mode=2, cap=119) == CAP
    assert _sel(lib, mode=2, wsb=wsb - 1, ws=P) == CAP
    assert _sel(lib, mode=2, wsb=wsb, ws=NUL) == INV
    assert _sel(lib, mode=2, wsb=wsb, ws=ctypes.c_void_p(0x10080)) == ALN
    assert _sel(lib, n_c=0) == INV
    assert _sel(lib, cap=4 * 30 - 1) == CAP
    assert _sel(lib, mode=1, cap=2 * 60 - 1) == CAP
    assert _sel(lib, off=P4) == ALN
    assert _sel(lib, sc=P2) == ALN


def test_select_noalloc_validation(lib):
    """The allocation-free selection rejects the same arguments as
    kv_topk_select (minus the workspace ones) before touching a device."""
    def sel(sc=P, L=2, H=2, n_c=100, r=0.3, mode=0, off=P, idx=P, cap=1000):
        return lib.kv_topk_select_noalloc(sc, L, H, n_c, r, mode, off, idx, cap, NUL)
    assert sel(sc=NUL) == INV
    assert sel(off=NUL) == INV
    assert sel(idx=NUL) == INV
    for r in (0.0, 1.01, math.nan):
        assert sel(r=r) == INV
    assert sel(mode=3) == UNS
    assert sel(n_c=0) == INV
    assert sel(mode=2, cap=119) == CAP
    assert sel(cap=4 * 30 - 1) == CAP
    assert sel(off=P4) == ALN
    assert sel(sc=P2) == ALN
    # the largest mode-2 state fits the library's fixed device array
    assert lib.kv_topk_workspace_bytes(1 << 9, 1 << 10, 1 << 21, 2) <= 48 * 1024


def test_head_scores_validation(lib):
    f = lib.kv_head_scores
    assert f(NUL, 2, 2, 10, P, NUL) == INV
    assert f(P, 2, 2, 10, NUL, NUL) == INV
    assert f(P, 0, 2, 10, P, NUL) == INV
    assert f(P, 2, 2, 0, P, NUL) == INV
    assert f(P2, 2, 2, 10, P, NUL) == ALN
    assert f(P, 2, 2, 10, P2, NUL) == ALN


def _cmp(lib, kc=P, vc=P, off=P, idx=P, ko=P, vo=P, L=2, H=2, d=128, n_c=100, total=120):
    return lib.kv_compact(kc, vc, off, idx, ko, vo, L, H, d, n_c, total, NUL)


def test_compact_validation(lib):
    for name in ("kc", "vc", "off", "idx", "ko", "vo"):
        assert _cmp(lib, **{name: NUL}) == INV
    assert _cmp(lib, d=32) == UNS
    assert _cmp(lib, d=100) == UNS
    assert _cmp(lib, total=-1) == INV
    assert _cmp(lib, total=401) == INV                # more rows than L*H*n_c
    assert _cmp(lib, n_c=2 ** 31) == INV              # positions are int32
    assert _cmp(lib, L=0) == INV
    assert _cmp(lib, ko=P4) == ALN
    assert _cmp(lib, off=P4) == ALN
    assert _cmp(lib, idx=P2) == ALN
    # an empty kept set: nothing is enqueued and its empty buffers may be null
    assert _cmp(lib, total=0) == OK
    assert _cmp(lib, idx=NUL, ko=NUL, vo=NUL, total=0) == OK
    for name in ("kc", "vc", "off"):
        assert _cmp(lib, **{name: NUL}, total=0) == INV
    assert _cmp(lib, total=0, d=96) == UNS


def test_binding_rejects_host_tensors():
    import torch
    import query_agnostic_eviction_amd as kvq
    q = torch.zeros((1, 1, 1, 4, 64), dtype=torch.bfloat16)
    k = torch.zeros((1, 1, 4, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kvq.kvscore_lse(q, k, k)
    with pytest.raises(ValueError):
        kvq.kv_topk_select(torch.zeros((1, 1, 4)), 0.5)


def test_chunk_layout(lib):
    nch, rows = ctypes.c_int64(), ctypes.c_int64()
    for n_c, n_p, chunk, want in [(131072, 32, 2048, (64, 64 * 32 + 131072)),
                                  (1000, 3, 300, (4, 12 + 1000)), (7, 0, 10, (1, 7)),
                                  (5, 2, 1, (5, 15))]:
        assert lib.kv_chunk_layout(n_c, n_p, chunk, ctypes.byref(nch), ctypes.byref(rows)) == OK
        assert (nch.value, rows.value) == want
    assert lib.kv_chunk_layout(0, 1, 1, ctypes.byref(nch), ctypes.byref(rows)) == INV
    assert lib.kv_chunk_layout(5, 1, 0, ctypes.byref(nch), ctypes.byref(rows)) == INV


@pytest.mark.parametrize("name", ["kvscore_chunked_lse", "kvscore_chunked_colmax"])
def test_chunked_validation(lib, name):
    fn = getattr(lib, name)

    def call(q=P, a=P, b=P, c=P, L=1, H=1, G=4, d=128, n_c=64, n_p=2, chunk=16, scale=0.1):
        return fn(q, a, b, c, L, H, G, d, n_c, n_p, chunk, scale, NUL)
    assert call(chunk=0) == INV
    assert call(chunk=-5) == INV
    assert call(q=NUL) == INV
    assert call(c=NUL) == INV
    assert call(d=96) == UNS
    assert call(G=9) == UNS
    assert call(n_c=0) == INV
    assert call(scale=math.nan) == INV
    assert call(q=P2) == ALN


def test_epikv_validation(lib):
    d = lib.kv_epi_deltas
    assert d(NUL, 2, 100, 4096, P, NUL) == INV
    assert d(P, 2, 100, 4096, NUL, NUL) == INV
    assert d(P, 0, 100, 4096, P, NUL) == INV
    assert d(P, 2, 0, 4096, P, NUL) == INV
    assert d(P, 64, 2 ** 30, 4096, P, NUL) == INV      # grid would exceed 2^31 workgroups
    for D in (0, 4, 12, 8200, 16384):
        assert d(P, 2, 100, D, P, NUL) == UNS
    assert d(P2, 2, 100, 4096, P, NUL) == ALN
    assert d(P, 2, 100, 4096, P2, NUL) == ALN

    s = lib.kv_epi_scores
    assert s(NUL, 1, 1, 100, 64, 1e-6, 1, P, NUL) == INV
    assert s(P, 0, 1, 100, 64, 1e-6, 1, P, NUL) == INV
    assert s(P, 1, 0, 100, 64, 1e-6, 1, P, NUL) == INV
    assert s(P, 1, 1, 0, 64, 1e-6, 1, P, NUL) == INV
    assert s(P, 1, 1, 100, 0, 1e-6, 1, P, NUL) == INV
    assert s(P, 1, 1, 100, 1025, 1e-6, 1, P, NUL) == UNS
    for eps in (0.0, -1e-6, math.nan, math.inf):
        assert s(P, 1, 1, 100, 64, eps, 1, P, NUL) == INV
    assert s(P, 1, 1, 100, 64, 1e-6, 2, P, NUL) == INV
    assert s(P2, 1, 1, 100, 64, 1e-6, 1, P, NUL) == ALN

    t = lib.kv_select_tokens
    wsb = lib.kv_select_tokens_workspace_bytes(100)
    assert wsb >= 16384 and lib.kv_select_tokens_workspace_bytes(0) == 0
    assert lib.kv_select_tokens_workspace_bytes(65536) == wsb + 16 * 15   # a block per 4096
    assert t(NUL, 100, 10, P, P, wsb, NUL) == INV
    assert t(P, 100, 0, P, P, wsb, NUL) == INV
    assert t(P, 100, 101, P, P, wsb, NUL) == INV
    assert t(P, 100, 10, P, NUL, wsb, NUL) == INV
    assert t(P, 2 ** 31, 10, P, P, wsb, NUL) == INV
    assert t(P, 100, 10, P2, P, wsb, NUL) == ALN
    assert t(P, 100, 10, P, ctypes.c_void_p(0x10080), wsb, NUL) == ALN
    assert t(P, 100, 10, P, P, wsb - 1, NUL) == CAP

    c = lib.kv_compact_tokens
    assert c(NUL, P, P, P, P, 2, 2, 128, 100, 10, NUL) == INV
    assert c(P, P, P, P, P, 2, 2, 128, 100, 101, NUL) == INV
    assert c(P, P, P, P, P, 2, 2, 128, 100, -1, NUL) == INV
    assert c(P, P, P, P, P, 2, 2, 96, 100, 10, NUL) == UNS
    assert c(P, P, P, P4, P, 2, 2, 128, 100, 10, NUL) == ALN
    assert c(P, P, P2, P, P, 2, 2, 128, 100, 10, NUL) == ALN
    assert c(P, P, P, P, P, 2, 2, 128, 100, 0, NUL) == OK      # nothing to copy, no launch
    assert c(P, P, NUL, NUL, NUL, 2, 2, 128, 100, 0, NUL) == OK   # empty buffers may be null
    assert c(P, P, NUL, P, P, 2, 2, 128, 100, 10, NUL) == INV
    assert c(P, NUL, NUL, NUL, NUL, 2, 2, 128, 100, 0, NUL) == INV


def test_merge_validation(lib):
    f = lib.kv_merge_compact

    def call(kc=P, vc=P, off=P, idx=P, so=P, si=P, ko=P, vo=P, g=P, m=P, L=2, H=2, d=128,
             n_c=100, total=50, n_src=30):
        return f(kc, vc, off, idx, so, si, ko, vo, g, m, L, H, d, n_c, total, n_src, NUL)
    for name in ("kc", "vc", "off", "idx", "so", "ko", "vo"):
        assert call(**{name: NUL}) == INV
    assert call(si=NUL) == INV
    assert call(si=NUL, n_src=0, total=0) == OK          # nothing to do, no launch
    assert call(g=NUL, m=NUL, total=0) == OK
    assert call(idx=NUL, ko=NUL, vo=NUL, si=NUL, g=NUL, m=NUL, total=0, n_src=0) == OK
    assert call(so=NUL, total=0, n_src=0) == INV
    assert call(total=401) == INV
    assert call(n_src=-1) == INV
    assert call(d=96) == UNS
    assert call(so=P4) == ALN
    assert call(g=P2) == ALN
    assert call(ko=P4) == ALN
