"""Host logic of the build: the digests that tie the loaded library and the
recorded hardware-counter figures to the sources.

- source_digest covers every C/HIP source, the public header and the flags
  (the loader refuses a library built from other sources);
- kernel_digest(entry) covers the source file holding that entry point's
  kernels, the shared device headers and the flags, and nothing else, so a
  counter record stays valid exactly while its kernel is unchanged."""
import os
import shutil

import pytest

import query_agnostic_eviction_amd.build as B
from query_agnostic_eviction_amd import _lib


@pytest.fixture
def tree(tmp_path, monkeypatch):
    """A copy of the sources the digests read, with build.py pointed at it."""
    csrc, inc = tmp_path / "csrc", tmp_path / "include"
    shutil.copytree(B.CSRC, csrc)
    shutil.copytree(B.INCLUDE, inc)
    monkeypatch.setattr(B, "CSRC", str(csrc))
    monkeypatch.setattr(B, "INCLUDE", str(inc))
    return csrc, inc


def _touch(path):
    with open(path, "a") as fh:
        fh.write("\n// edited\n")


def test_every_entry_point_has_a_kernel_source():
    exported = set(_lib.EXPORTS)
    host_only = {"kv_status_string", "kv_last_hip_error", "kv_keep_count", "kv_chunk_layout",
                 "kv_topk_total", "kv_topk_workspace_bytes",
                 "kv_select_tokens_workspace_bytes"}
    chunked = {"kvscore_chunked_lse", "kvscore_chunked_colmax"}   # the pass kernels
    for name in exported - host_only - chunked:
        assert name in B.KERNEL_SOURCES, name
    for src in set(B.KERNEL_SOURCES.values()):
        assert os.path.exists(os.path.join(B.CSRC, src)) and src in B.SOURCES
    for h in B.DEVICE_HEADERS:
        assert os.path.exists(os.path.join(B.CSRC, h))


def test_kernel_digest_follows_its_own_source_only(tree):
    csrc, _ = tree
    entries = sorted(B.KERNEL_SOURCES)
    before = {e: B.kernel_digest(e) for e in entries}
    _touch(csrc / "selkv_merge.hip")
    after = {e: B.kernel_digest(e) for e in entries}
    for e in entries:
        changed = B.KERNEL_SOURCES[e] == "selkv_merge.hip"
        assert (before[e] != after[e]) == changed, e


def test_device_header_and_flags_change_every_kernel_digest(tree, monkeypatch):
    csrc, _ = tree
    entries = sorted(B.KERNEL_SOURCES)
    d0 = {e: B.kernel_digest(e) for e in entries}
    _touch(csrc / "kvq_device.h")
    d1 = {e: B.kernel_digest(e) for e in entries}
    assert all(d0[e] != d1[e] for e in entries)
    monkeypatch.setattr(B, "CFLAGS", B.CFLAGS[:1] + ["-O2"] + B.CFLAGS[2:])
    d2 = {e: B.kernel_digest(e) for e in entries}
    assert all(d1[e] != d2[e] for e in entries)
    # a per-file flag moves only that file's kernels
    monkeypatch.setattr(B, "EXTRA_FLAGS", {**B.EXTRA_FLAGS, "kv_compact.hip": ["-DX"]})
    d3 = {e: B.kernel_digest(e) for e in entries}
    for e in entries:
        assert (d2[e] != d3[e]) == (B.KERNEL_SOURCES[e] == "kv_compact.hip"), e


def test_host_only_sources_leave_kernel_digests_alone(tree):
    csrc, inc = tree
    entries = sorted(B.KERNEL_SOURCES)
    d0 = {e: B.kernel_digest(e) for e in entries}
    whole0, src0 = B.kernel_digest(), B.source_digest()
    _touch(csrc / "kvq_api.hip")
    _touch(inc / "kvq.h")
    assert {e: B.kernel_digest(e) for e in entries} == d0
    assert B.kernel_digest() == whole0
    assert B.source_digest() != src0          # the loader still sees the change
