"""Build libkvq.so (the gfx950 HIP kernels and their C ABI) in-tree.

    python -m query_agnostic_eviction_amd.build

Each HIP source is compiled with hipcc for gfx950 in parallel, then linked
into query_agnostic_eviction_amd/libkvq.so next to this file.  Packed-fp32
instruction selection is disabled for all device code.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvq.so")

SOURCES = ["kvscore_lse.hip", "kvscore_colmax.hip", "kv_topk.hip",
           "kv_compact.hip", "epikv.hip", "selkv_merge.hip",
           "kvq_api.hip"]

# per-source extra flags: pass 2 reduces with max3 on finite values and -inf
# padding only, so NaN semantics (and their canonicalising copies) are off
EXTRA_FLAGS = {"kvscore_colmax.hip": ["-fno-honor-nans"]}

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-op accumulators in ordinary VGPRs: the softmax reductions read
    # them directly instead of copying them out of AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def source_digest() -> str:
    """Digest of everything that determines libkvq.so: sources, header, flags."""
    h = hashlib.sha256()
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    for f in files:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    with open(os.path.join(INCLUDE, "kvq.h"), "rb") as fh:
        h.update(fh.read())
    h.update(" ".join(CFLAGS[:-2]).encode())
    h.update(repr(sorted(EXTRA_FLAGS.items())).encode())
    return h.hexdigest()


# host-only sources: argument checks and dispatch of the C ABI, no device code
HOST_ONLY = ("kvq_api.hip",)
# headers every kernel source includes
DEVICE_HEADERS = ("kvq_device.h", "kvq_internal.h")
# the source file that holds the kernels of each entry point
KERNEL_SOURCES = {
    "kvscore_lse": "kvscore_lse.hip", "kvscore_colmax": "kvscore_colmax.hip",
    "kv_topk_select": "kv_topk.hip", "kv_topk_select_noalloc": "kv_topk.hip",
    "kv_head_scores": "kv_topk.hip",
    "kv_select_tokens": "kv_topk.hip", "kv_compact": "kv_compact.hip",
    "kv_compact_tokens": "kv_compact.hip", "kv_copy": "kv_compact.hip", "kv_epi_deltas": "epikv.hip",
    "kv_epi_scores": "epikv.hip", "kv_merge_compact": "selkv_merge.hip",
}


def kernel_digest(entry: str = None) -> str:
    """Digest of device code: with `entry`, the source holding that entry
    point's kernels plus the device headers and the flags it is built with;
    without, every kernel source.  A hardware-counter record of a kernel
    stays valid while its digest is unchanged (the C ABI's host checks, the
    public header's documentation and the other kernels do not touch it)."""
    if entry is None:
        files = sorted(f for f in os.listdir(CSRC)
                       if f.endswith((".hip", ".h")) and f not in HOST_ONLY)
        extra = sorted(EXTRA_FLAGS.items())
    else:
        src = KERNEL_SOURCES[entry]
        files = [src, *DEVICE_HEADERS]
        extra = EXTRA_FLAGS.get(src, [])
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    h.update(" ".join(CFLAGS[:-2]).encode())
    h.update(repr(extra).encode())
    return h.hexdigest()


STAMP = LIB + ".stamp"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libkvq")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 target feature; that
    # warning is expected and harmless
    lines = [ln for ln in r.stdout.splitlines()
             if "packed-fp32-ops' is not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError("command failed: " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([hipcc, *CFLAGS, *EXTRA_FLAGS.get(src, []), "-c",
                     os.path.join(CSRC, src), "-o", obj])
    workers = max(1, min(len(cmds), os.cpu_count() or 1))
    with ThreadPoolExecutor(workers) as ex:
        outs = list(ex.map(_run, cmds))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    with open(STAMP, "w") as fh:   # lets the loader refuse a stale library
        fh.write(source_digest() + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
