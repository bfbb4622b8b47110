"""bench.py's `traffic` field: the calibrated bytes recorded under profiles/
count only while the recorded digest matches the kernel as it is now, and a
workload's own profile is read before any other."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from query_agnostic_eviction_amd.build import kernel_digest  # noqa: E402


def _write(d, name, lines):
    (d / "profiles").mkdir(exist_ok=True)
    (d / "profiles" / name).write_text("# header\n\n" + "\n".join(lines) + "\n")


def test_digest_gates_the_record(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    good, stale = kernel_digest("kvscore_lse"), "0" * 64
    _write(tmp_path, "kvq_kernels_w_traffic.md", [
        f"    traffic kernel=kvscore_lse workload=w bytes=123 digest={stale}",
        f"    traffic kernel=kv_compact workload=w bytes=7 digest={kernel_digest('kv_compact')}"])
    assert bench.recorded_traffic("kvscore_lse", "w") is None       # stale record
    assert bench.recorded_traffic("kv_compact", "w") == 7.0
    assert bench.recorded_traffic("kv_compact", "other") is None    # other workload
    assert bench.recorded_traffic("not_an_entry", "w") is None
    _write(tmp_path, "kvq_kernels_w_traffic.md", [
        f"    traffic kernel=kvscore_lse workload=w bytes=123 digest={good}"])
    assert bench.recorded_traffic("kvscore_lse", "w") == 123.0


def test_own_profile_first(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    dg = kernel_digest("kvscore_lse")
    # "w-merge" sorts before "w_", so without the preference it would win
    _write(tmp_path, "kvq_kernels_w-merge_traffic.md",
           [f"    traffic kernel=kvscore_lse workload=w bytes=1 digest={dg}"])
    _write(tmp_path, "kvq_kernels_w_traffic.md",
           [f"    traffic kernel=kvscore_lse workload=w bytes=2 digest={dg}"])
    assert bench.recorded_traffic("kvscore_lse", "w") == 2.0
    os.remove(tmp_path / "profiles" / "kvq_kernels_w_traffic.md")
    assert bench.recorded_traffic("kvscore_lse", "w") == 1.0


def test_no_profiles_folder(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("kvscore_lse", "w") is None
