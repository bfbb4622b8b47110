"""bench.py's command-line contract: one JSON line with the documented
fields (GPU), and a clear refusal of more than one GPU (CPU: the refusal
comes before anything touches a device)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, timeout=300):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
@pytest.mark.parametrize("workload", ["tiny", "epikv-tiny"])
def test_json_line_fields(workload):
    print("bench contract:", workload, flush=True)
    r = _bench("--workload", workload, "--steps", "2", "--warmup", "1", "--cpu-seconds", "0.5")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1, r.stdout
    j = json.loads(lines[0])
    assert j["metric"] == "context KV pairs scored+compacted/sec" and j["unit"] == "KV pairs/s"
    assert j["value"] > 0 and j["ms_per_step"] > 0
    assert (j["n_gpus"], j["steps"], j["warmup"]) == (1, 2, 1)
    assert j["higher_is_better"] is True and j["scaling"] == "weak"
    assert j["vs_baseline"] is None and j["data"] == "synthetic"
    assert isinstance(j["dtype"], str) and j["config"]["workload"] == workload
    roof = j["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof
    cpu = j["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1
    assert cpu["unit"] == j["unit"] and cpu["sample"]
