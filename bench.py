#!/usr/bin/env python3
"""Benchmark of the query-agnostic eviction path on one MI355X.

One step = one pass of the whole path over the workload's full batch of
synthetic inputs already resident in HBM:
    kvscore_lse -> kvscore_colmax -> kv_topk_select -> kv_compact
(KVzip page, "KVzip: Query-Agnostic KV Cache Compression with Context
Reconstruction": section 3.2 scoring, section 4.1 budget, section 2.1 KV_p).

Prints one JSON line: throughput in context KV pairs scored and compacted per
second, the roofline of the dominant kernel (timed with HIP events on the
stream the kernels run on), and the float64 oracle timed on the host cores
over a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
CALIB_BYTES = 1 << 30       # plain copy used to calibrate HBM byte counters


def algorithmic_work(w, mode=0, chunk=None):
    """Work the method itself requires (no padding, no masked tiles).  With
    chunked scoring every chunk of m cached keys has n_prompt + m rows."""
    G, d, n_c = w.G, w.d, w.n_c
    heads = w.L * w.H
    if chunk:
        ms = [min(chunk, n_c - s) for s in range(0, n_c, min(chunk, n_c))]
    else:
        ms = [n_c]
    logits1 = logits2 = 0
    for m in ms:
        n_in = w.n_prompt + m
        logits1 += G * (n_in * m + n_in * (n_in + 1) // 2)   # every seen key, every row
        logits2 += G * n_in * m                              # cached columns only
    total = synth_total(w, mode)
    return {
        "lse_flops": 2.0 * d * logits1 * heads,
        "lse_exps": float(logits1 * heads),
        "colmax_flops": 2.0 * d * logits2 * heads,
        # scores read by 3 histogram passes and 1 ordered pass (mode 2 adds a
        # counting pass); idx + offsets written
        "select_bytes": 4.0 * (5 if mode == 2 else 4) * heads * n_c + 4.0 * total
                        + 8.0 * (heads + 1),
        # K and V rows read and written, plus the index of each row
        "compact_bytes": 2.0 * 2 * 2 * d * total + 4.0 * total,
        "kept_rows": total,
    }


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` recorded under profiles/ by rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (calibrated against a plain copy), or None
    if no record matches the library sources as they are now."""
    from query_agnostic_eviction_amd.build import source_digest
    digest = source_digest()
    prof = os.path.join(ROOT, "profiles")
    if not os.path.isdir(prof):
        return None
    for name in sorted(os.listdir(prof)):
        if not name.endswith("_traffic.md"):
            continue
        with open(os.path.join(prof, name)) as fh:
            for line in fh:
                f = dict(kv.split("=", 1) for kv in line.split() if "=" in kv)
                if (line.strip().startswith("traffic") and f.get("workload") == workload
                        and f.get("kernel", "").split("<")[0] == kernel
                        and f.get("digest") == digest):
                    return float(f["bytes"])
    return None


def synth_total(w, mode):
    import math
    if mode == 0:
        k = min(max(math.floor(w.keep_ratio * w.n_c), 1), w.n_c)
        return w.L * w.H * k
    if mode == 2:
        n = w.L * w.H * w.n_c
        return min(max(math.floor(w.keep_ratio * n), 1), n)
    kl = min(max(math.floor(w.keep_ratio * w.H * w.n_c), 1), w.H * w.n_c)
    return w.L * kl


def cpu_baseline(w, seconds: float, mode: int = 0, chunk=None):
    """The float64 oracle on whole heads of the workload, head after head,
    until `seconds` have passed (at least one head)."""
    import oracle
    workers = min(16, synth.default_workers())
    done, t_oracle, heads = 0, 0.0, []
    order = [(l, h) for l in range(w.L) for h in range(w.H)]
    for (l, h) in order:
        gen = synth.generate_chunked_head(w, l, h, chunk) if chunk else synth.generate_head(w, l, h)
        q, kc, kn = oracle.workload_head_inputs(gen)
        t0 = time.perf_counter()
        if chunk:
            S, _ = oracle.chunked_head_scores(q, kc, kn, float(w.scale), w.n_prompt, chunk,
                                              w.G, workers=workers)
        else:
            S, _ = oracle.head_scores_parallel(q, kc, kn, float(w.scale), workers=workers)
        off, idx = oracle.select(S[None, None], w.keep_ratio, 0)
        oracle.compact(gen["k_ctx"][None, None], gen["v_ctx"][None, None], off, idx)
        t_oracle += time.perf_counter() - t0
        done += w.n_c
        heads.append((l, h))
        if t_oracle >= seconds:
            break
    return {
        "value": done / t_oracle,
        "unit": "KV pairs/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{len(heads)} whole (layer, KV head) slices of {w.name} "
                  f"({done} context KV pairs): float64 attention rows, max score, "
                  f"top-k and gather; {t_oracle:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=synth.LLAMA8B_8K.name,
                    choices=sorted(synth.BY_NAME))
    ap.add_argument("--mode", type=int, default=0, choices=(0, 1, 2))
    ap.add_argument("--chunk", type=int, default=0,
                    help="chunked scoring with this chunk length (0 = whole context)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time budget for the CPU baseline (0 = skip)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path is built and timed on a "
              "single MI355X (every (layer, KV head) is independent; see the "
              "sharding notes in the design document). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    w = synth.BY_NAME[args.workload]
    chunk = args.chunk or None
    work = algorithmic_work(w, args.mode, chunk)

    # host work first: input generation and the oracle baseline (thread pools)
    t0 = time.perf_counter()
    if chunk:
        gen = synth.generate_chunked_workload(w, chunk, workers=min(16, synth.default_workers()))
    else:
        gen = synth.generate_workload(w, workers=min(16, synth.default_workers()))
    t_gen = time.perf_counter() - t0
    print(f"# generated {w.name} in {t_gen:.1f} s", file=sys.stderr, flush=True)
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, args.cpu_seconds, args.mode, chunk)
        print(f"# cpu baseline: {cpu['value']:.3g} pairs/s", file=sys.stderr, flush=True)

    import torch
    import query_agnostic_eviction_amd as kvq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
           for k, v in gen.items()}
    del gen
    L, H, G, n_c, n_in, d = w.L, w.H, w.G, w.n_c, w.n_in, w.d
    scale = float(w.scale)
    total = work["kept_rows"]
    if chunk:
        lse = torch.empty((L, H, synth.chunk_rows(w, chunk) * G), dtype=torch.float32,
                          device="cuda")
    else:
        lse = torch.empty((L, H, G, n_in), dtype=torch.float32, device="cuda")
    scores = torch.empty((L, H, n_c), dtype=torch.float32, device="cuda")
    offsets = torch.empty(L * H + 1, dtype=torch.int64, device="cuda")
    idx = torch.empty(total, dtype=torch.int32, device="cuda")
    k_out = torch.empty((total, d), dtype=torch.bfloat16, device="cuda")
    v_out = torch.empty((total, d), dtype=torch.bfloat16, device="cuda")
    ws_bytes = kvq.kv_topk_workspace_bytes(w.L, w.H, w.n_c, args.mode)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    names = ("kvscore_lse", "kvscore_colmax", "kv_topk_select", "kv_compact")

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        if chunk:
            kvq.kvscore_chunked_lse(dev["q"], dev["k_ctx"], dev["k_new"], G, w.n_prompt,
                                    chunk, lse, scale, stream)
        else:
            kvq.kvscore_lse(dev["q"], dev["k_ctx"], dev["k_new"], lse, scale, stream)
        mark(1)
        if chunk:
            kvq.kvscore_chunked_colmax(dev["q"], dev["k_ctx"], lse, G, w.n_prompt, chunk,
                                       scores, scale, stream)
        else:
            kvq.kvscore_colmax(dev["q"], dev["k_ctx"], lse, scores, scale, stream)
        mark(2)
        kvq.kv_topk_select(scores, w.keep_ratio, args.mode, offsets, idx, stream, ws)
        mark(3)
        kvq.kv_compact(dev["k_ctx"], dev["v_ctx"], offsets, idx, k_out, v_out, stream)
        mark(4)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        print(f"# warmup step {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms = {n: float(np.mean([events[s][i].elapsed_time(events[s][i + 1])
                            for s in range(args.steps)]))
          for i, n in enumerate(names)}

    # a plain device copy of known size after the timed region: under
    # rocprofv3 --pmc its FETCH_SIZE / WRITE_SIZE calibrate the counters
    calib_src = torch.empty(CALIB_BYTES // 2, dtype=torch.int16, device="cuda")
    torch.empty_like(calib_src).copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src

    ms_per_step = 1e3 * elapsed / args.steps
    value = w.context_pairs / (elapsed / args.steps)
    lse_tf = work["lse_flops"] / (ms["kvscore_lse"] * 1e-3) / 1e12
    col_tf = work["colmax_flops"] / (ms["kvscore_colmax"] * 1e-3) / 1e12
    scoring_tf = (work["lse_flops"] + work["colmax_flops"]) / (
        (ms["kvscore_lse"] + ms["kvscore_colmax"]) * 1e-3) / 1e12
    cmp_gbs = work["compact_bytes"] / (ms["kv_compact"] * 1e-3) / 1e9
    sel_gbs = work["select_bytes"] / (ms["kv_topk_select"] * 1e-3) / 1e9

    dominant = max(names, key=lambda n: ms[n])
    traffic = recorded_traffic(dominant, w.name) if not chunk else None
    if dominant in ("kvscore_lse", "kvscore_colmax"):
        achieved = lse_tf if dominant == "kvscore_lse" else col_tf
        roof = {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    else:
        achieved = cmp_gbs if dominant == "kv_compact" else sel_gbs
        roof = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}

    line = {
        "metric": "context KV pairs scored+compacted/sec",
        "value": value,
        "unit": "KV pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "L": L, "H": H, "G": G, "d": d, "n_c": n_c,
                   "n_prompt": w.n_prompt, "keep_ratio": w.keep_ratio,
                   "select_mode": args.mode, "chunk": chunk},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels_ms": {n: round(v, 4) for n, v in ms.items()},
        "scoring_mfma_frac": round(scoring_tf / PEAK_BF16_TFLOPS, 4),
        "lse_mfma_frac": round(lse_tf / PEAK_BF16_TFLOPS, 4),
        "colmax_mfma_frac": round(col_tf / PEAK_BF16_TFLOPS, 4),
        "compact_hbm_frac": round(cmp_gbs / PEAK_HBM_GBS, 4),
        "select_gbs": round(sel_gbs, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
