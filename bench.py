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
    # HBM reads of the scores per select: a segment of at most 32,768 scores
    # (mode 0: a head, mode 1: a layer) is staged in LDS once; longer ones are
    # read by 3 histogram passes and 1 ordered pass; mode 2 reads 5 times
    seg = n_c if mode == 0 else w.H * n_c
    reads = 5 if mode == 2 else (1 if seg <= 32768 else 4)
    return {
        "lse_flops": 2.0 * d * logits1 * heads,
        "lse_exps": float(logits1 * heads),
        "colmax_flops": 2.0 * d * logits2 * heads,
        # scores read, idx + offsets written
        "select_bytes": 4.0 * reads * heads * n_c + 4.0 * total
                        + 8.0 * (heads + 1),
        # K and V rows read and written, plus the index of each row
        "compact_bytes": 2.0 * 2 * 2 * d * total + 4.0 * total,
        "kept_rows": total,
    }


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` recorded under profiles/ by rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (calibrated against a plain copy), or None
    if no record matches the device code as it is now."""
    from query_agnostic_eviction_amd.build import KERNEL_SOURCES, kernel_digest
    if kernel not in KERNEL_SOURCES:
        return None
    digest = kernel_digest(kernel)
    prof = os.path.join(ROOT, "profiles")
    if not os.path.isdir(prof):
        return None
    own = f"kvq_kernels_{workload}_traffic.md"   # this workload's own profile first
    for name in sorted(os.listdir(prof), key=lambda n: (n != own, n)):
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def calibration_copy(torch):
    """A plain 1 GiB device-to-device copy, run once untimed and once timed:
    its bytes read + written per second are the practical HBM ceiling of a
    streaming kernel on this part, and under rocprofv3 --pmc its FETCH_SIZE /
    WRITE_SIZE calibrate the counters."""
    src = torch.empty(CALIB_BYTES // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    return 2.0 * CALIB_BYTES / (e0.elapsed_time(e1) * 1e-3) / 1e9


def calibration_gemm(torch, n=8192, reps=400, warm=50):
    """A plain n x n x n bf16 matrix product through the vendor BLAS
    (torch.matmul, contiguous operands), run after the timed region for about
    0.3 s: its TFLOP/s is the practically attainable dense bf16 matrix rate of
    this part under sustained load, the reference point for the scoring passes'
    fraction of the nominal peak."""
    gen = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn((n, n), device="cuda", generator=gen).to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda", generator=gen).to(torch.bfloat16).contiguous()
    c = torch.matmul(a, b)
    for _ in range(warm):   # sustained rate, not the first burst
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    flops = 2.0 * n * n * n * reps
    return flops / (e0.elapsed_time(e1) * 1e-3) / 1e12


def cold_time_ms(torch, fn, reps=5):
    """Median time of fn() on the current stream, each run preceded by a
    1 GiB write to a scratch buffer so that no input is left in the 256 MB
    last-level cache (MALL) when fn starts."""
    scratch = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    times = []
    for r in range(reps):
        scratch.fill_(float(r))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del scratch
    return float(np.median(times))


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


def cpu_baseline(w, seconds: float, mode: int = 0, chunk=None, merge=False):
    """The float64 oracle on whole heads of the workload, head after head,
    until `seconds` have passed (at least one head)."""
    import oracle
    workers = min(16, synth.default_workers())
    # logits of one whole head: every row sees the cached keys and the new
    # keys up to its own position
    head_logits = w.G * (w.n_in * w.n_c + w.n_in * (w.n_in + 1) // 2)
    if not chunk and head_logits > 2e10:
        return cpu_baseline_rows(w, seconds, workers, head_logits)
    done, t_oracle, heads, ref = 0, 0.0, [], {}
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
        if merge:
            so, si = synth.nearest_position_routes(off, idx, w.n_c)
            oracle.selkv.merge_compact(oracle.bf16_to_f64(gen["k_ctx"])[None, None],
                                       oracle.bf16_to_f64(gen["v_ctx"])[None, None],
                                       off, idx, so, si)
        else:
            oracle.compact(gen["k_ctx"][None, None], gen["v_ctx"][None, None], off, idx)
        t_oracle += time.perf_counter() - t0
        done += w.n_c
        heads.append((l, h))
        ref[(l, h)] = S
        if t_oracle >= seconds:
            break
    return {
        "value": done / t_oracle,
        "unit": "KV pairs/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{len(heads)} whole (layer, KV head) slices of {w.name} "
                  f"({done} context KV pairs): float64 attention rows, max score, "
                  f"top-k and {'gated merge' if merge else 'gather'}; {t_oracle:.1f} s",
        "cpu_model": cpu_model(),
        # every head costs the same, so the whole workload would take this long
        "extrapolated_full_s": round(t_oracle / len(heads) * w.L * w.H, 1),
        # the oracle's scores of those heads, for the accuracy fields (not printed)
        "_ref_scores": ref,
    }


def cpu_baseline_rows(w, seconds, workers, head_logits):
    """For heads too large to finish within the budget (the 128K context):
    the oracle on the first R query rows of one head.  Row i sees the cached
    keys and new keys 0..i, so rows 0..R-1 are exactly that part of the whole
    head's work; the head's time is extrapolated by the logit count."""
    import oracle
    gen = synth.generate_head(w, 0, 0)
    q, kc, kn = oracle.workload_head_inputs(gen)
    rate_guess = 1e9                      # logits/s of the oracle on 16 cores, roughly
    R = int(min(w.n_in, max(128, seconds * rate_guess / (w.G * (w.n_c + 1)))))
    part = w.G * (R * w.n_c + R * (R + 1) // 2)
    t0 = time.perf_counter()
    oracle.head_scores_parallel(q[:, :R], kc, kn[:R], float(w.scale), workers=workers)
    t = time.perf_counter() - t0
    t_head = t * head_logits / part
    return {
        "value": w.n_c / t_head,
        "unit": "KV pairs/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"query rows 0..{R - 1} of all {w.G} query heads of one (layer, KV head) slice "
                  f"of {w.name} ({part / head_logits:.1%} of that slice's logits): float64 "
                  f"attention rows and running max; {t:.1f} s, extrapolated to the slice "
                  f"by logit count ({t_head:.0f} s)",
        "cpu_model": cpu_model(),
        "extrapolated_full_s": round(t_head * w.L * w.H, 1),
    }


SCORE_RTOL, SCORE_ATOL = 2e-3, 1e-6   # score tolerance against the oracle


def accuracy_fields(ref, scores_gpu, offsets, idx, keep_ratio, mode):
    """Per-run accuracy of the GPU scores on the heads the CPU baseline ran:
    the largest relative score error, whether every score is within
    |s - S| <= atol + rtol * S, and (per-head budget) the near-tie band: with
    tau the k-th largest oracle score of a head, the keys with
    (tau (1 - rtol) - 2 atol) / (1 + rtol) <= S <= (tau (1 + rtol) + 2 atol) / (1 - rtol)
    could swap places within the tolerance; every key above the band must be
    kept and every key below it dropped.  Plain arithmetic on the stored
    oracle scores and the GPU outputs."""
    import math
    if not ref:
        return {"max_rel_err": None, "scores_within_tol": None, "near_tie_band": None,
                "topk_outside_band_ok": None, "heads_checked": 0}
    H = scores_gpu.shape[1]
    max_rel, ok, band_pop, sel_ok = 0.0, True, 0, True
    for (l, h), S in ref.items():
        g = scores_gpu[l, h].astype(np.float64)
        err = np.abs(g - S)
        max_rel = max(max_rel, float(np.max(err / S)))
        ok = ok and bool(np.all(err <= SCORE_ATOL + SCORE_RTOL * S))
        if mode == 0:
            n = S.size
            k = min(max(math.floor(keep_ratio * n), 1), n)
            tau = float(np.sort(S)[n - k])
            lo = (tau * (1 - SCORE_RTOL) - 2 * SCORE_ATOL) / (1 + SCORE_RTOL)
            hi = (tau * (1 + SCORE_RTOL) + 2 * SCORE_ATOL) / (1 - SCORE_RTOL)
            band_pop += int(np.count_nonzero((S >= lo) & (S <= hi)))
            lh = l * H + h
            kept = np.zeros(n, bool)
            kept[idx[offsets[lh]:offsets[lh + 1]]] = True
            sel_ok = sel_ok and bool(kept[S > hi].all()) and not bool(kept[S < lo].any()) \
                and int(kept.sum()) == k
    return {"max_rel_err": max_rel, "scores_within_tol": ok,
            "near_tie_band": band_pop if mode == 0 else None,
            "topk_outside_band_ok": sel_ok if mode == 0 else None,
            "heads_checked": len(ref)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=synth.LLAMA8B_8K.name,
                    choices=sorted(synth.BY_NAME) + sorted(synth.EPI_BY_NAME))
    ap.add_argument("--mode", type=int, default=0, choices=(0, 1, 2))
    ap.add_argument("--chunk", type=int, default=0,
                    help="chunked scoring with this chunk length (0 = whole context)")
    ap.add_argument("--device-inputs", action="store_true",
                    help="fill the inputs with seeded N(0,1) values made on the GPU instead of "
                         "the host generator (for timing the largest workloads; the kernels' "
                         "time does not depend on the values)")
    ap.add_argument("--merge", action="store_true",
                    help="gated merge (soft cosine gate) of the evicted tokens into their "
                         "nearest kept position instead of plain compaction")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="oracle time budget for the CPU baseline (0 = skip)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path is built and timed on a "
              "single MI355X. Every (layer, KV head) is independent, so several "
              "GPUs would each score their own share of the heads. Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.workload in synth.EPI_BY_NAME:
        return run_epikv(args)
    w = synth.BY_NAME[args.workload]
    chunk = args.chunk or None
    work = algorithmic_work(w, args.mode, chunk)

    # host work first: input generation and the oracle baseline (thread pools)
    t0 = time.perf_counter()
    gen = None
    if args.device_inputs:
        pass
    elif chunk:
        gen = synth.generate_chunked_workload(w, chunk, workers=min(16, synth.default_workers()))
    else:
        gen = synth.generate_workload(w, workers=min(16, synth.default_workers()))
    t_gen = time.perf_counter() - t0
    print(f"# generated {w.name} in {t_gen:.1f} s", file=sys.stderr, flush=True)
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, args.cpu_seconds, args.mode, chunk, args.merge)
        print(f"# cpu baseline: {cpu['value']:.3g} pairs/s", file=sys.stderr, flush=True)

    import torch
    import query_agnostic_eviction_amd as kvq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if gen is not None:
        dev = {k: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
               for k, v in gen.items()}
        del gen
    else:
        rows = synth.chunk_rows(w, chunk) if chunk else w.n_in
        shapes = {"q": (w.L, w.H, rows * w.G, w.d) if chunk else (w.L, w.H, w.G, w.n_in, w.d),
                  "k_ctx": (w.L, w.H, w.n_c, w.d), "k_new": (w.L, w.H, rows, w.d),
                  "v_ctx": (w.L, w.H, w.n_c, w.d)}
        rng = torch.Generator(device="cuda").manual_seed(w.seed)
        dev = {}
        for k, shp in shapes.items():
            t = torch.empty(shp, dtype=torch.bfloat16, device="cuda")
            for l in range(w.L):   # per layer: bounded fp32 temporaries
                t[l] = torch.randn(shp[1:], generator=rng, device="cuda").to(torch.bfloat16)
            dev[k] = t
        torch.cuda.synchronize()
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

    names = ("kvscore_lse", "kvscore_colmax", "kv_topk_select",
             "kv_merge_compact" if args.merge else "kv_compact")
    route = {}
    gate = mass = None

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
        if route:
            kvq.kv_merge_compact(dev["k_ctx"], dev["v_ctx"], offsets, idx, route["so"],
                                 route["si"], k_out, v_out, gate, mass, stream)
        else:
            kvq.kv_compact(dev["k_ctx"], dev["v_ctx"], offsets, idx, k_out, v_out, stream)
        mark(4)

    for i in range(max(args.warmup, 1 if args.merge else 0)):
        step()
        torch.cuda.synchronize()
        print(f"# warmup step {i + 1}/{args.warmup} done", file=sys.stderr, flush=True)
        if args.merge and not route:
            # routing is an input of the merge: built once on the host from the
            # kept set (identical in every step: same inputs, same scores)
            so, si = synth.nearest_position_routes(offsets.cpu().numpy(), idx.cpu().numpy(),
                                                   n_c)
            route["so"] = torch.from_numpy(so).cuda()
            route["si"] = torch.from_numpy(si).cuda()
            gate = torch.empty(max(si.size, 1), dtype=torch.float32, device="cuda")
            mass = torch.empty(total, dtype=torch.float32, device="cuda")
            work["merge_bytes"] = (2.0 * 2 * d * (total + si.size) + 2.0 * 2 * d * total
                                   + 8.0 * si.size + 12.0 * total + 8.0 * (L * H + 1))

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
    copy_gbs = calibration_copy(torch)
    gemm_tflops = calibration_gemm(torch)

    # compaction alone with no input left in the last-level cache
    def compact_only():
        if route:
            kvq.kv_merge_compact(dev["k_ctx"], dev["v_ctx"], offsets, idx, route["so"],
                                 route["si"], k_out, v_out, gate, mass, stream)
        else:
            kvq.kv_compact(dev["k_ctx"], dev["v_ctx"], offsets, idx, k_out, v_out, stream)
    cold_ms = cold_time_ms(torch, compact_only)
    # the library's own streaming copy over the same byte count (half read,
    # half written), also with nothing cached: the compaction's HBM reference
    cbytes = work["merge_bytes" if args.merge else "compact_bytes"]
    n16 = int(cbytes // 2) // 16
    csrc = torch.empty(n16 * 16, dtype=torch.uint8, device="cuda")
    cdst = torch.empty_like(csrc)
    copy_cold_ms = cold_time_ms(torch, lambda: kvq.kv_copy(csrc, cdst, stream))
    stream_copy_gbs = 2.0 * n16 * 16 / (copy_cold_ms * 1e-3) / 1e9
    del csrc, cdst

    ref = cpu.pop("_ref_scores", None) if cpu else None
    if args.device_inputs:   # the oracle ran on the generator's inputs, not these
        ref = None
    acc = accuracy_fields(ref, scores.cpu().numpy(), offsets.cpu().numpy(), idx.cpu().numpy(),
                          w.keep_ratio, args.mode)

    ms_per_step = 1e3 * elapsed / args.steps
    value = w.context_pairs / (elapsed / args.steps)
    lse_tf = work["lse_flops"] / (ms["kvscore_lse"] * 1e-3) / 1e12
    col_tf = work["colmax_flops"] / (ms["kvscore_colmax"] * 1e-3) / 1e12
    scoring_tf = (work["lse_flops"] + work["colmax_flops"]) / (
        (ms["kvscore_lse"] + ms["kvscore_colmax"]) * 1e-3) / 1e12
    cmp_name = names[3]
    cmp_gbs = work["merge_bytes" if args.merge else "compact_bytes"] / (
        ms[cmp_name] * 1e-3) / 1e9
    sel_gbs = work["select_bytes"] / (ms["kv_topk_select"] * 1e-3) / 1e9

    dominant = max(names, key=lambda n: ms[n])
    traffic = recorded_traffic(dominant, w.name + (f"-chunk{chunk}" if chunk else ""))
    if dominant in ("kvscore_lse", "kvscore_colmax"):
        achieved = lse_tf if dominant == "kvscore_lse" else col_tf
        roof = {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    else:
        achieved = cmp_gbs if dominant == cmp_name else sel_gbs
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
                   "select_mode": args.mode, "chunk": chunk,
                   "merge": "soft cosine gate, nearest kept position" if args.merge else None,
                   "inputs": "device N(0,1)" if args.device_inputs else "synth generator"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels_ms": {n: round(v, 4) for n, v in ms.items()},
        "scoring_mfma_frac": round(scoring_tf / PEAK_BF16_TFLOPS, 4),
        "lse_mfma_frac": round(lse_tf / PEAK_BF16_TFLOPS, 4),
        "colmax_mfma_frac": round(col_tf / PEAK_BF16_TFLOPS, 4),
        "compact_hbm_frac": round(cmp_gbs / PEAK_HBM_GBS, 4),
        "compact_cold_hbm_frac": round(cbytes / (cold_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        # the library's streaming copy of the same bytes, cold, and the cold
        # compaction's rate as a fraction of it
        "stream_copy_cold_gbs": round(stream_copy_gbs, 1),
        "compact_cold_frac_of_copy": round(cbytes / (cold_ms * 1e-3) / 1e9 / stream_copy_gbs, 4),
        "select_gbs": round(sel_gbs, 1),
        "copy_gbs": round(copy_gbs, 1),
        # attainable dense bf16 rate (vendor GEMM, 8192^3) and the two
        # scoring passes' combined rate as a fraction of it
        "gemm_tflops": round(gemm_tflops, 1),
        "scoring_frac_of_gemm": round(scoring_tf / gemm_tflops, 4),
        # GPU scores of the CPU baseline's heads against the oracle's
        # (KVzip page, section 4.1: the band the budget decision guards)
        **acc,
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# attention-free EpiKV path (EpiKV page, section 3.2): hidden-state deltas,
# band scores, top-K tokens, token compaction of every (layer, head)
# ---------------------------------------------------------------------------
def epikv_work(w):
    nl = len(w.layers)
    kept = w.L * w.H * w.budget
    return {
        # each hidden row read once, g written
        "deltas_bytes": 2.0 * nl * w.n * w.D + 4.0 * nl * w.n,
        "scores_bytes": 4.0 * nl * w.n + 4.0 * w.n,
        # scores read by 3 histogram passes, a counting pass and the write
        "select_bytes": 4.0 * 5 * w.n + 4.0 * w.budget,
        # K and V rows read and written
        "compact_bytes": 2.0 * 2 * 2 * w.d * kept + 4.0 * w.budget,
    }


def epikv_cpu_baseline(w, hidden, seconds):
    """The float64 oracle on a prefix of the trace (the first N tokens, N
    doubled until a run takes half the budget or covers the trace)."""
    import oracle
    from oracle import epikv as E
    from threadpoolctl import threadpool_limits
    rng = np.random.default_rng(0)
    na = len(w.band_a)
    N = min(4096, w.n)
    while True:
        k = max(1, w.budget * N // w.n)
        kc = rng.integers(0, 2 ** 16, size=(w.L, w.H, N, w.d), dtype=np.uint16)
        vc = rng.integers(0, 2 ** 16, size=(w.L, w.H, N, w.d), dtype=np.uint16)
        with threadpool_limits(1):
            t0 = time.perf_counter()
            g = [E.hidden_deltas(oracle.bf16_to_f64(hidden[l, :N]))
                 for l in range(hidden.shape[0])]
            sc = E.token_scores(g[:na], g[na:], w.window, w.eps, True)
            idx = E.select_tokens(sc, k)
            E.compact_tokens(kc, vc, idx)
            t = time.perf_counter() - t0
        del kc, vc
        if t >= seconds / 2 or N >= w.n:
            break
        N = min(w.n, 2 * N)
    return {
        "value": w.L * w.H * N / t,
        "unit": "KV pairs/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"first {N} of {w.n} tokens of {w.name}: float64 deltas of "
                  f"{hidden.shape[0]} hidden layers, rolling z-scores, top-{k}, gather of "
                  f"{w.L}x{w.H} heads; {t:.1f} s",
        "cpu_model": cpu_model(),
        # work is linear in the trace length
        "extrapolated_full_s": round(t * w.n / N, 1),
    }


def run_epikv(args):
    w = synth.EPI_BY_NAME[args.workload]
    work = epikv_work(w)
    t0 = time.perf_counter()
    hidden = synth.generate_hidden(w, workers=min(16, synth.default_workers()))
    print(f"# generated {w.name} hidden states in {time.perf_counter() - t0:.1f} s",
          file=sys.stderr, flush=True)
    cpu = None
    if args.cpu_seconds > 0:
        cpu = epikv_cpu_baseline(w, hidden, args.cpu_seconds)
        print(f"# cpu baseline: {cpu['value']:.3g} pairs/s", file=sys.stderr, flush=True)

    import torch
    import query_agnostic_eviction_amd as kvq

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    h = torch.from_numpy(hidden.view(np.int16)).view(torch.bfloat16).cuda()
    del hidden
    gen = torch.Generator(device="cuda").manual_seed(w.seed)
    shape = (w.L, w.H, w.n, w.d)
    kc = torch.randint(-32768, 32767, shape, dtype=torch.int16, device="cuda",
                       generator=gen).view(torch.bfloat16)
    vc = torch.randint(-32768, 32767, shape, dtype=torch.int16, device="cuda",
                       generator=gen).view(torch.bfloat16)
    nl, na = len(w.layers), len(w.band_a)
    g = torch.empty((nl, w.n), dtype=torch.float32, device="cuda")
    scores = torch.empty(w.n, dtype=torch.float32, device="cuda")
    idx = torch.empty(w.budget, dtype=torch.int32, device="cuda")
    k_out = torch.empty((w.L, w.H, w.budget, w.d), dtype=torch.bfloat16, device="cuda")
    v_out = torch.empty_like(k_out)
    sel_ws = torch.empty(kvq.kv_select_tokens_workspace_bytes(w.n), dtype=torch.uint8,
                         device="cuda")
    stream = torch.cuda.current_stream()
    names = ("kv_epi_deltas", "kv_epi_scores", "kv_select_tokens", "kv_compact_tokens")

    def step(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        kvq.kv_epi_deltas(h, g, stream)
        mark(1)
        kvq.kv_epi_scores(g, na, w.window, w.eps, True, scores, stream)
        mark(2)
        kvq.kv_select_tokens(scores, w.budget, idx, stream, sel_ws)
        mark(3)
        kvq.kv_compact_tokens(kc, vc, idx, k_out, v_out, stream)
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
    copy_gbs = calibration_copy(torch)
    cold = {"kv_epi_deltas": cold_time_ms(torch, lambda: kvq.kv_epi_deltas(h, g, stream)),
            "kv_compact_tokens": cold_time_ms(
                torch, lambda: kvq.kv_compact_tokens(kc, vc, idx, k_out, v_out, stream))}

    key = {"kv_epi_deltas": "deltas_bytes", "kv_epi_scores": "scores_bytes",
           "kv_select_tokens": "select_bytes", "kv_compact_tokens": "compact_bytes"}
    gbs = {n: work[key[n]] / (ms[n] * 1e-3) / 1e9 for n in names}
    dominant = max(names, key=lambda n: ms[n])
    roof = {"kernel": dominant, "bound": "hbm", "achieved": round(gbs[dominant], 1),
            "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs[dominant] / PEAK_HBM_GBS, 4),
            "traffic": recorded_traffic(dominant, w.name)}
    line = {
        "metric": "context KV pairs scored+compacted/sec",
        "value": w.kv_pairs / (elapsed / args.steps),
        "unit": "KV pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * elapsed / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "L": w.L, "H": w.H, "d": w.d, "D": w.D, "n": w.n,
                   "budget": w.budget, "band_a": list(w.band_a), "band_b": list(w.band_b),
                   "window": w.window, "score": "EpiKV detrended (eq. 3)"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels_ms": {n: round(v, 4) for n, v in ms.items()},
        "hbm_frac": {n: round(gbs[n] / PEAK_HBM_GBS, 4) for n in names},
        "cold_hbm_frac": {n: round(work[key[n]] / (cold[n] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                          for n in cold},
        "copy_gbs": round(copy_gbs, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
