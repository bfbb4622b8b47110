"""Writes the float64 oracle's scores of one whole head (layer l, KV head h)
of the llama3.1-8b-128k workload (131,072 cached keys, 131,104 query rows
per query head) to tests/golden/llama3.1-8b-128k_head{l}-{h}.npz.  The
parity tests use the first and the last head, (0, 0) and (31, 7).

Inputs come from the seeded generator (synth) and the values from the
oracle only (KVzip page, section 3.2: each cached key's score is the max of
its softmax probabilities over all grouped query rows).  Stored: the scores
as float32 (relative rounding 6e-8, far inside the 2e-3 test tolerance) and
the lse of every 16th row of each query head as float32 (rows 0, 16, ...).

Run from the repository root:
    python tests/golden/make_llama128k_head.py [l h]     (default: 31 7)
(about 10 minutes per head on 8 cores).
"""
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def out_path(l, h):
    return os.path.join(ROOT, "tests", "golden", f"llama3.1-8b-128k_head{l}-{h}.npz")


def main():
    w = synth.LLAMA8B_128K
    l, h = (int(sys.argv[1]), int(sys.argv[2])) if len(sys.argv) > 2 else (w.L - 1, w.H - 1)
    assert 0 <= l < w.L and 0 <= h < w.H
    OUT = out_path(l, h)
    gen = synth.generate_head(w, l, h)
    q, kc, kn = oracle.workload_head_inputs(gen)
    t0 = time.time()
    S, lse = oracle.head_scores_parallel(q, kc, kn, float(w.scale),
                                         workers=synth.default_workers())
    print(f"oracle head ({l},{h}) of {w.name}: {time.time() - t0:.0f} s", flush=True)
    np.savez_compressed(OUT, scores=S.astype(np.float32),
                        lse_rows16=lse[:, ::16].astype(np.float32),
                        layer=np.int64(l), head=np.int64(h),
                        workload=np.array(w.name))
    print("wrote", OUT)


if __name__ == "__main__":
    main()
