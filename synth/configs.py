"""Workload shapes for the scoring / eviction path.

Each workload fixes the attention geometry named in the KVzip page's notation
("KVzip: Query-Agnostic KV Cache Compression with Context Reconstruction",
section 2.1 and section 3.2): L layers, H KV heads, G query heads per KV head,
head dimension d, n_c context tokens, n_prompt repeat-prompt tokens, and
n_in = n_prompt + n_c query positions.  The keep ratio r is the budget of the
eviction structure in section 4.1 of the same page.

The shapes follow public model geometries (Llama-3.1-8B, Qwen2.5-14B,
Gemma3-12B); every value is synthetic.  This module holds no arithmetic of the
method itself: it only describes inputs.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int            # stream id mixed into every seed
    L: int
    H: int
    G: int
    d: int
    n_c: int
    n_prompt: int
    keep_ratio: float
    rank: int              # rank of the per-head shared component
    alpha: float           # weight of the shared component
    sink_rows: Tuple[int, ...] = ()
    sink_scale: float = 1.0
    structure: str = "none"   # none | near_dup | span_repeat | student_t
    v_lowrank: bool = False
    modes: Tuple[int, ...] = (0,)
    seed: int = 0

    @property
    def n_in(self) -> int:
        return self.n_prompt + self.n_c

    @property
    def scale(self) -> np.float32:
        # the model's own attention temperature 1/sqrt(d), rounded to fp32
        return np.float32(1.0 / np.sqrt(self.d))

    @property
    def heads(self) -> int:
        return self.L * self.H

    @property
    def context_pairs(self) -> int:
        return self.L * self.H * self.n_c

    def shrink(self, **kw) -> "Workload":
        """A copy with some fields replaced (used by tests for ragged shapes)."""
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


TINY = Workload(
    name="tiny", cfg_id=0, L=1, H=1, G=4, d=64, n_c=512, n_prompt=16,
    keep_ratio=0.3, rank=4, alpha=2.0, sink_rows=(0,), sink_scale=8.0,
    v_lowrank=True)

LLAMA8B_8K = Workload(
    name="llama3.1-8b-8k", cfg_id=1, L=32, H=8, G=4, d=128, n_c=8192,
    n_prompt=32, keep_ratio=0.3, rank=8, alpha=1.5, sink_rows=(0, 1, 2, 3),
    sink_scale=6.0)

QWEN14B_32K = Workload(
    name="qwen2.5-14b-32k", cfg_id=2, L=48, H=8, G=5, d=128, n_c=32768,
    n_prompt=32, keep_ratio=0.25, rank=8, alpha=1.5, sink_rows=(0, 1, 2, 3),
    sink_scale=6.0, structure="near_dup")

LLAMA8B_128K = Workload(
    name="llama3.1-8b-128k", cfg_id=3, L=32, H=8, G=4, d=128, n_c=131072,
    n_prompt=32, keep_ratio=0.3, rank=8, alpha=1.5, sink_rows=(0, 1, 2, 3),
    sink_scale=6.0, structure="span_repeat")

GEMMA12B_16K = Workload(
    name="gemma3-12b-16k", cfg_id=4, L=48, H=8, G=2, d=256, n_c=16384,
    n_prompt=32, keep_ratio=0.1, rank=16, alpha=1.5, structure="student_t",
    modes=(0, 1))

ALL = (TINY, LLAMA8B_8K, QWEN14B_32K, LLAMA8B_128K, GEMMA12B_16K)
BY_NAME = {w.name: w for w in ALL}

# structure parameters (fixed by the workload descriptions)
NEAR_DUP_FRACTION = 0.10      # share of context keys copied from earlier rows
NEAR_DUP_NOISE_STD = 0.01     # standard deviation of the copy noise
NEAR_DUP_MIN_DST = 5          # copies land on rows >= 5 ...
NEAR_DUP_MIN_SRC = 4          # ... and come from rows in [4, dst)
SPAN_LEN = 64                 # repeated span length
SPAN_PERIOD = 4096            # a span every 4096 tokens
SPAN_SRC = 64                 # the span copied is rows [64, 128)
STUDENT_T_NU = 3.0            # degrees of freedom of the key-norm multiplier
