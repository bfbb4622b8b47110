"""Seeded synthetic hidden states and KV caches for the EpiKV token score.

Shapes follow the EpiKV page ("EpiKV"): a 32-layer reasoning model (section
1: the two-band anatomy is found in a 32-layer model), reasoning traces of
10^4 - 10^5 decoded tokens with single forward passes up to 65,536 tokens
(figure 1), cache budgets of 4,096 and 8,192 tokens (abstract), bands A and B
scored through layers 10 and 21 (section 3.2, equation 2).  The geometry
(hidden size 4096, 8 KV heads of dimension 128) is that of a public
Llama-8B-class model; every value is synthetic.

Hidden states follow a stationary AR(1) process per layer around a fixed
mean with a few massive channels: most tokens move the state a little, while
"epiphany" tokens (a few percent) move it far.  Band A's step size falls
with position and band B's rises, which is the position confound the page
reports and its equation 3 removes.  Position 0 is an attention-sink-like
outlier.  This module holds no arithmetic of the score itself.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace
from typing import Tuple

import numpy as np

from .generate import default_workers, f64_to_bf16_bits

STREAM_HIDDEN, STREAM_KV, STREAM_EPI = 20, 21, 22


@dataclass(frozen=True)
class EpiWorkload:
    name: str
    cfg_id: int
    L: int                 # layers of the KV cache
    H: int                 # KV heads
    d: int                 # head dimension
    D: int                 # hidden size
    n: int                 # trace length (cached tokens)
    budget: int            # K kept tokens
    band_a: Tuple[int, ...] = (10,)
    band_b: Tuple[int, ...] = (21,)
    window: int = 64
    eps: float = 1e-6
    jump_prob: float = 0.03
    seed: int = 0

    @property
    def layers(self) -> Tuple[int, ...]:
        return self.band_a + self.band_b

    @property
    def kv_pairs(self) -> int:
        return self.L * self.H * self.n

    def shrink(self, **kw) -> "EpiWorkload":
        return replace(self, **kw)


EPIKV_TINY = EpiWorkload("epikv-tiny", 11, L=2, H=2, d=64, D=512, n=700, budget=100,
                         band_a=(1,), band_b=(2,))
EPIKV_R1_8B_64K = EpiWorkload("epikv-r1-8b-64k", 10, L=32, H=8, d=128, D=4096,
                              n=65536, budget=8192)
EPI_ALL = (EPIKV_TINY, EPIKV_R1_8B_64K)
EPI_BY_NAME = {w.name: w for w in EPI_ALL}


def _rng(w: EpiWorkload, a: int, b: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([w.seed, w.cfg_id, a, b, stream])))


def generate_hidden_layer(w: EpiWorkload, layer: int, rising: bool) -> np.ndarray:
    """bf16 bits [n][D] of one layer's hidden states."""
    rng = _rng(w, layer, 0, STREAM_HIDDEN)
    n, D = w.n, w.D
    mu = rng.normal(size=D) * 0.5
    massive = rng.choice(D, size=min(4, D), replace=False)
    mu[massive] = rng.choice([-1.0, 1.0], size=massive.size) * 40.0
    pos = np.arange(n) / max(n - 1, 1)
    sigma = (0.6 + 0.6 * pos) if rising else (1.2 - 0.6 * pos)
    jump = rng.random(n) < w.jump_prob
    rho = np.where(jump, 0.2, 0.9 + 0.08 * rng.random(n))
    out = np.empty((n, D), dtype=np.uint16)
    x = np.zeros(D)
    block = 4096
    for b0 in range(0, n, block):
        b1 = min(n, b0 + block)
        xi = rng.standard_normal(size=(b1 - b0, D))
        rows = np.empty((b1 - b0, D))
        for t in range(b0, b1):
            if t == 0:
                x = 8.0 * sigma[0] * xi[0]
            else:
                x = rho[t] * x + np.sqrt(1.0 - rho[t] ** 2) * sigma[t] * xi[t - b0]
            rows[t - b0] = mu + x
        out[b0:b1] = f64_to_bf16_bits(rows)
    return out


def generate_hidden(w: EpiWorkload, workers: int = 0) -> np.ndarray:
    """bf16 bits [len(band_a) + len(band_b)][n][D], band A's layers first."""
    jobs = [(l, False) for l in w.band_a] + [(l, True) for l in w.band_b]
    workers = workers or min(default_workers(), len(jobs))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        layers = list(ex.map(lambda j: generate_hidden_layer(w, *j), jobs))
    return np.stack(layers)


def generate_kv(w: EpiWorkload) -> Tuple[np.ndarray, np.ndarray]:
    """bf16 bits [L][H][n][d] of the K and V caches (small workloads only)."""
    rng = _rng(w, 0, 0, STREAM_KV)
    shape = (w.L, w.H, w.n, w.d)
    return (f64_to_bf16_bits(rng.normal(size=shape)),
            f64_to_bf16_bits(rng.normal(size=shape)))
