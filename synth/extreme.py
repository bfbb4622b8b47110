"""Seeded inputs with extreme logit ranges, for the numerical edge cases of
the scoring passes: cached keys whose norms rise or fall by two orders of
magnitude along the context, or a few keys scaled far above the rest.

Only the random recipe lives here (no scoring arithmetic).  With queries
~ N(0, I_d) and a key of norm factor s, the logit scale * <q, k> has standard
deviation s (scale = 1/sqrt(d)), so the shapes below give logits spanning
several hundred natural-log units.
"""
from __future__ import annotations

import numpy as np

from .generate import f64_to_bf16_bits

PROFILES = ("rising", "falling", "spikes")


def key_norm_factors(profile: str, n_c: int, rng: np.random.Generator) -> np.ndarray:
    """Per cached key norm factor s_j."""
    ramp = 1.0 + 149.0 * np.arange(n_c) / max(n_c - 1, 1)    # 1 .. 150
    if profile == "rising":
        return ramp
    if profile == "falling":
        return ramp[::-1].copy()
    if profile == "spikes":
        s = np.ones(n_c)
        spikes = rng.choice(n_c, size=max(1, n_c // 64), replace=False)
        s[spikes] = rng.uniform(40.0, 120.0, size=spikes.size)
        return s
    raise ValueError(f"unknown profile {profile!r}")


def generate_extreme_workload(profile: str, L: int, H: int, G: int, d: int, n_c: int,
                              n_prompt: int, seed: int = 0) -> dict:
    """bf16 bit patterns q [L][H][G][n_in][d], k_ctx and v_ctx [L][H][n_c][d],
    k_new [L][H][n_in][d]; every (l, h) draws from its own seeded stream."""
    n_in = n_prompt + n_c
    out = {"q": np.empty((L, H, G, n_in, d), np.uint16),
           "k_ctx": np.empty((L, H, n_c, d), np.uint16),
           "k_new": np.empty((L, H, n_in, d), np.uint16),
           "v_ctx": np.empty((L, H, n_c, d), np.uint16)}
    for l in range(L):
        for h in range(H):
            ss = np.random.SeedSequence([seed, PROFILES.index(profile), G, d, n_c, n_prompt, l, h])
            rng = np.random.Generator(np.random.PCG64(ss))
            s = key_norm_factors(profile, n_c, rng)
            out["q"][l, h] = f64_to_bf16_bits(rng.standard_normal((G, n_in, d)))
            out["k_ctx"][l, h] = f64_to_bf16_bits(rng.standard_normal((n_c, d)) * s[:, None])
            out["k_new"][l, h] = f64_to_bf16_bits(rng.standard_normal((n_in, d)))
            out["v_ctx"][l, h] = f64_to_bf16_bits(rng.standard_normal((n_c, d)))
    return out
