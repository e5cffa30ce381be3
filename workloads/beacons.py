"""Seeded history queries for beacon k-means: N(0, 1) rows (the configuration's
history) or well separated groups, as bf16 bit patterns, and initial centroids drawn as
distinct history rows.  Input generation only: no clustering arithmetic lives here."""
from __future__ import annotations

import numpy as np

from .philox import f64_to_bf16_bits

D = 128


def normal_history(rng: np.random.Generator, P: int, N: int) -> np.ndarray:
    """bf16 bits [P][N][128] of N(0, 1) draws."""
    return f64_to_bf16_bits(rng.standard_normal((P, N, D)))


def grouped_history(rng: np.random.Generator, N: int, K: int, spread: float = 4.0, noise: float = 0.3):
    """(bf16 bits [N][128], labels [N]): K groups with N(0, spread^2) centres and
    N(0, noise^2) scatter, every group non-empty (the first K rows are one per group)."""
    centres = rng.normal(0.0, spread, (K, D))
    lab = np.concatenate([np.arange(K), rng.integers(0, K, N - K)]) if N >= K else np.arange(N)
    x = centres[lab] + rng.normal(0.0, noise, (len(lab), D))
    return f64_to_bf16_bits(x), lab


def initial_rows(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """K distinct row indices (all rows, then repeats, when N < K)."""
    if N >= K:
        return rng.choice(N, K, replace=False)
    return np.concatenate([np.arange(N), rng.integers(0, N, K - N)])
