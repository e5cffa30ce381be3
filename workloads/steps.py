"""Seeded reasoning-step structure and attention scores for step-aware ranking.

An agent trajectory alternates short reasoning steps, tool calls and long observations
(tool outputs); each step is a contiguous run of cache entries.  Attention scores are
drawn with a per-step relevance (some steps matter much more than others) times a
per-token spread, and a share of entries with no attention at all.  Input generation
only: none of the ranking's arithmetic lives here.
"""
from __future__ import annotations

import numpy as np

# (kind, mean length in tokens, log-normal sigma)
STEP_KINDS = (("reason", 120, 0.6), ("call", 40, 0.4), ("observe", 700, 0.9))


def step_bounds(rng: np.random.Generator, n: int, empty: float = 0.0) -> np.ndarray:
    """Boundaries 0 = b_0 <= ... <= b_m = n of a trajectory of n entries: steps cycle
    reason -> call -> observe with log-normal lengths; with probability `empty` a
    step is empty (all its entries were evicted earlier)."""
    if n == 0:
        return np.zeros(1, np.int64)
    b = [0]
    pos, kind = 0, 0
    while pos < n:
        _, mean, sig = STEP_KINDS[kind % 3]
        kind += 1
        if rng.random() < empty:
            b.append(pos)
            continue
        ln = max(1, int(rng.lognormal(np.log(mean) - sig * sig / 2, sig)))
        pos = min(n, pos + ln)
        b.append(pos)
    return np.asarray(b, np.int64)


def step_scores(rng: np.random.Generator, bounds: np.ndarray, total: float = 256.0,
                zero: float = 0.1, quantum: float | None = None) -> np.ndarray:
    """fp32 scores of one stream: relevance(step) x Exp(1) per entry, a `zero` share of
    exact zeros, scaled so that they sum to about `total` (the observer rows of a
    round); with `quantum`, values are multiples of it (many exact ties)."""
    n = int(bounds[-1])
    rel = rng.gamma(0.5, 1.0, len(bounds) - 1)
    step_of = np.repeat(np.arange(len(bounds) - 1), np.diff(bounds))
    s = rel[step_of] * rng.exponential(1.0, n)
    s[rng.random(n) < zero] = 0.0
    tot = s.sum()
    if tot > 0:
        s *= total / tot
    if quantum is not None:
        s = np.round(s / quantum) * quantum
    return s.astype(np.float32)


def batch_steps(rng: np.random.Generator, lengths, empty: float = 0.0):
    """(step_off int64 [S+1], first int32 [M], per-sequence bounds list)."""
    bl = [step_bounds(rng, int(n), empty) for n in lengths]
    counts = [len(b) - 1 if int(n) > 0 else 0 for b, n in zip(bl, lengths)]
    off = np.zeros(len(bl) + 1, np.int64)
    off[1:] = np.cumsum(counts)
    first = np.concatenate([b[:-1] for b, c in zip(bl, counts) if c > 0] or [np.zeros(0, np.int64)])
    return off, first.astype(np.int32), bl
