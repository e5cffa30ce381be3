"""Seeded synthetic decode-step logits for the confidence monitor (test and benchmark
plumbing; none of the monitor's arithmetic lives here).

A row stands for one decode step's output logits over a vocabulary.  Recipe
(numpy PCG64, seed per call):
  * the long tail: -6 + 1.5 N(0, 1) per token;
  * the step's plausible continuations: m ~ U{2..8} distinct random tokens; the
    leading one sits at `boost`, the others at U(-1, 1);
  * the boost is the step's sharpness: a trajectory passes its own per-step values
    in (above about 4, a larger boost means a more confident step; around 1 the
    leader is one of several equal alternatives: a hesitant step).
Special rows for edge cases: constant rows (all ties), ascending rows, rows whose
large values all sit in positions that one GPU thread owns, rows with -inf tokens.
bf16 rows are rounded to nearest even from fp32.
"""
from __future__ import annotations

import numpy as np

from .philox import f32_to_bf16_bits

LLAMA3_VOCAB = 128256


def lm_rows(seed: int, rows: int, vocab: int, boost=None) -> np.ndarray:
    """fp32 [rows][vocab] LM-like logits; boost: per-row sharpness (default U[4, 16))."""
    rng = np.random.default_rng(seed)
    z = np.float32(-6.0) + rng.standard_normal((rows, vocab), dtype=np.float32) * np.float32(1.5)
    b = rng.uniform(4.0, 16.0, rows) if boost is None else np.broadcast_to(np.asarray(boost, np.float64), (rows,))
    for r in range(rows):
        m = min(int(rng.integers(2, 9)), vocab)
        toks = rng.choice(vocab, size=m, replace=False)
        z[r, toks[1:]] = rng.uniform(-1.0, 1.0, m - 1).astype(np.float32)
        z[r, toks[0]] = np.float32(b[r])
    return z


def lm_rows_device(seed: int, rows: int, vocab: int, device, dtype):
    """The same recipe drawn on the device with torch's seeded generator (large
    benchmark batches): tail -6 + 1.5 N(0,1), 8 candidate slots per row at random
    positions (collisions allowed), the first at U[4, 16), the rest at U(-1, 1)."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    z = torch.randn((rows, vocab), generator=g, device=device, dtype=torch.float32).mul_(1.5).sub_(6.0)
    pos = torch.randint(0, vocab, (rows, 8), generator=g, device=device)
    val = torch.rand((rows, 8), generator=g, device=device) * 2.0 - 1.0
    val[:, 0] = torch.rand((rows,), generator=g, device=device) * 12.0 + 4.0
    z.scatter_(1, pos, val)
    return z.to(dtype)


def special_rows(seed: int, vocab: int) -> np.ndarray:
    """fp32 [6][vocab]: constant, ascending, descending, thread-clustered maxima,
    half -inf, and all but three tokens -inf."""
    rng = np.random.default_rng(seed)
    out = np.empty((6, vocab), np.float32)
    out[0] = 1.5
    out[1] = np.linspace(-5.0, 5.0, vocab, dtype=np.float32)
    out[2] = out[1][::-1]
    out[3] = rng.standard_normal(vocab).astype(np.float32)
    # every 4096th position (one thread's slice of a chunk) gets the largest values
    out[3, ::4096] += np.float32(20.0) + rng.random(out[3, ::4096].size).astype(np.float32)
    out[4] = rng.standard_normal(vocab).astype(np.float32) * 3
    out[4, rng.permutation(vocab)[: vocab // 2]] = -np.inf
    out[5] = -np.inf
    out[5, rng.choice(vocab, size=min(3, vocab), replace=False)] = np.float32([2.0, 1.0, 0.5][: min(3, vocab)])
    return out


def to_bf16_bits(z: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of fp32 values (round to nearest even; +-inf kept)."""
    return f32_to_bf16_bits(np.asarray(z, np.float32))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def trajectory_boost(seed: int, steps: int, drift: float, collapses=()) -> np.ndarray:
    """Per-step sharpness of a decode trajectory: 12 + N(0, 0.8^2) noise, changing
    linearly by `drift` from the first step to the last, and dropping to 1 for 16
    steps from each position in `collapses`."""
    rng = np.random.default_rng(seed)
    b = 12.0 + rng.standard_normal(steps) * 0.8 + np.linspace(0.0, drift, steps)
    for s in collapses:
        b[s:s + 16] = 1.0
    return b
