"""Plain, slow CPU oracle for step-aware ranking of cache entries (StepKV).

TEST INFRASTRUCTURE ONLY. Nothing in the product library may import, call or
execute this module; the tests, the smoke check and the benchmark's CPU baseline
use it.  It shares no code with the HIP path.

Source: "StepKV: Step-Aware KV Cache Compression for LLM Agents" (mlsanity.com),
Abstract: reasoning steps are the retention unit; every cache entry is associated
with the step that generated it; a step's utility is estimated from signals taken
from the trajectory and combined with token-level saliency; the combined scores
rank the prunable tokens globally and the top-scoring ones are kept under a target
budget.

Readings (the page gives the method in outline only; stated here and in the design
notes):
  S1. A sequence's live entries are cut into steps, contiguous runs given by
      boundaries 0 = b_0 <= b_1 <= ... <= b_m = n (step k holds entries
      b_k .. b_{k+1}-1).  Every layer and KV head uses the same boundaries.
  S2. Token saliency is the entry's attention score s_j of the stream (what the
      observer scorer or the decode tally produces).
  S3. Step utility is the attention the step receives per entry: the mean of s over
      the step's entries.  It is taken on the fixed-point grid of the mass cut
      (a_j = floor(s_j 2^32), exact integers), U_int = floor(sum a_j / len), and
      rounded once to fp32: U = fp32(U_int 2^-32).  An empty step has U = 0.
  S4. The combination is convex with a caller weight beta in [0, 1]:
      c_j = fp32(beta * U + fp32(fp32(1 - beta) * s_j)), one fused multiply-add.
  S5. Every live entry is prunable.  Per stream, exactly K = min(B, n) entries are
      kept: the first K of the order (c desc, s desc, slot asc).

Integer and exact-rounding arithmetic throughout, so the keep set is defined to the
bit.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

from .kvs_oracle import fixed_point_mass, fma_f32, round_fraction_to_f32, select_top_b


def check_bounds(bounds, n: int) -> np.ndarray:
    b = np.asarray(bounds, np.int64)
    if b.ndim != 1 or b.shape[0] < 2 or b[0] != 0 or b[-1] != n or np.any(np.diff(b) < 0):
        raise ValueError("step boundaries must run from 0 to n without decreasing")
    return b


def step_utility(s: np.ndarray, bounds) -> np.ndarray:
    """U_k (fp32) for every step k of one stream (reading S3)."""
    s = np.asarray(s, np.float32)
    b = check_bounds(bounds, s.shape[0])
    a = fixed_point_mass(s)
    out = np.zeros(b.shape[0] - 1, np.float32)
    for k in range(b.shape[0] - 1):
        lo, hi = int(b[k]), int(b[k + 1])
        if hi == lo:
            continue
        total = sum(int(x) for x in a[lo:hi])          # exact
        u_int = total // (hi - lo)
        out[k] = round_fraction_to_f32(Fraction(u_int, 2 ** 32))
    return out


def step_utility_mean(s: np.ndarray, bounds) -> np.ndarray:
    """The plain step mean, for comparison with reading S3: U_k = (sum of s over the
    step) / len, taken exactly from the fp32 scores and rounded once to fp32.  S3's grid
    mean differs from it by at most 2^-31 plus one fp32 spacing of U: each
    floor(s 2^32) loses less than one grid unit, so the grid sum is within len units
    of sum(s) 2^32, and the floored quotient within 2 units of the exact mean; the two
    roundings to fp32 add half a spacing each."""
    s = np.asarray(s, np.float32)
    b = check_bounds(bounds, s.shape[0])
    out = np.zeros(b.shape[0] - 1, np.float32)
    for k in range(b.shape[0] - 1):
        lo, hi = int(b[k]), int(b[k + 1])
        if hi > lo:
            out[k] = round_fraction_to_f32(sum(Fraction(float(x)) for x in s[lo:hi]) / (hi - lo))
    return out


def step_keys(s: np.ndarray, bounds, beta: float) -> tuple[np.ndarray, np.ndarray]:
    """(c [n] fp32, U [steps] fp32): c_j = beta U_step(j) + (1 - beta) s_j (reading S4)."""
    s = np.asarray(s, np.float32)
    b = check_bounds(bounds, s.shape[0])
    beta32 = np.float32(beta)
    if not (0.0 <= float(beta32) <= 1.0):
        raise ValueError("beta must lie in [0, 1]")
    u = step_utility(s, b)
    step_of = np.repeat(np.arange(b.shape[0] - 1), np.diff(b))
    w = np.float32(np.float32(1.0) - beta32)
    t = (w * s).astype(np.float32)                       # fp32 products, rounded to nearest
    c = fma_f32(np.full(s.shape[0], beta32, np.float32), u[step_of], t)
    return c, u


def step_select(s: np.ndarray, bounds, beta: float, budget: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(keep [n] bool, c [n], U [steps]) of one stream (reading S5)."""
    c, u = step_keys(s, bounds, beta)
    return select_top_b(c, s, budget), c, u
