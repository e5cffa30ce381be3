"""Plain, slow CPU oracle for the confidence monitor that drives the budget ratchet.

TEST INFRASTRUCTURE ONLY. Nothing in the product library may import, call or
execute this module; the tests, the smoke check and the benchmark's CPU baseline
use it to check the HIP kernels against an obviously correct fp64 rendering.
It shares no code with the HIP path.

Source: "ActKV Dissected: 99% of an Agent's KV Cache Is Scratch Work, and the
Budget Follows Hesitation" (zhichai.net), Component 2 (budget follows hesitation)
and the Summary.  The pages describe the monitor in four steps:
  1. per decode step, hesitation is measured as the average negative
     log-probability of the 20 most probable tokens of that step's output
     distribution;
  2. these token-level values are turned into a trajectory-level confidence
     series by min-pooling over sliding windows of 64 tokens, stride 8;
  3. a linear fit over that series with a negative slope means the budget is too
     small;
  4. which raises the ratchet flag (the 1.75x expansion is kvs_oracle.ratchet).
Readings where the pages leave a step open are stated at each function.

Precision: every step is evaluated in fp64 from the exact stored input values.
"""
from __future__ import annotations

import numpy as np

TOP_K = 20        # Component 2: top-20 tokens
WINDOW = 64       # Component 2: min-pooling window
STRIDE = 8        # Component 2: min-pooling stride


def log_sum_exp(z: np.ndarray) -> float:
    """ln sum_j exp(z_j) in fp64, shifted by the maximum (z finite or -inf)."""
    z = np.asarray(z, dtype=np.float64)
    m = float(np.max(z))
    if m == -np.inf:
        return -np.inf
    return m + float(np.log(np.sum(np.exp(z - m))))


def token_confidence(logits_row: np.ndarray, k: int = TOP_K) -> float:
    """Mean negative log-probability of the k most probable tokens of one step.

    [ActKV] Component 2.  Reading: the step's output distribution is the softmax
    of its logits z over the vocabulary (temperature 1); the k most probable tokens
    are the k largest logits (which k-subset is taken among equal logits does not
    change the mean); the log is natural.  With p_j = exp(z_j - LSE(z)):
        c = (1/k) * sum over the top k of (-ln p_j) = LSE(z) - mean(top-k z).
    A peaked distribution gives a large c (the runners-up are improbable); a flat
    one gives c close to ln(vocab): c is a confidence, and its collapses are what
    the min-pooling looks for.
    """
    z = np.asarray(logits_row, dtype=np.float64).ravel()
    if not 1 <= k <= z.size:
        raise ValueError("need 1 <= k <= vocab")
    top = np.sort(z)[::-1][:k]           # library sort as the selection step
    return log_sum_exp(z) - float(np.mean(top))


def min_pool(conf: np.ndarray, window: int = WINDOW, stride: int = STRIDE) -> np.ndarray:
    """Trajectory-level confidence: the minimum of each window of `window`
    consecutive token values, windows starting every `stride` tokens.

    [ActKV] Component 2 (sliding-window min-pooling, window 64, stride 8).
    Reading: only full windows count; the windows start at 0, stride, 2*stride, ...
    while start + window <= T.  A trajectory shorter than one window has no
    pooled values.
    """
    c = np.asarray(conf, dtype=np.float64).ravel()
    out = []
    s = 0
    while s + window <= c.size:
        out.append(float(np.min(c[s:s + window])))
        s += stride
    return np.array(out, dtype=np.float64)


def lsq_slope(y: np.ndarray) -> float | None:
    """Ordinary least-squares slope of y against its index 0, 1, ..., P-1.

    [ActKV] Component 2 (a linear fit over trajectory-level confidence).  Reading:
    the abscissa is the window index; fewer than two points have no slope (None).
        slope = sum (x - xbar)(y - ybar) / sum (x - xbar)^2
    """
    y = np.asarray(y, dtype=np.float64).ravel()
    if y.size < 2:
        return None
    x = np.arange(y.size, dtype=np.float64)
    xb = x.mean()
    yb = y.mean()
    return float(np.sum((x - xb) * (y - yb)) / np.sum((x - xb) ** 2))


def trend_flag(conf: np.ndarray, window: int = WINDOW, stride: int = STRIDE,
               fit_last: int = 0) -> tuple[float | None, int, bool]:
    """(slope, pooled count, flag) for a trajectory's token confidences.

    [ActKV] Component 2: a negative slope of the fitted line means information was
    compressed away, and the budget expands.  Reading: the fit covers the last
    `fit_last` pooled values (0 = all of the trajectory's pooled values); the flag is
    slope < 0, and no slope means no flag.
    """
    pooled = min_pool(conf, window, stride)
    if fit_last > 0:
        pooled = pooled[-fit_last:]
    slope = lsq_slope(pooled)
    return slope, int(min_pool(conf, window, stride).size), bool(slope is not None and slope < 0)
