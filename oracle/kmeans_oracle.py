"""Plain, slow CPU oracle for beacon maintenance: Lloyd k-means over a head's
history queries.

TEST INFRASTRUCTURE ONLY. Nothing in the product library may import, call or
execute this module; the tests, the smoke check and the benchmark's CPU baseline
use it.  It shares no code with the HIP path.

Source: "BeaconKV Compresses KV Cache for Long-Reasoning Models with Beacon Queries"
(cctest.ai), Key ideas: queries that revisit distant context fall into a small number
of similarity groups, and one representative per group (a beacon query) stands for the
group alongside the recent queries.

Readings (the page names no algorithm; stated here and in the design notes):
  K1. The groups are found by Lloyd's k-means in squared Euclidean distance, with k
      groups per (layer, query head), over that head's history queries (bf16 rows of
      128), from given initial centroids, for a given number of iterations; the beacons
      are the final centroids rounded to bf16.
  K2. Assignment: a_i = the k minimising ||c_k||^2 - 2 <x_i, c_k> (the squared distance
      less ||x_i||^2); ties go to the lower k.
  K3. Update on a fixed-point grid, so that centroids do not depend on summation order:
      q_id = trunc(x_id 2^16) (exact integers, |x| < 2^15), and for a group with n_k > 0
      members c_kd = fp32(fp64(fp64(sum_i q_id) / n_k) 2^-16), each step rounded to
      nearest; an empty group keeps its centroid.
  K4. The assignments reported are those of the last iteration's assignment step.

The assignment here is taken in fp64 from the exact inputs; the GPU takes it in fp32,
so the tests accept any choice whose exact score is within the fp32 error bound of
the minimum (several answers are then correct), and check the update bit for bit.
"""
from __future__ import annotations

import numpy as np

GRID = 2.0 ** 16


def check_points(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) >= 2.0 ** 15):
        raise ValueError("points must be finite with |x| < 2^15")
    return x


def assign(x: np.ndarray, c: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(a [N], scores [N][K]) with scores = ||c_k||^2 - 2 <x_i, c_k> in fp64 (reading K2)."""
    x = np.asarray(x, np.float64)
    c = np.asarray(c, np.float32).astype(np.float64)
    sc = (c * c).sum(axis=1)[None, :] - 2.0 * (x @ c.T)
    return np.argmin(sc, axis=1), sc          # argmin returns the first (lowest k) minimum


def update(x: np.ndarray, a: np.ndarray, c_prev: np.ndarray) -> np.ndarray:
    """New fp32 centroids from assignments a (reading K3)."""
    x = check_points(x)
    K = c_prev.shape[0]
    q = np.trunc(x * GRID)                    # exact integers below 2^31
    out = np.array(c_prev, np.float32, copy=True)
    for k in range(K):
        members = np.nonzero(a == k)[0]
        if members.size == 0:
            continue
        sums = [sum(int(v) for v in q[members, d]) for d in range(x.shape[1])]   # exact
        out[k] = [np.float32((float(s) / float(members.size)) * (1.0 / GRID)) for s in sums]
    return out


def lloyd(x: np.ndarray, c0: np.ndarray, iters: int) -> tuple[np.ndarray, np.ndarray | None]:
    """(centroids fp32 [K][D], assignments of the last iteration or None) after iters
    Lloyd iterations from c0 (readings K1-K4)."""
    x = check_points(x)
    c = np.array(c0, np.float32, copy=True)
    a = None
    for _ in range(iters):
        a, _ = assign(x, c)
        c = update(x, a, c)
    return c, a


def to_bf16_bits(c: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 bit patterns, nearest with ties to even (finite inputs)."""
    u = np.asarray(c, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)
