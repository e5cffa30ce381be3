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
  K3. Update: the plain member mean.  For a group with n_k > 0 members,
      c_kd = (sum over members of x_id) / n_k, taken exactly (rational arithmetic) and
      rounded once to fp32, nearest with ties to even; an empty group keeps its
      centroid.
  K4. The assignments reported are those of the last iteration's assignment step.
  K5. Initial centroids by k-means++ (the configuration's seeded start), drawn by
      inverting the cumulative distribution of the squared distances in row order with
      given uniforms u_0 .. u_{k-1} in [0, 1); the first row is floor(u_0 n).

The assignment here is taken in fp64 from the exact inputs; the GPU takes it in fp32,
so the tests accept any choice whose exact score is within the fp32 error bound of
the minimum (several answers are then correct), and compare the update with the plain
mean of the GPU's assignments.
"""
from __future__ import annotations

import math

import numpy as np


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


def round_to_f32(num: int, den: int) -> np.float32:
    """The rational num / den (den > 0) rounded once to fp32: nearest, ties to even,
    with gradual underflow below 2^-126 (IEEE 754 round-to-nearest-even)."""
    if den <= 0:
        raise ValueError("den must be positive")
    if num == 0:
        return np.float32(0.0)
    a = abs(num)
    e = a.bit_length() - den.bit_length()          # 2^e <= a/den < 2^(e+2)
    if (a << max(0, -e)) < (den << max(0, e)):
        e -= 1                                      # now 2^e <= a/den < 2^(e+1)
    qexp = max(e - 23, -149)                        # the fp32 spacing at that magnitude
    n2, d2 = (a, den << qexp) if qexp >= 0 else (a << -qexp, den)
    q, r = divmod(n2, d2)
    if 2 * r > d2 or (2 * r == d2 and (q & 1)):
        q += 1
    v = math.ldexp(q, qexp)                         # q <= 2^24: exact
    if v >= 2.0 ** 128:
        v = math.inf
    return np.float32(-v if num < 0 else v)


def exact_column_sums(x: np.ndarray) -> tuple[list[int], int]:
    """Exact sums of the columns of a finite fp64 array as (integers S_d, exponent b),
    column sum d = S_d 2^b.  Each x = m 2^e with m 2^53 an integer (frexp), grouped by
    exponent and added in Python integers."""
    x = np.asarray(x, np.float64)
    if x.shape[0] == 0:
        return [0] * x.shape[1], 0
    m, e = np.frexp(x)
    M = (m * 2.0 ** 53).astype(np.int64)            # exact, |M| < 2^53
    base = int(e.min()) - 53
    Mh, Ml = M >> 26, M & ((1 << 26) - 1)           # M = Mh 2^26 + Ml; column sums stay in int64
    sums = [0] * x.shape[1]
    for ev in np.unique(e):
        sel = e == ev
        h = np.where(sel, Mh, 0).sum(axis=0)
        lo = np.where(sel, Ml, 0).sum(axis=0)
        sh = int(ev) - 53 - base
        for d in range(x.shape[1]):
            if h[d] or lo[d]:
                sums[d] += ((int(h[d]) << 26) + int(lo[d])) << sh
    return sums, base


def member_mean(x: np.ndarray) -> np.ndarray:
    """fp32 [D]: the exact mean of the rows of x, each coordinate rounded once."""
    n = x.shape[0]
    sums, b = exact_column_sums(x)
    if b >= 0:
        return np.array([round_to_f32(s << b, n) for s in sums], np.float32)
    return np.array([round_to_f32(s, n << -b) for s in sums], np.float32)


def update(x: np.ndarray, a: np.ndarray, c_prev: np.ndarray) -> np.ndarray:
    """New fp32 centroids from assignments a: each group's plain member mean, exact
    and rounded once; an empty group keeps its centroid (reading K3)."""
    x = check_points(x)
    K = c_prev.shape[0]
    out = np.array(c_prev, np.float32, copy=True)
    for k in range(K):
        members = np.nonzero(a == k)[0]
        if members.size:
            out[k] = member_mean(x[members])
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


def seed_index(u: float, n: int) -> int:
    """Row floor(u n) (at most n - 1) for a uniform u in [0, 1) (reading K5)."""
    return min(int(np.floor(float(np.float32(u)) * n)), n - 1)


def kmeanspp(x: np.ndarray, uniforms: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """(centroids fp32 [k][D], chosen rows [k]): k-means++ seeding (reading K5).

    The first centroid is row floor(u_0 n).  Then, with D2_i the squared distance from
    row i to its nearest chosen centroid, centroid c is the first row i (in row order)
    whose running sum of D2 exceeds u_c * sum(D2), i.e. row i is drawn with probability
    D2_i / sum(D2) by inverting the cumulative sum; if every D2 is 0 the row is
    floor(u_c n).  Distances in fp64 from the exact values.
    """
    x = check_points(x)
    n = x.shape[0]
    u = np.asarray(uniforms, np.float32).astype(np.float64)
    rows = [seed_index(u[0], n)]
    d2 = ((x - x[rows[0]]) ** 2).sum(axis=1)
    for c in range(1, len(u)):
        tot = d2.sum()
        if not tot > 0:
            rows.append(seed_index(u[c], n))
        else:
            cum = np.cumsum(d2)
            i = int(np.searchsorted(cum, u[c] * tot, side="right"))
            rows.append(min(i, n - 1))
        d2 = np.minimum(d2, ((x - x[rows[-1]]) ** 2).sum(axis=1))
    return x[rows].astype(np.float32), np.asarray(rows, np.int64)


def seed_step_valid(x: np.ndarray, rows_before, u: float, row: int, rtol: float) -> bool:
    """Whether `row` is a correct k-means++ draw for uniform u given the rows chosen
    before it: the target u * sum(D2) lies in [cum_{row-1}, cum_row] up to rtol * sum(D2)
    (fp32 sums may move the target across a boundary by that much)."""
    x = check_points(x)
    n = x.shape[0]
    d2 = np.full(n, np.inf)
    for r in rows_before:
        d2 = np.minimum(d2, ((x - x[int(r)]) ** 2).sum(axis=1))
    tot = d2.sum()
    if not tot > 0:
        return row == seed_index(u, n)
    cum = np.cumsum(d2)
    t = float(np.float32(u)) * tot
    lo = cum[row - 1] if row > 0 else 0.0
    return d2[row] > 0 and lo - rtol * tot <= t <= cum[row] + rtol * tot
