"""Plain, slow CPU oracle for attention-guided KV eviction and paged compaction.

TEST INFRASTRUCTURE ONLY. Nothing in the product library may import, call or
execute this module; it exists so that the tests, the smoke check and the CPU
baseline leg of the benchmark can compare the HIP kernels against an obviously
correct fp64 rendering of the method.  It shares no code with the HIP path.

Sources (cited by page title and section):
  [ActKV]  "ActKV Dissected: 99% of an Agent's KV Cache Is Scratch Work, and the
           Budget Follows Hesitation" (zhichai.net forum write-up of ActKV).
  [Beacon] "BeaconKV Compresses KV Cache for Long-Reasoning Models with Beacon
           Queries" (cctest.ai).

Data model (the same paged layout the library consumes):
  k_pool, v_pool : uint16 bf16 bit patterns [L][P][Hkv][16][D]
  crf_pool       : float32 [L][P][Hkv][16]  (LRFU state, one value per slot)
  block_table    : int32 [S][max_pages]      logical page -> physical page
  start, length  : int32 [S]                 first live slot in logical page 0; live count n
  q              : uint16 bf16 [L][Hq][O_tot][D], lse float32 [L][Hq][O_tot]
  obs_off        : int64 [S+1]               observer rows of sequence i are [obs_off[i], obs_off[i+1])
A *stream* is one (sequence i, layer l, KV head g).  Live slot j of sequence i
sits at logical position start_i + j, i.e. page block_table[i][(start_i+j)//16],
row (start_i+j) % 16.

Precision: every floating-point step is evaluated in fp64 from the exact values
of the stored inputs; results are rounded once to the storage format (fp32).
Where the pages leave a step open, the reading taken is stated at the function.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

PAGE = 16

# ---------------------------------------------------------------------------
# storage helpers
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def slot_location(block_table_row: np.ndarray, start: int, j: np.ndarray):
    """(physical page, row in page) of live slots j of one sequence.

    [ActKV] Component 3: the cache is held in fixed-size blocks addressed through
    logical blocks; live slot j is logical position start + j.
    """
    pos = int(start) + np.asarray(j, dtype=np.int64)
    return np.asarray(block_table_row)[pos // PAGE].astype(np.int64), pos % PAGE


def gather_stream_rows(pool: np.ndarray, layer: int, kv_head: int,
                       block_table_row: np.ndarray, start: int, n: int) -> np.ndarray:
    """Rows of live slots 0..n-1 of one stream, in logical order (raw storage values)."""
    page, row = slot_location(block_table_row, start, np.arange(n))
    return pool[layer, page, kv_head, row]


def observer_rows(q: np.ndarray, lse: np.ndarray, layer: int, kv_head: int, group: int,
                  o0: int, o1: int):
    """Observer rows r = (query head h, observer o) that read KV head g.

    Query head h reads KV head h // G (grouped-query attention), so KV head g is
    read by heads gG .. gG+G-1.  Rows are ordered head-major.
    """
    hs = range(kv_head * group, (kv_head + 1) * group)
    qr = np.concatenate([bf16_bits_to_f64(q[layer, h, o0:o1]) for h in hs], axis=0)
    lr = np.concatenate([lse[layer, h, o0:o1].astype(np.float64) for h in hs], axis=0)
    return qr, lr


# ---------------------------------------------------------------------------
# S1: attention recovered from the log-sum-exp, summed per entry
# ---------------------------------------------------------------------------


def score_stream(q_rows: np.ndarray, lse_rows: np.ndarray, keys: np.ndarray,
                 scale: float) -> np.ndarray:
    """s_j = sum_r exp(scale * <q_r, k_j> - LSE_r), returned as float32.

    [ActKV] Component 3: the log-sum-exp of each query row is a byproduct of the
    paged attention kernel, so the probability that row r puts on entry j is the
    row's logit minus its LSE, exponentiated -- no softmax pass and no attention
    matrix recomputation.  [ActKV] Component 1: each entry's signal is the sum of
    the attention it receives from all observer (action) tokens; the sum also runs
    over the query heads that share the entry's KV head.
    """
    logits = float(scale) * (q_rows @ keys.T)          # [R][n], fp64
    p = np.exp(logits - lse_rows[:, None])
    return p.sum(axis=0).astype(np.float32)


def score(k_pool, q, lse, obs_off, block_table, start, length, num_q_heads, scale,
          streams=None):
    """Scores for every (or the listed) stream: dict (i, l, g) -> float32[n_i]."""
    L, _, Hkv = k_pool.shape[:3]
    G = num_q_heads // Hkv
    out = {}
    todo = streams if streams is not None else [
        (i, l, g) for i in range(len(length)) for l in range(L) for g in range(Hkv)]
    for (i, l, g) in todo:
        n = int(length[i])
        keys = bf16_bits_to_f64(gather_stream_rows(k_pool, l, g, block_table[i], start[i], n))
        qr, lr = observer_rows(q, lse, l, g, G, int(obs_off[i]), int(obs_off[i + 1]))
        if n == 0:
            out[(i, l, g)] = np.zeros(0, np.float32)
        elif qr.shape[0] == 0:
            out[(i, l, g)] = np.zeros(n, np.float32)
        else:
            out[(i, l, g)] = score_stream(qr, lr, keys, scale)
    return out


# ---------------------------------------------------------------------------
# S2: the 90 % attention-mass cut ("action-critical" entries)
# ---------------------------------------------------------------------------


def fixed_point_mass(s: np.ndarray) -> np.ndarray:
    """m_j = floor(s_j * 2^32) as exact integers (s_j >= 0, fp32).

    Integer mass makes the cumulative sums exact, so the cut does not depend on
    summation order.  Multiplying an fp32 value by 2^32 only shifts its exponent,
    so the product is exact in fp64.
    """
    s64 = np.asarray(s, dtype=np.float32).astype(np.float64)
    if np.any(~np.isfinite(s64)) or np.any(s64 < 0):
        raise ValueError("scores must be finite and non-negative")
    return np.floor(s64 * 2.0 ** 32).astype(np.uint64)


def mass_cut(s: np.ndarray, num: int = 9, den: int = 10) -> np.ndarray:
    """hit_j = True for the shortest prefix of the (s desc, j asc) order whose
    integer mass reaches ceil(num/den * M), M = total integer mass.

    [ActKV] Component 1: for each entry the attention from all action tokens is
    tallied and the entries "in the top 90%" are action-critical.  Reading: 90 %
    of the tallied attention *mass* (a percentile of entries would mark 90 % of
    them whatever the attention).  Ties in s are broken by the lower slot index.
    If the total mass is zero there are no hits.
    """
    s = np.asarray(s, dtype=np.float32)
    n = s.shape[0]
    hit = np.zeros(n, dtype=bool)
    if n == 0:
        return hit
    m = fixed_point_mass(s)
    M = int(m.sum(dtype=np.uint64))             # < 2^59: no overflow
    T = -((-num * M) // den)                     # ceil(num*M/den) in integers
    if T <= 0:
        return hit
    order = np.lexsort((np.arange(n), -s.astype(np.float64)))   # s desc, j asc
    cum = np.cumsum(m[order], dtype=np.uint64)
    t = int(np.searchsorted(cum, np.uint64(T), side="left")) + 1  # first cum >= T
    hit[order[:t]] = True
    return hit


# ---------------------------------------------------------------------------
# S3: LRFU update with the "hit by action attention" signal
# ---------------------------------------------------------------------------


def lrfu_decay(lam: float, dt: int) -> np.float32:
    """d = fp32(2^(-lambda * dt)): the LRFU weighting of one elapsed interval.

    [ActKV] Component 1: LRFU with decay coefficient lambda = 0.5.  Reading: dt is
    the number of decode steps since the previous round, and all entries are
    decayed together once per round (the same ranking as lazy LRFU, because all
    entries share the current time).
    """
    return np.float32(np.exp2(-float(lam) * float(dt)))


def fma_f32(a, b, c) -> np.ndarray:
    """Single-rounded fp32 value of a*b + c for fp32 a, b, c (round to nearest even).

    a*b is exact in fp64 (24+24 significant bits).  The sum is taken exactly as
    s + e (Knuth's TwoSum), and s is rounded to fp32; the only case where that
    rounding differs from rounding the exact sum is when s lies exactly halfway
    between two fp32 neighbours, and then the sign of e decides.
    """
    a = np.asarray(a, np.float32).astype(np.float64)
    b = np.asarray(b, np.float32).astype(np.float64)
    c = np.asarray(c, np.float32).astype(np.float64)
    p = a * b
    s = p + c
    bb = s - p
    e = (p - (s - bb)) + (c - bb)
    f = s.astype(np.float32)
    f64 = f.astype(np.float64)
    r = s - f64                                           # exact
    up = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(f, np.float32(-np.inf)).astype(np.float64)
    mid_up = (r > 0) & (r == (up - f64) / 2)
    mid_dn = (r < 0) & (r == (dn - f64) / 2)
    out = f.copy()
    fix_up = mid_up & (e > 0)
    fix_dn = mid_dn & (e < 0)
    out = np.where(fix_up, np.nextafter(f, np.float32(np.inf)), out)
    out = np.where(fix_dn, np.nextafter(f, np.float32(-np.inf)), out)
    return out.astype(np.float32)


def lrfu_update(crf_prev: np.ndarray, hit: np.ndarray, d: np.float32, n_prev: int) -> np.ndarray:
    """CRF_j <- hit_j + d * CRF_j (single fp32 rounding); CRF_j <- hit_j for j >= n_prev.

    [ActKV] Component 1: LRFU (the classic page-replacement policy) with its hit
    replaced by "hit by action attention".  The combined recency-frequency value
    of an entry is F(0) = 1 for a hit now plus the previous value weighted by
    2^(-lambda*dt).  Entries appended since the previous round have no history:
    their prior is 0 whatever the reused page memory holds.
    """
    crf_prev = np.asarray(crf_prev, np.float32)
    n = crf_prev.shape[0]
    hitf = np.asarray(hit, bool).astype(np.float32)
    prior = crf_prev.copy()
    prior[min(max(int(n_prev), 0), n):] = 0.0
    return fma_f32(np.full(n, d, np.float32), prior, hitf)


# ---------------------------------------------------------------------------
# S4: per-(layer, KV head) top-B keep set
# ---------------------------------------------------------------------------


def select_top_b(crf: np.ndarray, s: np.ndarray, budget: int) -> np.ndarray:
    """keep = the first min(B, n) entries of the order (CRF desc, s desc, j asc).

    [ActKV] Summary / Results: eviction retains an entry budget.  Reading: the
    budget applies to each (layer, KV head) stream, exactly min(B, n) entries are
    kept, and ties in CRF (common: every hit of the same round has the same CRF
    when dt is large) are broken by this round's attention s, then by slot index.
    """
    crf = np.asarray(crf, np.float32)
    s = np.asarray(s, np.float32)
    n = crf.shape[0]
    keep = np.zeros(n, dtype=bool)
    K = min(int(budget), n)
    if K <= 0:
        return keep
    order = np.lexsort((np.arange(n), -s.astype(np.float64), -crf.astype(np.float64)))
    keep[order[:K]] = True
    return keep


# ---------------------------------------------------------------------------
# S5: the one-way budget ratchet
# ---------------------------------------------------------------------------

RATCHET_INITIAL = 512
RATCHET_NUM, RATCHET_DEN = 7, 4          # x1.75 exactly
RATCHET_CAP = 30000


def ratchet(budget: int, flag: bool, num: int = RATCHET_NUM, den: int = RATCHET_DEN,
            cap: int = RATCHET_CAP) -> int:
    """B <- min(cap, floor(B * 1.75)) when the low-confidence flag fires; never shrinks.

    [ActKV] Component 2: a declining-confidence signal expands the entry budget by
    1.75x up to 30,000; expansion is one-way.  [ActKV] Lineage: the adaptive mode
    starts at 512.
    """
    if not flag:
        return int(budget)
    return max(int(budget), min(int(cap), (int(budget) * num) // den))


# ---------------------------------------------------------------------------
# S6: conflict-free slot plan
# ---------------------------------------------------------------------------


def plan_stream(keep: np.ndarray):
    """Move pairs (src slot -> dst slot) for one stream.

    [ActKV] Component 3: survivors skew toward the tail, so the tail becomes the
    target region; survivors outside it are paired one-to-one with holes inside it
    and all pairs are copied in one pass.  Reading: the target is the last K live
    slots (slot-granular), K = number kept, so the counts match exactly.  With
    D = n - K: sources are the kept slots j < D in ascending order, destinations
    the evicted slots j >= D in ascending order, paired in order.
    """
    keep = np.asarray(keep, bool)
    n = keep.shape[0]
    K = int(keep.sum())
    D = n - K
    src = np.nonzero(keep[:D])[0].astype(np.int32)
    dst = (np.nonzero(~keep[D:])[0] + D).astype(np.int32)
    assert src.shape == dst.shape
    return src, dst


def plan_sequence(n: int, kept: int, start: int, block_table_row: np.ndarray):
    """Host bookkeeping of one sequence after compaction.

    [ActKV] Component 3: freed blocks are returned to the scheduler.  Every stream
    of a sequence keeps the same count, so the live region becomes logical
    positions start + D .. start + n - 1 for all of them: the first
    shift = (start + D) // 16 logical pages are free, the new first-slot offset is
    (start + D) % 16 and the new length is K.
    """
    D = int(n) - int(kept)
    shift = (int(start) + D) // PAGE
    new_start = (int(start) + D) % PAGE
    freed = np.asarray(block_table_row[:shift], dtype=np.int32).copy()
    return shift, new_start, int(kept), freed


# ---------------------------------------------------------------------------
# S7: in-place compaction
# ---------------------------------------------------------------------------


def compact_stream(k_pool, v_pool, crf_pool, layer, kv_head, block_table_row, start,
                   src, dst):
    """Copy the K row, V row and CRF of every source slot onto its destination slot.

    [ActKV] Component 3: one parallel pass, no extra KV buffer.  Sources and
    destinations are disjoint, so the pairs may be applied in any order.  Pools are
    modified in place; every byte other than the destination rows is unchanged.
    """
    if len(src) == 0:
        return
    ps, rs = slot_location(block_table_row, start, src)
    pd, rd = slot_location(block_table_row, start, dst)
    k_pool[layer, pd, kv_head, rd] = k_pool[layer, ps, kv_head, rs]
    v_pool[layer, pd, kv_head, rd] = v_pool[layer, ps, kv_head, rs]
    crf_pool[layer, pd, kv_head, rd] = crf_pool[layer, ps, kv_head, rs]


# ---------------------------------------------------------------------------
# one full eviction round
# ---------------------------------------------------------------------------


def eviction_round(k_pool, v_pool, crf_pool, q, lse, obs_off, block_table, start, length,
                   num_q_heads, scale, lam, dt, n_prev, budget, mass_num=9, mass_den=10,
                   streams=None):
    """Score -> cut -> LRFU -> top-B -> plan -> compact, on the given pools (modified in place).

    Returns per-stream dicts of s, hit, crf (after the update), keep, (src, dst),
    and per-sequence (shift, new_start, new_len, freed).  With streams=None every
    stream is processed; otherwise only the listed (i, l, g) streams (the host
    bookkeeping is per sequence and does not depend on the stream set).
    """
    L, _, Hkv = k_pool.shape[:3]
    S = len(length)
    todo = streams if streams is not None else [
        (i, l, g) for i in range(S) for l in range(L) for g in range(Hkv)]
    scores = score(k_pool, q, lse, obs_off, block_table, start, length, num_q_heads, scale,
                   streams=todo)
    res = {"s": scores, "hit": {}, "crf": {}, "keep": {}, "pairs": {}, "seq": {}}
    for (i, l, g) in todo:
        n = int(length[i])
        s = scores[(i, l, g)]
        hit = mass_cut(s, mass_num, mass_den)
        d = lrfu_decay(lam, int(dt[i]))
        page, row = slot_location(block_table[i], start[i], np.arange(n))
        crf_prev = crf_pool[l, page, g, row]
        crf_new = lrfu_update(crf_prev, hit, d, int(n_prev[i]))
        crf_pool[l, page, g, row] = crf_new
        keep = select_top_b(crf_new, s, int(budget[i]))
        src, dst = plan_stream(keep)
        compact_stream(k_pool, v_pool, crf_pool, l, g, block_table[i], start[i], src, dst)
        res["hit"][(i, l, g)] = hit
        res["crf"][(i, l, g)] = crf_new
        res["keep"][(i, l, g)] = keep
        res["pairs"][(i, l, g)] = (src, dst)
    for i in range(S):
        n = int(length[i])
        K = min(int(budget[i]), n)
        res["seq"][i] = plan_sequence(n, K, int(start[i]), block_table[i])
    return res


# ---------------------------------------------------------------------------
# exact rational helpers (used by the self-tests of this module)
# ---------------------------------------------------------------------------


def round_fraction_to_f32(x: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32 (ties to even), subnormals included."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    while Fraction(2) ** (e + 1) <= x:
        e += 1
    e = max(e, -126)                     # below the normal range the grid is fixed
    ulp = Fraction(2) ** (e - 23)
    q = x / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * ulp
    if val >= Fraction(2) ** 128:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(val))
