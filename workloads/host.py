"""Host (numpy) generation of the synthetic inputs, shared by the oracle side and
the GPU side of the tests.  It holds none of the eviction method's arithmetic:
only layouts, random draws, planted keys, k-means beacons and the log-sum-exp
that the upstream paged-attention decode kernel would hand over.

Every value is a pure function of (workload key, tensor tag, element index), so
any stream can be regenerated alone, in any order.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import philox
from .configs import (OBS_MAX, TAG_CRF, TAG_DT, TAG_HDT, TAG_HIST, TAG_K, TAG_KMPP, TAG_LAYOUT,
                      TAG_LEN, TAG_OBS, TAG_PLANT, TAG_Q, TAG_V, TOKENS_MAX, Workload)

PAGE = 16


@dataclass
class Layout:
    block_table: np.ndarray      # int32 [S][max_pages], unused entries -1
    start: np.ndarray            # int32 [S]
    length: np.ndarray           # int32 [S]
    obs: np.ndarray              # int32 [S] observers per sequence
    obs_off: np.ndarray          # int64 [S+1]
    entry_off: np.ndarray        # int64 [S+1]
    num_pages: int
    dt: np.ndarray               # int32 [S]
    n_prev: np.ndarray           # int32 [S]
    tok0: np.ndarray             # int64 [S]: token id of live slot 0 (slot j holds token tok0+j)


def _pages_needed(start, n):
    return (int(start) + int(n) + PAGE - 1) // PAGE


def make_layout(w: Workload) -> Layout:
    S = w.num_seqs
    key = w.key
    if w.len_lo == w.len_hi:
        length = np.full(S, w.len_lo, np.int64)
    else:
        length = philox.randint(key, TAG_LEN, S, w.len_lo, w.len_hi)
    if w.obs_lo == w.obs_hi:
        obs = np.full(S, w.obs_lo, np.int64)
    else:
        obs = philox.randint(key, TAG_OBS, S, w.obs_lo, w.obs_hi)
    if w.dt_lo == w.dt_hi:
        dt = np.full(S, w.dt_lo, np.int64)
    else:
        dt = philox.randint(key, TAG_DT, S, w.dt_lo, w.dt_hi)
    start = np.zeros(S, np.int64)
    npg = np.array([_pages_needed(start[i], length[i]) for i in range(S)], np.int64)
    max_pages = int(npg.max()) if S else 0
    bt = np.full((S, max_pages), -1, np.int64)
    if w.page_placement == "in_order":
        P = w.pool_pages or int(npg.sum())
        nxt = 0
        for i in range(S):
            bt[i, :npg[i]] = np.arange(nxt, nxt + npg[i])
            nxt += npg[i]
    elif w.page_placement in ("random", "permutation"):
        P = w.pool_pages or int(npg.sum())
        perm = philox.permutation(key, TAG_LAYOUT, P)
        nxt = 0
        for i in range(S):
            bt[i, :npg[i]] = perm[nxt:nxt + npg[i]]
            nxt += npg[i]
        assert nxt <= P
    elif w.page_placement == "interleaved":
        # pages handed out round-robin, as if all sequences grew in lockstep
        P = int(npg.sum())
        nxt = 0
        for p in range(max_pages):
            for i in range(S):
                if p < npg[i]:
                    bt[i, p] = nxt
                    nxt += 1
    else:
        raise ValueError(w.page_placement)
    obs_off = np.zeros(S + 1, np.int64)
    obs_off[1:] = np.cumsum(obs)
    entry_off = np.zeros(S + 1, np.int64)
    entry_off[1:] = np.cumsum(length)
    n_prev = length.copy() if w.prior_crf else np.zeros(S, np.int64)
    return Layout(bt.astype(np.int32), start.astype(np.int32), length.astype(np.int32),
                  obs.astype(np.int32), obs_off, entry_off, int(P), dt.astype(np.int32),
                  n_prev.astype(np.int32), np.zeros(S, np.int64))


def history_dt(w: Workload) -> np.ndarray:
    """int32 [history_rounds][S]: the decode steps between the history rounds that
    precede the measured round, uniform in [dt_lo, dt_hi].  History round r (1-based)
    uses the observer set of round index r (observers(..., rnd=r))."""
    H, S = w.history_rounds, w.num_seqs
    if H == 0:
        return np.zeros((0, S), np.int32)
    return philox.randint(w.key, TAG_HDT, H * S, w.dt_lo, w.dt_hi).reshape(H, S).astype(np.int32)


# ---------------------------------------------------------------------------
# element-indexed draws
# ---------------------------------------------------------------------------


def _token_index(w: Workload, i, l, g, t):
    return ((((np.int64(i) * w.num_layers + l) * w.num_kv_heads + g) * TOKENS_MAX)
            + np.asarray(t, np.int64))


def token_normals(w: Workload, tag: int, i: int, l: int, g: int, tokens: np.ndarray) -> np.ndarray:
    """N(0,1) fp64 [len(tokens)][D]: element (token t, dim d) uses Philox index
    token_index*D + d (D = 128 is a multiple of 4, so each row is 32 whole counters)."""
    D = w.head_dim
    tok = _token_index(w, i, l, g, np.asarray(tokens, np.int64)).astype(np.uint64)
    ctr = (tok[:, None] * np.uint64(D // 4) + np.arange(D // 4, dtype=np.uint64)[None, :]).reshape(-1)
    w0, w1, w2, w3 = philox.words(w.key, tag, ctr)
    u0, u1, u2, u3 = (philox.uniform01(x) for x in (w0, w1, w2, w3))
    r0 = np.sqrt(-2.0 * np.log(u0))
    r1 = np.sqrt(-2.0 * np.log(u2))
    z = np.stack([r0 * np.cos(2.0 * np.pi * u1), r0 * np.sin(2.0 * np.pi * u1),
                  r1 * np.cos(2.0 * np.pi * u3), r1 * np.sin(2.0 * np.pi * u3)], axis=1)
    return z.reshape(len(tok), D)


def observer_normals(w: Workload, rnd: int, i: int, l: int, h: int, o: np.ndarray) -> np.ndarray:
    """N(0,1) fp64 [len(o)][D] for observer o of (round, sequence, layer, query head)."""
    D = w.head_dim
    base = (((np.int64(rnd) * w.num_seqs + i) * w.num_layers + l) * w.num_q_heads + h) * OBS_MAX
    tok = (base + np.asarray(o, np.int64)).astype(np.uint64)
    ctr = (tok[:, None] * np.uint64(D // 4) + np.arange(D // 4, dtype=np.uint64)[None, :]).reshape(-1)
    w0, w1, w2, w3 = philox.words(w.key, TAG_Q, ctr)
    u0, u1, u2, u3 = (philox.uniform01(x) for x in (w0, w1, w2, w3))
    r0 = np.sqrt(-2.0 * np.log(u0))
    r1 = np.sqrt(-2.0 * np.log(u2))
    z = np.stack([r0 * np.cos(2.0 * np.pi * u1), r0 * np.sin(2.0 * np.pi * u1),
                  r1 * np.cos(2.0 * np.pi * u3), r1 * np.sin(2.0 * np.pi * u3)], axis=1)
    return z.reshape(len(tok), D)


def history_normals(w: Workload, l: int, h: int, count: int) -> np.ndarray:
    """The beacon history: count N(0,1) queries of (layer, query head), fp64 [count][D]."""
    D = w.head_dim
    base = (np.int64(l) * w.num_q_heads + h) * TOKENS_MAX
    tok = (base + np.arange(count, dtype=np.int64)).astype(np.uint64)
    ctr = (tok[:, None] * np.uint64(D // 4) + np.arange(D // 4, dtype=np.uint64)[None, :]).reshape(-1)
    w0, w1, w2, w3 = philox.words(w.key, TAG_HIST, ctr)
    u0, u1, u2, u3 = (philox.uniform01(x) for x in (w0, w1, w2, w3))
    r0 = np.sqrt(-2.0 * np.log(u0))
    r1 = np.sqrt(-2.0 * np.log(u2))
    z = np.stack([r0 * np.cos(2.0 * np.pi * u1), r0 * np.sin(2.0 * np.pi * u1),
                  r1 * np.cos(2.0 * np.pi * u3), r1 * np.sin(2.0 * np.pi * u3)], axis=1)
    return z.reshape(count, D)


def kmeans_beacons(w: Workload, l: int, h: int) -> np.ndarray:
    """k cluster centroids (fp64 [k][D]) of the (layer, head) query history.

    BeaconKV, Key ideas: revisit-related queries form a few similarity groups and
    one representative per group is kept.  Lloyd's algorithm in fp64 with a seeded
    k-means++ start and a fixed number of iterations; an empty cluster keeps its
    previous centroid.
    """
    X = history_normals(w, l, h, w.beacon_history)
    k = w.beacons
    idx = (np.int64(l) * w.num_q_heads + h) * 64
    draws = philox.uniform01(np.stack(philox.words(w.key, TAG_KMPP,
                                                   np.arange(idx, idx + k, dtype=np.uint64)),
                                      axis=1)[:, 0])
    cent = np.empty((k, X.shape[1]))
    cent[0] = X[min(int(draws[0] * len(X)), len(X) - 1)]
    d2 = ((X - cent[0]) ** 2).sum(1)
    for c in range(1, k):
        cdf = np.cumsum(d2)
        pick = int(np.searchsorted(cdf, draws[c] * cdf[-1], side="right"))
        cent[c] = X[min(pick, len(X) - 1)]
        d2 = np.minimum(d2, ((X - cent[c]) ** 2).sum(1))
    xx = (X * X).sum(1)
    for _ in range(w.kmeans_iters):
        dist = xx[:, None] - 2.0 * X @ cent.T + (cent * cent).sum(1)[None, :]
        a = np.argmin(dist, axis=1)
        for c in range(k):
            m = a == c
            if m.any():
                cent[c] = X[m].mean(0)
    return cent


def observers(w: Workload, lay: Layout, rnd: int = 0, heads=None, only_heads: bool = False,
              rest_zero: bool = False) -> np.ndarray:
    """Observer queries, bf16 bits [L][Hq][O_tot][D].

    heads: optional set of (l, h) for which k-means beacons are computed on the
    host; beacon rows of other heads are left as plain N(0,1) draws (callers that
    need them fill them in elsewhere).
    only_heads: the listed heads get the counter-based draws; every other head gets
    N(0,1) from numpy's seeded PCG64 (much faster, for full-size workloads whose
    other heads are never compared with the oracle), or zeros with rest_zero.
    """
    L, Hq, D = w.num_layers, w.num_q_heads, w.head_dim
    O_tot = int(lay.obs_off[-1])
    q = np.empty((L, Hq, O_tot, D), np.uint16)
    if only_heads:
        if rest_zero:
            q[:] = 0
        else:
            rng = np.random.default_rng([w.key & 0xFFFFFFFF, w.key >> 32, rnd])
            for l in range(L):
                q[l] = philox.f32_to_bf16_bits(rng.standard_normal((Hq, O_tot, D), dtype=np.float32))
        for (l, h) in sorted(heads or ()):
            for i in range(w.num_seqs):
                o0, o1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
                if o1 == o0:
                    continue
                z = observer_normals(w, rnd, i, l, h, np.arange(o1 - o0))
                if w.beacons:
                    z[:w.beacons] = kmeans_beacons(w, l, h)
                q[l, h, o0:o1] = philox.f64_to_bf16_bits(z)
        return q
    for i in range(w.num_seqs):
        o0, o1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
        if o1 == o0:
            continue
        for l in range(L):
            # all heads of (sequence, layer) at once; the same draws as observer_normals
            z = _observer_normals_heads(w, rnd, i, l, np.arange(o1 - o0))
            if w.beacons:
                for h in range(Hq):
                    if heads is None or (l, h) in heads:
                        z[h, :w.beacons] = kmeans_beacons(w, l, h)
            q[l, :, o0:o1] = philox.f64_to_bf16_bits(z)
    return q


def _observer_normals_heads(w: Workload, rnd: int, i: int, l: int, o: np.ndarray) -> np.ndarray:
    """observer_normals for every query head of (round, sequence, layer): fp64 [Hq][len(o)][D]."""
    D = w.head_dim
    h = np.arange(w.num_q_heads, dtype=np.int64)
    base = (((np.int64(rnd) * w.num_seqs + i) * w.num_layers + l) * w.num_q_heads + h) * OBS_MAX
    tok = (base[:, None] + np.asarray(o, np.int64)[None, :]).reshape(-1).astype(np.uint64)
    ctr = (tok[:, None] * np.uint64(D // 4) + np.arange(D // 4, dtype=np.uint64)[None, :]).reshape(-1)
    w0, w1, w2, w3 = philox.words(w.key, TAG_Q, ctr)
    u0, u1, u2, u3 = (philox.uniform01(x) for x in (w0, w1, w2, w3))
    r0 = np.sqrt(-2.0 * np.log(u0))
    r1 = np.sqrt(-2.0 * np.log(u2))
    z = np.stack([r0 * np.cos(2.0 * np.pi * u1), r0 * np.sin(2.0 * np.pi * u1),
                  r1 * np.cos(2.0 * np.pi * u3), r1 * np.sin(2.0 * np.pi * u3)], axis=1)
    return z.reshape(w.num_q_heads, len(o), D)


def stream_observer_rows(w: Workload, lay: Layout, q: np.ndarray, i: int, l: int, g: int) -> np.ndarray:
    """fp64 [R][D] observer rows of stream (i, l, g), head-major (r = (h - gG)*O + o)."""
    o0, o1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
    G = w.group
    rows = [philox.bf16_bits_to_f32(q[l, h, o0:o1]).astype(np.float64)
            for h in range(g * G, (g + 1) * G)]
    return np.concatenate(rows, axis=0)


def stream_keys(w: Workload, q_rows: np.ndarray, i: int, l: int, g: int,
                tokens: np.ndarray, planted_frac: float | None = None) -> np.ndarray:
    """K rows (bf16 bits [len(tokens)][D]) for the given tokens of a stream.

    A fraction of keys is planted to draw attention: for a token whose Philox word
    falls under f * 2^32, one observer row r is picked (second word, scaled to R)
    and the key becomes 3 * q_r / |q_r| + z, where z is the token's own N(0,1) draw.
    """
    f = w.planted_frac if planted_frac is None else planted_frac
    z = token_normals(w, TAG_K, i, l, g, tokens)
    if f > 0 and q_rows.shape[0] > 0:
        tok = _token_index(w, i, l, g, np.asarray(tokens, np.int64)).astype(np.uint64)
        w0, w1, _, _ = philox.words(w.key, TAG_PLANT, tok)
        thr = np.uint64(int(f * 4294967296.0))
        planted = w0.astype(np.uint64) < thr
        R = q_rows.shape[0]
        r = ((w1.astype(np.uint64) * np.uint64(R)) >> np.uint64(32)).astype(np.int64)
        qn = q_rows / np.sqrt((q_rows * q_rows).sum(1))[:, None]
        z[planted] = 3.0 * qn[r[planted]] + z[planted]
    return philox.f64_to_bf16_bits(z)


def stream_values(w: Workload, i: int, l: int, g: int, tokens: np.ndarray) -> np.ndarray:
    return philox.f64_to_bf16_bits(token_normals(w, TAG_V, i, l, g, tokens))


def stream_prior_crf(w: Workload, i: int, l: int, g: int, tokens: np.ndarray) -> np.ndarray:
    """Prior CRF in [0, 2) per token (fp32), the range a binary-hit LRFU history reaches."""
    tok = _token_index(w, i, l, g, np.asarray(tokens, np.int64)).astype(np.uint64)
    w0, _, _, _ = philox.words(w.key, TAG_CRF, tok)
    return (2.0 * (w0.astype(np.float64) * (1.0 / 4294967296.0))).astype(np.float32)


def lse_rows(q_rows: np.ndarray, keys_bits: np.ndarray, scale: float) -> np.ndarray:
    """Natural-log LSE of each observer row over the live keys, fp64 rounded to fp32.

    This stands in for the log-sum-exp that a paged decode-attention kernel returns
    as a byproduct (same scale, same live entries, no causal mask).
    """
    keys = philox.bf16_bits_to_f32(keys_bits).astype(np.float64)
    x = scale * (q_rows @ keys.T)
    m = x.max(axis=1)
    return (m + np.log(np.exp(x - m[:, None]).sum(axis=1))).astype(np.float32)


@dataclass
class HostInputs:
    """Full pools for small workloads (every stream generated on the host)."""
    k_pool: np.ndarray       # uint16 [L][P][Hkv][16][D]
    v_pool: np.ndarray
    crf_pool: np.ndarray     # float32 [L][P][Hkv][16]
    q: np.ndarray            # uint16 [L][Hq][O_tot][D]
    lse: np.ndarray          # float32 [L][Hq][O_tot]


def full_inputs(w: Workload, lay: Layout, q: np.ndarray | None = None, rnd: int = 0) -> HostInputs:
    L, Hkv, D = w.num_layers, w.num_kv_heads, w.head_dim
    P = lay.num_pages
    if q is None:
        q = observers(w, lay, rnd)
    k_pool = np.zeros((L, P, Hkv, PAGE, D), np.uint16)
    v_pool = np.zeros((L, P, Hkv, PAGE, D), np.uint16)
    crf_pool = np.zeros((L, P, Hkv, PAGE), np.float32)
    lse = np.zeros(q.shape[:3], np.float32)
    G = w.group
    for i in range(w.num_seqs):
        n = int(lay.length[i])
        st = int(lay.start[i])
        pos = st + np.arange(n)
        page = lay.block_table[i][pos // PAGE]
        row = pos % PAGE
        tokens = lay.tok0[i] + np.arange(n)
        o0, o1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
        for l in range(L):
            for g in range(Hkv):
                qr = stream_observer_rows(w, lay, q, i, l, g)
                kb = stream_keys(w, qr, i, l, g, tokens)
                k_pool[l, page, g, row] = kb
                v_pool[l, page, g, row] = stream_values(w, i, l, g, tokens)
                if w.prior_crf:
                    crf_pool[l, page, g, row] = stream_prior_crf(w, i, l, g, tokens)
                if qr.shape[0] and n:
                    lr = lse_rows(qr, kb, w.scale)
                    O = o1 - o0
                    for hh in range(G):
                        lse[l, g * G + hh, o0:o1] = lr[hh * O:(hh + 1) * O]
    return HostInputs(k_pool, v_pool, crf_pool, q, lse)
