"""Small seeded batches for edge-case parity tests: ragged lengths, start offsets,
observer counts on both sides of the MFMA threshold, several layers and heads.

Host-only generation (numpy); the LSE is the exact fp64 log-sum-exp rounded to
fp32, as a paged decode kernel would return it.
"""
from __future__ import annotations

import numpy as np

from . import philox
from .host import PAGE, HostInputs, Layout


def random_batch(seed: int, L: int, Hkv: int, Hq: int, lengths, starts, observers,
                 spare_pages: int = 3, prior_crf: bool = True, planted: float = 0.05,
                 key_scale: float = 1.0):
    """Build (Layout, HostInputs) for a batch with the given per-sequence shapes.

    Pages are a random permutation of the pool (distinct across sequences); the
    pool has `spare_pages` unused pages whose contents are random too.
    """
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, np.int64)
    starts = np.asarray(starts, np.int64)
    observers = np.asarray(observers, np.int64)
    S = len(lengths)
    npg = np.array([(int(starts[i]) + int(lengths[i]) + PAGE - 1) // PAGE if lengths[i] else 0
                    for i in range(S)], np.int64)
    P = int(npg.sum()) + spare_pages
    perm = rng.permutation(P)
    mp = max(int(npg.max()) if S else 0, 1)
    bt = np.full((S, mp), -1, np.int64)
    nxt = 0
    for i in range(S):
        bt[i, :npg[i]] = perm[nxt:nxt + npg[i]]
        nxt += npg[i]
    obs_off = np.zeros(S + 1, np.int64)
    obs_off[1:] = np.cumsum(observers)
    entry_off = np.zeros(S + 1, np.int64)
    entry_off[1:] = np.cumsum(lengths)
    D = 128
    G = Hq // Hkv
    O_tot = int(obs_off[-1])
    q = philox.f64_to_bf16_bits(rng.standard_normal((L, Hq, max(O_tot, 0), D)))
    k = philox.f64_to_bf16_bits(key_scale * rng.standard_normal((L, P, Hkv, PAGE, D)))
    v = philox.f64_to_bf16_bits(rng.standard_normal((L, P, Hkv, PAGE, D)))
    crf = (2.0 * rng.random((L, P, Hkv, PAGE))).astype(np.float32) if prior_crf else \
        np.zeros((L, P, Hkv, PAGE), np.float32)
    lse = np.zeros((L, Hq, O_tot), np.float32)
    scale = 1.0 / np.sqrt(D)
    for i in range(S):
        n, st = int(lengths[i]), int(starts[i])
        o0, o1 = int(obs_off[i]), int(obs_off[i + 1])
        if n == 0 or o1 == o0:
            continue
        pos = st + np.arange(n)
        pg, row = bt[i][pos // PAGE], pos % PAGE
        for l in range(L):
            for g in range(Hkv):
                qr = np.concatenate([philox.bf16_bits_to_f32(q[l, h, o0:o1]).astype(np.float64)
                                     for h in range(g * G, (g + 1) * G)])
                if planted > 0:
                    pm = rng.random(n) < planted
                    r = rng.integers(0, qr.shape[0], n)
                    z = philox.bf16_bits_to_f32(k[l, pg, g, row]).astype(np.float64)
                    qn = qr / np.linalg.norm(qr, axis=1, keepdims=True)
                    z[pm] = 3.0 * qn[r[pm]] + z[pm]
                    k[l, pg, g, row] = philox.f64_to_bf16_bits(z)
                keys = philox.bf16_bits_to_f32(k[l, pg, g, row]).astype(np.float64)
                x = scale * (qr @ keys.T)
                m = x.max(1)
                lr = (m + np.log(np.exp(x - m[:, None]).sum(1))).astype(np.float32)
                O = o1 - o0
                for hh in range(G):
                    lse[l, g * G + hh, o0:o1] = lr[hh * O:(hh + 1) * O]
    n_prev = lengths.copy() if prior_crf else np.zeros(S, np.int64)
    lay = Layout(bt.astype(np.int32), starts.astype(np.int32), lengths.astype(np.int32),
                 observers.astype(np.int32), obs_off, entry_off, P,
                 rng.integers(1, 65, S).astype(np.int32), n_prev.astype(np.int32),
                 np.zeros(S, np.int64))
    return lay, HostInputs(k, v, crf, q, lse)


CRAFTED_KINDS = ("quantised", "zeros_and_tiny", "dominant", "uniform", "all_zero", "low_bits",
                 "large", "below_grid", "subnormal_mix")


def crafted_scores(rng: np.random.Generator, n: int, kind: str) -> np.ndarray:
    """fp32 [n] scores built to stress the attention-mass cut: many exact duplicates at
    the crossing value, zero and sub-grid (< 2^-32) values, one dominant entry, values
    that differ only in their low mantissa bits, and values near the top of the range."""
    if kind == "quantised":                       # 9 levels k 2^-10: every level a large tie class
        s = rng.integers(0, 9, n) * 2.0 ** -10
    elif kind == "zeros_and_tiny":                # 60 % zeros, 20 % below 2^-32, 20 % two levels
        u = rng.random(n)
        s = np.where(u < 0.6, 0.0, np.where(u < 0.8, 2.0 ** rng.uniform(-60, -33, n),
                                             rng.integers(1, 3, n) * 2.0 ** -9))
    elif kind == "dominant":                      # one entry with nearly all of the mass
        s = np.full(n, 2.0 ** -20)
        s[rng.integers(0, n)] = 1000.0
    elif kind == "uniform":
        s = np.full(n, 0.0078125)
    elif kind == "all_zero":
        s = np.zeros(n)
    elif kind == "low_bits":                      # same exponent and high bits, few low-bit patterns
        s = 2.0 ** -8 * (1.0 + rng.integers(0, 4, n) * 2.0 ** -22)
    elif kind == "large":                         # masses near 2^42 mixed with small ones
        s = np.where(rng.random(n) < 0.01, 1023.5, rng.integers(0, 3, n) * 0.25)
    elif kind == "below_grid":                    # positive scores, all of zero integer mass
        s = 2.0 ** rng.uniform(-80, -32.5, n)
    elif kind == "subnormal_mix":                 # fp32 subnormals (mass 0) among two levels
        s = np.where(rng.random(n) < 0.5, rng.integers(1, 100, n) * 2.0 ** -149,
                     rng.integers(1, 3, n) * 2.0 ** -12)
    else:
        raise ValueError(kind)
    return np.asarray(s, np.float32)


def quantised_priors(rng: np.random.Generator, shape) -> np.ndarray:
    """Prior CRF values from a few levels, so that updated CRFs tie exactly."""
    return rng.choice(np.array([0.0, 0.25, 0.5, 1.0, 1.5], np.float32), shape)
