"""Pins of the fp64 oracle to things other than itself: the mathematics (closed
forms, invariants, brute force on tiny inputs), library routines for special
cases, and the hand-worked values under tests/golden/ (each cited there).

Each pin is chosen so that a plausible slip in the oracle (dropped scale, wrong
LSE sign, wrong GQA head mapping, transposed operand, off-by-one in the cut, a
wrong tie-break, a wrong pairing) fails at least one test here.
"""
import itertools
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle as O

rng = np.random.default_rng(1234)


def bf16(x):
    """fp32 -> bf16 bits by truncation-free rounding through numpy (test-local helper)."""
    x = np.asarray(x, np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def make_pool(L, P, Hkv, D=128, seed=0):
    r = np.random.default_rng(seed)
    k = bf16(r.standard_normal((L, P, Hkv, 16, D)).astype(np.float32))
    v = bf16(r.standard_normal((L, P, Hkv, 16, D)).astype(np.float32))
    crf = r.random((L, P, Hkv, 16)).astype(np.float32)
    return k, v, crf


# ---------------------------------------------------------------------------
# S1 score
# ---------------------------------------------------------------------------


def _exact_lse(qr, keys, scale):
    return scipy.special.logsumexp(scale * (qr @ keys.T), axis=1)


def test_single_row_is_textbook_softmax():
    """R = 1: the recovered attention is the softmax row (scipy's routine)."""
    D, n = 128, 300
    keys = O.bf16_bits_to_f64(bf16(rng.standard_normal((n, D))))
    q = O.bf16_bits_to_f64(bf16(rng.standard_normal((1, D))))
    scale = 1.0 / np.sqrt(128.0)
    s = O.score_stream(q, _exact_lse(q, keys, scale), keys, scale)
    ref = scipy.special.softmax(scale * (q @ keys.T)[0])
    np.testing.assert_allclose(s, ref.astype(np.float32), rtol=2e-7, atol=0)


def test_rows_sum_to_one_and_total_mass_is_R():
    """Each softmax row sums to 1, so the per-entry tally sums to the row count R."""
    D, n, R = 128, 500, 24
    keys = O.bf16_bits_to_f64(bf16(rng.standard_normal((n, D))))
    q = O.bf16_bits_to_f64(bf16(rng.standard_normal((R, D))))
    scale = 1.0 / np.sqrt(128.0)
    lse = _exact_lse(q, keys, scale)
    p = np.exp(scale * (q @ keys.T) - lse[:, None])
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-12)
    s = O.score_stream(q, lse, keys, scale)
    assert abs(float(s.astype(np.float64).sum()) - R) < 1e-4


def test_lse_recovered_equals_recomputed():
    """With the fp32 LSE a decode kernel returns, p = exp(logit - LSE) matches the
    directly normalised softmax to the LSE's rounding (|dLSE| <= 2^-24 |LSE|)."""
    D, n, R = 128, 4096, 8
    keys = O.bf16_bits_to_f64(bf16(rng.standard_normal((n, D))))
    q = O.bf16_bits_to_f64(bf16(rng.standard_normal((R, D))))
    scale = 1.0 / np.sqrt(128.0)
    lse32 = _exact_lse(q, keys, scale).astype(np.float32).astype(np.float64)
    s = O.score_stream(q, lse32, keys, scale).astype(np.float64)
    direct = scipy.special.softmax(scale * (q @ keys.T), axis=1).sum(0)
    np.testing.assert_allclose(s, direct, rtol=3e-6)


def test_identical_keys_give_uniform_attention():
    D, n, R = 128, 64, 12
    k1 = bf16(rng.standard_normal(D))
    keys = O.bf16_bits_to_f64(np.tile(k1, (n, 1)))
    q = O.bf16_bits_to_f64(bf16(rng.standard_normal((R, D))))
    scale = 1.0 / np.sqrt(128.0)
    s = O.score_stream(q, _exact_lse(q, keys, scale), keys, scale)
    np.testing.assert_allclose(s, np.float32(R / n), rtol=1e-6)


def test_scale_is_applied():
    """A missing or doubled 1/sqrt(D) would change which entries dominate."""
    D, n = 128, 50
    keys = O.bf16_bits_to_f64(bf16(rng.standard_normal((n, D))))
    q = O.bf16_bits_to_f64(bf16(3 * rng.standard_normal((1, D))))
    for scale in (1.0 / np.sqrt(128.0), 0.25):
        s = O.score_stream(q, _exact_lse(q, keys, scale), keys, scale)
        ref = scipy.special.softmax(scale * (q @ keys.T)[0])
        np.testing.assert_allclose(s, ref, rtol=2e-6)


def _paged_case(L=2, Hkv=2, Hq=4, n=37, start=5, P=12, O_=3, seed=7):
    r = np.random.default_rng(seed)
    k, v, crf = make_pool(L, P, Hkv, seed=seed)
    npg = (start + n + 15) // 16
    bt = r.permutation(P)[:npg].astype(np.int32)[None, :]
    q = bf16(r.standard_normal((L, Hq, O_, 128)).astype(np.float32))
    lse = (np.log(n) + 0.5 + 0.1 * r.standard_normal((L, Hq, O_))).astype(np.float32)
    return k, v, crf, bt, q, lse


def test_gqa_head_mapping():
    """Query head h reads KV head h // G.  Zero queries give logit 0 everywhere, so with
    LSE = ln n the heads that read KV head 1 put exactly 1/n on every entry."""
    L, Hkv, Hq, n, start, P, O_ = 1, 2, 4, 40, 0, 4, 3
    k, v, crf, bt, q, lse = _paged_case(L, Hkv, Hq, n, start, P, O_)
    q[0, 2:4] = 0                     # heads 2, 3 -> KV head 1 when G = 2
    lse[0, 2:4] = np.float32(np.log(n))
    obs_off = np.array([0, O_])
    s = O.score(k, q, lse, obs_off, bt, np.array([start]), np.array([n]), Hq, 1 / np.sqrt(128))
    R = 2 * O_
    expect = np.float32(R * np.exp(-np.float64(np.float32(np.log(n))) + np.log(n)) / n)
    np.testing.assert_allclose(s[(0, 0, 1)], expect, rtol=1e-6)
    assert np.std(s[(0, 0, 0)]) > 1e-3 * np.mean(s[(0, 0, 0)])


def test_page_placement_and_start_offset_do_not_change_scores():
    """The same logical keys at other physical pages, or after a start offset,
    give the same scores (block-table indirection, not physical order)."""
    L, Hkv, Hq, n, P, O_ = 1, 1, 2, 45, 8, 4
    r = np.random.default_rng(3)
    keys = bf16(r.standard_normal((n, 128)).astype(np.float32))
    q = bf16(r.standard_normal((L, Hq, O_, 128)).astype(np.float32))
    lse = (np.log(n) + 0.5 + 0.1 * r.standard_normal((L, Hq, O_))).astype(np.float32)
    obs_off = np.array([0, O_])
    outs = []
    for start, perm_seed in ((0, 0), (9, 1), (15, 2)):
        k = np.zeros((L, P, Hkv, 16, 128), np.uint16)
        npg = (start + n + 15) // 16
        bt = np.random.default_rng(perm_seed).permutation(P)[:npg].astype(np.int32)
        pos = start + np.arange(n)
        k[0, bt[pos // 16], 0, pos % 16] = keys
        outs.append(O.score(k, q, lse, obs_off, bt[None, :], np.array([start]), np.array([n]),
                            Hq, 1 / np.sqrt(128))[(0, 0, 0)])
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def test_key_permutation_equivariance_and_row_order_invariance():
    D, n, R = 128, 77, 9
    keys = O.bf16_bits_to_f64(bf16(rng.standard_normal((n, D))))
    q = O.bf16_bits_to_f64(bf16(rng.standard_normal((R, D))))
    scale = 1 / np.sqrt(128)
    lse = _exact_lse(q, keys, scale)
    s = O.score_stream(q, lse, keys, scale)
    perm = rng.permutation(n)
    s2 = O.score_stream(q, lse, keys[perm], scale)
    np.testing.assert_allclose(s2, s[perm], rtol=1e-6)
    rp = rng.permutation(R)
    s3 = O.score_stream(q[rp], lse[rp], keys, scale)
    np.testing.assert_allclose(s3, s, rtol=1e-6)


def test_score_brute_force_tiny():
    """n <= 8, R <= 3: pure-Python loops with math.fsum over the exact products."""
    import math
    D = 128
    for trial in range(5):
        n, R = 1 + trial, 1 + trial % 3
        keys = O.bf16_bits_to_f64(bf16(rng.standard_normal((n, D))))
        q = O.bf16_bits_to_f64(bf16(rng.standard_normal((R, D))))
        lse = rng.standard_normal(R) + 2.0
        scale = 1 / math.sqrt(128)
        s = O.score_stream(q, lse, keys, scale)
        for j in range(n):
            tot = math.fsum(math.exp(scale * math.fsum(q[r, d] * keys[j, d] for d in range(D)) - lse[r])
                            for r in range(R))
            assert abs(float(s[j]) - tot) <= 1e-6 * tot


# ---------------------------------------------------------------------------
# S2 mass cut
# ---------------------------------------------------------------------------


def _brute_cut(s, num=9, den=10):
    """Smallest subset size reaching the integer target, and the ranked order."""
    m = [int(Fraction(float(np.float32(x))) * 2 ** 32) for x in s]     # floor of exact product
    M = sum(m)
    T = -((-num * M) // den)
    n = len(s)
    if T <= 0:
        return 0, M, T
    for size in range(1, n + 1):
        if max(sum(m[j] for j in c) for c in itertools.combinations(range(n), size)) >= T:
            return size, M, T
    raise AssertionError


@pytest.mark.parametrize("seed", range(40))
def test_mass_cut_brute_force(seed):
    r = random.Random(seed)
    n = r.randint(1, 9)
    vals = [r.choice([0.0, 0.125, 0.5, 1.0, 3.0]) if r.random() < 0.3 else r.random() for _ in range(n)]
    s = np.array(vals, np.float32)
    hit = O.mass_cut(s)
    size, M, T = _brute_cut(s)
    assert hit.sum() == size
    m = [int(Fraction(float(x)) * 2 ** 32) for x in s]
    assert sum(m[j] for j in range(n) if hit[j]) >= T
    # every hit ranks before every non-hit in (s desc, j asc)
    for a in range(n):
        for b in range(n):
            if hit[a] and not hit[b]:
                assert (s[a] > s[b]) or (s[a] == s[b] and a < b)


def test_mass_cut_uniform_closed_form():
    for n in (1, 7, 10, 11, 100, 4096):
        s = np.full(n, 1.0 / n, np.float32)
        assert O.mass_cut(s).sum() == -((-9 * n) // 10)       # ceil(0.9 n)


def test_mass_cut_dominant_entry_and_zero_mass():
    s = np.full(50, 0.001, np.float32)
    s[17] = 10.0
    hit = O.mass_cut(s)
    assert hit.sum() == 1 and hit[17]
    assert O.mass_cut(np.zeros(20, np.float32)).sum() == 0
    assert O.mass_cut(np.full(20, 1e-12, np.float32)).sum() == 0      # below 2^-32: no mass
    assert O.mass_cut(np.zeros(0, np.float32)).sum() == 0


def test_mass_cut_ties_take_lower_slot():
    s = np.array([0.25, 0.25, 0.25, 0.25], np.float32)     # needs ceil(3.6)=4? no: 0.9*4 -> 4 of 4
    assert O.mass_cut(s).tolist() == [True] * 4
    s = np.array([0.1] * 10, np.float32)                    # 9 of 10, the last one left out
    assert O.mass_cut(s).tolist() == [True] * 9 + [False]
    s = np.array([0.05, 0.3, 0.3, 0.35], np.float32)        # 0.35, 0.3 (j=1), 0.3 (j=2) = 0.95 >= 0.9
    assert O.mass_cut(s).tolist() == [False, True, True, True]


def test_mass_cut_rejects_invalid():
    with pytest.raises(ValueError):
        O.mass_cut(np.array([0.5, np.nan], np.float32))
    with pytest.raises(ValueError):
        O.mass_cut(np.array([0.5, -0.1], np.float32))


# ---------------------------------------------------------------------------
# S3 LRFU
# ---------------------------------------------------------------------------


def _load_lrfu_golden(golden_dir):
    rows = []
    for line in open(os.path.join(golden_dir, "lrfu_hand_worked.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        lam, dt, hits, hx, _ = line.split()
        rows.append((float(lam), int(dt), [int(h) for h in hits.split(",")], int(hx, 16)))
    return rows


def test_lrfu_hand_worked_golden(golden_dir):
    rows = _load_lrfu_golden(golden_dir)
    assert len(rows) >= 8
    for lam, dt, hits, hx in rows:
        crf = np.zeros(1, np.float32)
        n_prev = 0
        for h in hits:
            crf = O.lrfu_update(crf, np.array([bool(h)]), O.lrfu_decay(lam, dt), n_prev)
            n_prev = 1
        assert int(crf.view(np.uint32)[0]) == hx, (lam, dt, hits, hex(int(crf.view(np.uint32)[0])))


def test_lrfu_closed_form_power_of_two_decay():
    """With d = 2^-b and few enough rounds that every term fits in fp32's 24 bits, the
    iterated update equals the closed form CRF_k = sum_j hit_j d^(k-j) + d^k CRF_0."""
    r = np.random.default_rng(5)
    for lam, dt in ((0.5, 2), (0.5, 4), (1.0, 3), (0.25, 8)):
        d = O.lrfu_decay(lam, dt)
        b = int(round(lam * dt))
        assert float(d) == 2.0 ** (-b)
        rounds = (24 - 5) // b
        hits = r.random((rounds, 30)) < 0.6
        crf0 = (r.integers(0, 8, 30) / 4).astype(np.float32)
        crf = crf0.copy()
        for k in range(rounds):
            crf = O.lrfu_update(crf, hits[k], d, 30)
        for e in range(30):
            exact = sum(Fraction(int(hits[k, e])) * Fraction(float(d)) ** (rounds - 1 - k)
                        for k in range(rounds))
            exact += Fraction(float(d)) ** rounds * Fraction(float(crf0[e]))
            assert Fraction(float(crf[e])) == exact


def test_lrfu_new_entries_have_zero_prior():
    crf = np.array([1.5, 1.5, 7.0, 9.0], np.float32)     # slots 2, 3 hold stale page memory
    out = O.lrfu_update(crf, np.array([False, True, False, True]), np.float32(0.5), 2)
    assert out.tolist() == [0.75, 1.75, 0.0, 1.0]


def test_fma_single_rounding_against_exact_rationals():
    r = np.random.default_rng(9)
    a = r.random(2000).astype(np.float32)
    b = (r.random(2000) * 2).astype(np.float32)
    c = (r.random(2000) < 0.5).astype(np.float32)
    # adversarial: products that land on fp32 midpoints after adding 1
    a[:200] = np.float32(2.0 ** -24)
    b[:200] = np.float32(1.0) + np.float32(2.0 ** -23) * r.integers(0, 8, 200).astype(np.float32)
    c[:200] = 1.0
    a[200:400] = np.float32(2.0 ** -25)
    b[200:400] = np.float32(1.0) + np.float32(2.0 ** -23) * r.integers(1, 8, 200).astype(np.float32)
    c[200:400] = 1.0
    got = O.fma_f32(a, b, c)
    for i in range(len(a)):
        exact = Fraction(float(a[i])) * Fraction(float(b[i])) + Fraction(float(c[i]))
        assert got[i] == O.round_fraction_to_f32(exact), i


def test_round_fraction_to_f32_matches_numpy_on_doubles():
    """Rounding an fp64 value's exact rational equals numpy's fp64 -> fp32 cast."""
    r = np.random.default_rng(2)
    xs = np.concatenate([r.standard_normal(500), r.random(200) * 1e-38, r.random(100) * 1e-44])
    for x in xs:
        assert O.round_fraction_to_f32(Fraction(float(x))) == np.float32(x)


# ---------------------------------------------------------------------------
# S4 select
# ---------------------------------------------------------------------------


def _brute_select(crf, s, B):
    n = len(crf)
    keep = []
    for j in range(n):
        before = 0
        for i in range(n):
            if i == j:
                continue
            if (crf[i] > crf[j]) or (crf[i] == crf[j] and s[i] > s[j]) or \
               (crf[i] == crf[j] and s[i] == s[j] and i < j):
                before += 1
        keep.append(before < B)
    return np.array(keep)


@pytest.mark.parametrize("seed", range(30))
def test_select_brute_force(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(0, 13))
    crf = r.choice(np.array([0.0, 1.0, 1.5, 0.25], np.float32), n)
    s = r.choice(np.array([0.1, 0.2, 0.3], np.float32), n)
    for B in (0, 1, 3, n, n + 4):
        keep = O.select_top_b(crf, s, B)
        assert keep.sum() == min(B, n)
        np.testing.assert_array_equal(keep, _brute_select(crf, s, B))


def test_select_tie_breaks():
    crf = np.array([1.0, 1.0, 1.0, 0.5], np.float32)
    s = np.array([0.1, 0.3, 0.3, 0.9], np.float32)
    assert O.select_top_b(crf, s, 1).tolist() == [False, True, False, False]
    assert O.select_top_b(crf, s, 2).tolist() == [False, True, True, False]
    assert O.select_top_b(crf, s, 3).tolist() == [True, True, True, False]


# ---------------------------------------------------------------------------
# S5 ratchet
# ---------------------------------------------------------------------------


def test_ratchet_golden_sequence(golden_dir):
    vals = [int(x) for x in open(os.path.join(golden_dir, "ratchet_sequence.txt"))
            if x.strip() and not x.startswith("#")]
    B = O.RATCHET_INITIAL
    seq = [B]
    for _ in range(len(vals) - 1):
        B = O.ratchet(B, True)
        seq.append(B)
    assert seq == vals
    assert O.ratchet(896, False) == 896          # no flag: unchanged
    # "six doublings of headroom": log2(30000/512) ~ 5.87, eight x1.75 steps to the cap
    assert sum(1 for a, b in zip(vals, vals[1:]) if b > a) == 8


# ---------------------------------------------------------------------------
# S6 / S7 plan + compact
# ---------------------------------------------------------------------------


def _apply(ids, src, dst, order):
    out = ids.copy()
    for t in order:
        out[dst[t]] = ids[src[t]]
    return out


@pytest.mark.parametrize("n", range(0, 11))
def test_plan_every_keep_mask(n):
    for bits in range(1 << n):
        keep = np.array([(bits >> j) & 1 for j in range(n)], bool)
        src, dst = O.plan_stream(keep)
        K = int(keep.sum())
        D = n - K
        assert len(src) == len(dst)
        assert set(src.tolist()).isdisjoint(dst.tolist())
        assert len(set(dst.tolist())) == len(dst)
        assert all(j < D and keep[j] for j in src)
        assert all(j >= D and not keep[j] for j in dst)
        assert np.all(np.diff(src) > 0) and np.all(np.diff(dst) > 0)        # monotone pairing
        ids = np.arange(n)
        out = _apply(ids, src, dst, range(len(src)))
        assert sorted(out[D:].tolist()) == np.nonzero(keep)[0].tolist()     # exactly the kept rows
        for j in range(D, n):                                               # stayers unmoved
            if keep[j]:
                assert out[j] == j
        moved = [out[j] for j in range(D, n) if out[j] != j]
        assert moved == sorted(moved)                                        # moved rows keep order
        if len(src) > 1:
            np.testing.assert_array_equal(out, _apply(ids, src, dst, reversed(range(len(src)))))


@pytest.mark.parametrize("start", [0, 7, 15])
def test_plan_sequence_and_compact_bytes(start):
    r = np.random.default_rng(start)
    L, Hkv, P = 2, 2, 10
    for n in (1, 15, 16, 17, 40, 100):
        npg = (start + n + 15) // 16
        if npg > P:
            continue
        k, v, crf = make_pool(L, P, Hkv, seed=n)
        bt = r.permutation(P)[:npg].astype(np.int32)
        K = int(r.integers(0, n + 1))
        shift, new_start, new_len, freed = O.plan_sequence(n, K, start, bt)
        D = n - K
        assert shift * 16 + new_start == start + D and 0 <= new_start < 16 and new_len == K
        np.testing.assert_array_equal(freed, bt[:shift])
        for l in range(L):
            for g in range(Hkv):
                keep = np.zeros(n, bool)
                keep[r.choice(n, K, replace=False)] = True
                src, dst = O.plan_stream(keep)
                k0, v0, c0 = k.copy(), v.copy(), crf.copy()
                O.compact_stream(k, v, crf, l, g, bt, start, src, dst)
                ps, rs = O.slot_location(bt, start, src)
                pd, rd = O.slot_location(bt, start, dst)
                ek, ev, ec = k0.copy(), v0.copy(), c0.copy()
                for t in range(len(src)):
                    ek[l, pd[t], g, rd[t]] = k0[l, ps[t], g, rs[t]]
                    ev[l, pd[t], g, rd[t]] = v0[l, ps[t], g, rs[t]]
                    ec[l, pd[t], g, rd[t]] = c0[l, ps[t], g, rs[t]]
                np.testing.assert_array_equal(k, ek)
                np.testing.assert_array_equal(v, ev)
                np.testing.assert_array_equal(crf.view(np.uint32), ec.view(np.uint32))
                # the live region after compaction holds exactly the kept rows of this stream
                pos = start + D + np.arange(K)
                live = k[l, bt[pos // 16], g, pos % 16]
                kept_rows = k0[l, bt[(start + np.nonzero(keep)[0]) // 16], g,
                               (start + np.nonzero(keep)[0]) % 16]
                assert sorted(map(bytes, live)) == sorted(map(bytes, kept_rows))


def test_round_end_to_end_tiny_shape():
    """A whole round on a small two-sequence batch: counts, CRF placement, layout."""
    L, Hkv, Hq, P = 1, 2, 4, 20
    r = np.random.default_rng(11)
    k, v, crf = make_pool(L, P, Hkv, seed=11)
    lengths = np.array([70, 33]); starts = np.array([3, 0])
    bt = np.full((2, 6), -1, np.int32)
    perm = r.permutation(P)
    bt[0, :5] = perm[:5]; bt[1, :3] = perm[5:8]
    obs_off = np.array([0, 5, 9])
    q = bf16(r.standard_normal((L, Hq, 9, 128)).astype(np.float32))
    lse = np.zeros((L, Hq, 9), np.float32)
    for i in range(2):
        for h in range(Hq):
            pos = starts[i] + np.arange(lengths[i])
            keys = O.bf16_bits_to_f64(k[0, bt[i][pos // 16], h // 2, pos % 16])
            qq = O.bf16_bits_to_f64(q[0, h, obs_off[i]:obs_off[i + 1]])
            lse[0, h, obs_off[i]:obs_off[i + 1]] = _exact_lse(qq, keys, 1 / np.sqrt(128))
    k0 = k.copy()
    res = O.eviction_round(k, v, crf, q, lse, obs_off, bt, starts, lengths, Hq, 1 / np.sqrt(128),
                           0.5, np.array([8, 64]), np.array([70, 0]), np.array([16, 40]))
    for (i, l, g), keep in res["keep"].items():
        assert keep.sum() == min([16, 40][i], lengths[i])
        R = (obs_off[i + 1] - obs_off[i]) * 2
        assert abs(res["s"][(i, l, g)].astype(np.float64).sum() - R) < 1e-4
    shift, ns, nl, freed = res["seq"][0]
    assert (shift, ns, nl) == ((3 + 54) // 16, (3 + 54) % 16, 16)
    assert res["seq"][1] == (0, 0, 33, res["seq"][1][3]) and len(res["seq"][1][3]) == 0
    # kept keys now fill the tail, and the moved CRF sits with them
    keep = res["keep"][(0, 0, 1)]
    pos = 3 + 54 + np.arange(16)
    live = k[0, bt[0][pos // 16], 1, pos % 16]
    kept = k0[0, bt[0][(3 + np.nonzero(keep)[0]) // 16], 1, (3 + np.nonzero(keep)[0]) % 16]
    assert sorted(map(bytes, live)) == sorted(map(bytes, kept))
    crf_live = crf[0, bt[0][pos // 16], 1, pos % 16]
    crf_kept = res["crf"][(0, 0, 1)][np.nonzero(keep)[0]]
    assert sorted(crf_live.tolist()) == sorted(crf_kept.tolist())
