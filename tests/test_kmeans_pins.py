"""Pins of the beacon k-means oracle (oracle/kmeans_oracle.py): hand-worked examples
(including rounding and ties of the member mean), scikit-learn's Lloyd k-means on
separated groups at fp32 rounding, the one-group mean, tie and empty-group rules,
exact invariances, the non-increasing objective, the exact rational rounding against
numpy and against brute force over fp32 neighbours, and the bf16 rounding against
torch."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import kmeans_oracle as KO

rng = np.random.default_rng(77)
D = 128


def line_points(vals):
    x = np.zeros((len(vals), D))
    x[:, 0] = vals
    return x


def test_hand_worked_example():
    # points 0, 1, 10, 11 on the first axis; centroids 0 and 10: one iteration assigns
    # {0, 1} and {10, 11} and moves the centroids to 0.5 and 10.5; a second changes nothing
    x = line_points([0.0, 1.0, 10.0, 11.0])
    c0 = np.zeros((2, D), np.float32)
    c0[1, 0] = 10.0
    c, a = KO.lloyd(x, c0, 1)
    np.testing.assert_array_equal(a, [0, 0, 1, 1])
    assert c[0, 0] == 0.5 and c[1, 0] == 10.5 and np.all(c[:, 1:] == 0)
    c2, a2 = KO.lloyd(x, c0, 2)
    np.testing.assert_array_equal(c2, c)
    np.testing.assert_array_equal(a2, a)


def test_member_mean_rounds_once():
    # {1, 1 + 2^-7, 1 + 2^-7}: mean 1 + 2^-6/3; in steps of 2^-23 above 1 that is
    # 2^17/3 = 43690.67, so the fp32 mean is 1 + 43691 2^-23 (a second rounding through
    # a coarser grid would lose it)
    c = KO.member_mean(line_points([1.0, 1.0 + 2.0 ** -7, 1.0 + 2.0 ** -7]))
    assert c[0] == np.float32(1.0 + 43691 * 2.0 ** -23) and np.all(c[1:] == 0)
    # {2, 2^-23}: mean 1 + 2^-24, halfway between 1 and 1 + 2^-23 -> the even one, 1
    assert KO.member_mean(line_points([2.0, 2.0 ** -23]))[0] == np.float32(1.0)
    # {2 + 2^-6, 3 2^-23}: mean 1 + 2^-7 + 1.5 2^-23, halfway between 1 + 2^-7 + 2^-23
    # (odd) and 1 + 2^-7 + 2 2^-23 (even) -> the latter
    got = KO.member_mean(line_points([2.0 + 2.0 ** -6, 3 * 2.0 ** -23]))[0]
    assert got == np.float32(1.0 + 2.0 ** -7 + 2 * 2.0 ** -23)
    # a tiny coordinate counts in full: {2^-30, 0} has mean 2^-31
    assert KO.member_mean(line_points([2.0 ** -30, 0.0]))[0] == np.float32(2.0 ** -31)


def _f32_neighbours(v: np.float32):
    return [np.nextafter(v, np.float32(-np.inf)), v, np.nextafter(v, np.float32(np.inf))]


def test_round_to_f32_is_nearest_even():
    # rationals exact in fp64 (power-of-two denominators): numpy's single rounding
    # fp64 -> fp32 is the reference
    for _ in range(3000):
        num = int(rng.integers(-(2 ** 52), 2 ** 52)) or 1
        den = 1 << int(rng.integers(0, 170))
        want = np.float32(num / den) if abs(num / den) >= 2.0 ** -149 or num / den == 0 else None
        if want is not None:
            assert KO.round_to_f32(num, den) == want, (num, den)
    # general rationals: the result is the nearest fp32 value, checked by brute force
    # over its neighbours with exact fractions
    for _ in range(1500):
        num = int(rng.integers(1, 2 ** 62)) * int(rng.choice([-1, 1]))
        den = int(rng.integers(1, 2 ** 40)) << int(rng.integers(0, 60))
        got = KO.round_to_f32(num, den)
        exact = Fraction(num, den)
        err = abs(Fraction(float(got)) - exact)
        for nb in _f32_neighbours(got):
            if np.isfinite(nb):
                assert err <= abs(Fraction(float(nb)) - exact), (num, den)
    # ties go to the even neighbour, also in the subnormal range
    assert KO.round_to_f32(1, 1 << 150) == 0.0                        # 2^-150: halfway 0 / 2^-149
    assert KO.round_to_f32(3, 1 << 150) == np.float32(2.0 ** -148)    # 1.5 2^-149 -> 2 2^-149
    assert KO.round_to_f32((1 << 24) + 1, 1 << 24) == 1.0             # 1 + 2^-24 -> 1
    assert KO.round_to_f32((1 << 24) + 3, 1 << 24) == np.float32(1.0 + 2.0 ** -22)
    assert np.isinf(KO.round_to_f32(1 << 200, 1))


def test_exact_column_sums_against_fractions():
    # mixed magnitudes, signs and subnormal bf16-like values: the integer sums equal
    # the exact rational sums
    vals = np.concatenate([rng.normal(size=300) * 2.0 ** rng.integers(-140, 14, 300),
                           [2.0 ** -133, -(2.0 ** -133), 0.0, 2.0 ** 14]])
    x = vals.reshape(-1, 2)
    sums, b = KO.exact_column_sums(x)
    for d in range(2):
        assert Fraction(sums[d]) * Fraction(2) ** b == sum(Fraction(float(v)) for v in x[:, d])


def test_matches_scikit_learn_on_separated_groups():
    # 8 well separated groups: labels match scikit-learn's Lloyd k-means exactly, and the
    # centroids are its fp64 means rounded to fp32 (the exact mean rounded once; an fp64
    # mean could differ only within 2^-52 of an fp32 rounding midpoint)
    from sklearn.cluster import KMeans
    K, n = 8, 600
    centers = rng.normal(0.0, 4.0, (K, D))
    lab = rng.integers(0, K, n)
    x = centers[lab] + rng.normal(0.0, 0.3, (n, D))
    x = x.astype(np.float32).astype(np.float64)
    c0 = x[[int(np.nonzero(lab == k)[0][0]) for k in range(K)]].astype(np.float32)
    c, a = KO.lloyd(x, c0, 10)
    km = KMeans(n_clusters=K, init=c0.astype(np.float64), n_init=1, max_iter=10, algorithm="lloyd", tol=0.0)
    km.fit(x)
    np.testing.assert_array_equal(a, km.labels_)
    sk = km.cluster_centers_.astype(np.float32)
    np.testing.assert_array_max_ulp(c, sk, maxulp=1)
    # where they differ, scikit-learn's fp64 mean sat within fp64 rounding of an fp32
    # rounding midpoint, and the oracle's value is the even one of the two
    for k, d in np.argwhere(c != sk):
        mid = (Fraction(float(c[k, d])) + Fraction(float(sk[k, d]))) / 2
        assert abs(Fraction(float(km.cluster_centers_[k, d])) - mid) <= abs(mid) * Fraction(1, 2 ** 48)
        assert int(c[k:k + 1, d].view(np.uint32)[0]) % 2 == 0
    assert np.mean(c == sk) > 0.99
    # initial centroid k is a member of planted group k, and the groups are far apart
    np.testing.assert_array_equal(a, lab)


def test_one_group_is_the_mean():
    # K = 1: the centroid is the mean of all points; small integers with a power-of-two
    # count give an exact mean
    x = rng.integers(-50, 50, (64, D)).astype(np.float64)
    c, a = KO.lloyd(x, np.zeros((1, D), np.float32), 1)
    np.testing.assert_array_equal(c[0], x.mean(axis=0).astype(np.float32))
    assert np.all(a == 0)


def test_ties_and_empty_groups():
    x = rng.normal(size=(50, D))
    c0 = np.zeros((3, D), np.float32)
    c0[0] = c0[1] = x[0].astype(np.float32)          # two equal centroids: the lower one wins
    c0[2] = 1000.0                                   # far away: stays empty, keeps its centroid
    c, a = KO.lloyd(x, c0, 1)
    assert np.all(a == 0)
    np.testing.assert_array_equal(c[1], c0[1])
    np.testing.assert_array_equal(c[2], c0[2])


def test_invariances():
    x = rng.normal(size=(300, D)).astype(np.float32).astype(np.float64)
    c0 = x[:6].astype(np.float32)
    c, a = KO.lloyd(x, c0, 4)
    # the order of the points changes nothing (exact sums)
    perm = rng.permutation(300)
    cp, ap = KO.lloyd(x[perm], c0, 4)
    np.testing.assert_array_equal(cp, c)
    np.testing.assert_array_equal(ap, a[perm])
    # scaling by 2 scales scores by 4 and means by 2, exactly
    c2, a2 = KO.lloyd(2.0 * x, 2.0 * c0, 4)
    np.testing.assert_array_equal(a2, a)
    np.testing.assert_array_equal(c2, 2.0 * c)
    # a translation by an integer vector translates the centroids (to fp32 rounding)
    shift = rng.integers(-3, 4, D).astype(np.float64)
    ct, at = KO.lloyd(x + shift, (c0 + shift).astype(np.float32), 4)
    np.testing.assert_array_equal(at, a)
    np.testing.assert_allclose(ct, c + shift, atol=2.0 ** -20)


def test_objective_does_not_increase():
    x = rng.normal(size=(800, D))
    c = x[:16].astype(np.float32)
    prev = np.inf
    for _ in range(8):
        a, sc = KO.assign(x, c)
        obj = float(np.sum(sc[np.arange(len(a)), a]) + np.sum(x * x))
        assert obj <= prev * (1 + 1e-9) + 1e-6
        prev = obj
        c = KO.update(x, a, c)


def test_bf16_rounding_matches_torch():
    import torch
    v = np.concatenate([rng.normal(size=1000) * 10.0 ** rng.integers(-5, 5, 1000),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)]]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(KO.to_bf16_bits(v), want)


def test_bad_points():
    with pytest.raises(ValueError):
        KO.lloyd(line_points([2.0 ** 15]), np.zeros((1, D), np.float32), 1)


def test_kmeanspp_hand_worked():
    # rows 0, 1, 10 on the first axis; u_0 = 0 picks row 0, so D2 = [0, 1, 100] and
    # the cumulative sums are [0, 1, 101]: u = 0.5 (target 50.5) draws row 2, u = 0.005
    # (target 0.505) draws row 1
    x = line_points([0.0, 1.0, 10.0])
    c, rows = KO.kmeanspp(x, np.array([0.0, 0.5], np.float32))
    np.testing.assert_array_equal(rows, [0, 2])
    np.testing.assert_array_equal(c[:, 0], [0.0, 10.0])
    _, rows = KO.kmeanspp(x, np.array([0.0, 0.005], np.float32))
    np.testing.assert_array_equal(rows, [0, 1])
    # u_0 = 0.7 of 3 rows -> row 2
    assert KO.kmeanspp(x, np.array([0.7], np.float32))[1][0] == 2


def test_kmeanspp_draws_in_proportion_to_d2():
    # from row 0, rows 1..4 sit at squared distances 1, 2, 3, 4: over many uniforms the
    # second draw lands on row i with frequency D2_i / 10
    x = np.zeros((5, D))
    x[1:, 0] = np.sqrt([1.0, 2.0, 3.0, 4.0])
    u = (np.arange(20000) + 0.5) / 20000
    counts = np.zeros(5)
    for ui in u[::7]:
        counts[KO.kmeanspp(x, np.array([0.0, ui], np.float32))[1][1]] += 1
    freq = counts / counts.sum()
    np.testing.assert_allclose(freq, [0.0, 0.1, 0.2, 0.3, 0.4], atol=2e-3)


def test_kmeanspp_degenerate_and_consistency():
    # all rows equal: D2 is 0, so each draw is floor(u n)
    x = np.ones((10, D))
    _, rows = KO.kmeanspp(x, np.array([0.05, 0.55, 0.95], np.float32))
    np.testing.assert_array_equal(rows, [0, 5, 9])
    # random rows: chosen rows are distinct, and every draw is a valid step
    y = rng.normal(size=(300, D)).astype(np.float32).astype(np.float64)
    uu = rng.random(16).astype(np.float32)
    _, rows = KO.kmeanspp(y, uu)
    assert len(set(rows.tolist())) == 16
    for c in range(1, 16):
        assert KO.seed_step_valid(y, rows[:c], uu[c], int(rows[c]), 0.0)
        assert not KO.seed_step_valid(y, rows[:c], uu[c], int(rows[c - 1]), 0.0)
