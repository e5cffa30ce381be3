"""Pins of the StepKV oracle (oracle/stepkv_oracle.py): a hand-worked example, the
two end points of the weight (token-only and step-only ranking), exact rational
recomputation of every key on small inputs, round-half-even of the step mean, and
invariances."""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from oracle import stepkv_oracle as SO

rng = np.random.default_rng(2024)


def test_hand_worked_example():
    # steps [0.5, 0.25 | 0.125, 1.0, 0.0]; both steps have mean 0.375.  beta = 1/2:
    # c = 0.1875 + s / 2 = [0.4375, 0.3125, 0.25, 0.6875, 0.1875]; budget 2 keeps
    # slots 3 and 0
    s = np.array([0.5, 0.25, 0.125, 1.0, 0.0], np.float32)
    keep, c, u = SO.step_select(s, [0, 2, 5], 0.5, 2)
    np.testing.assert_array_equal(u, [0.375, 0.375])
    np.testing.assert_array_equal(c, [0.4375, 0.3125, 0.25, 0.6875, 0.1875])
    np.testing.assert_array_equal(keep, [True, False, False, True, False])
    # beta = 3/4 with steps [1.0 | 0.25, 0.25, 0.0 | 0.5]: U = [1, 1/6, 0.5];
    # c = 0.75 U + 0.25 s = [1.0, 0.1875, 0.1875, 0.125, 0.5]; budget 3 keeps slots
    # 0, 4 and (tie between 1 and 2 on c and s) the lower slot 1
    s = np.array([1.0, 0.25, 0.25, 0.0, 0.5], np.float32)
    keep, c, u = SO.step_select(s, [0, 1, 4, 5], 0.75, 3)
    assert u[0] == 1.0 and u[2] == 0.5
    # 1/6 on the 2^-32 grid: floor(2^31 / 3) 2^-32, rounded to fp32
    assert u[1] == np.float32(Fraction(2 ** 31 // 3, 2 ** 32))
    np.testing.assert_array_equal(keep, [True, True, False, False, True])


def test_beta_zero_is_token_ranking():
    # beta = 0: c = s exactly, so the keep set is the plain top-B by saliency
    for n in (1, 7, 100):
        s = rng.exponential(1.0, n).astype(np.float32)
        s[rng.random(n) < 0.2] = 0.0
        b = np.sort(np.concatenate([[0, n], rng.integers(0, n + 1, 3)]))
        for B in (0, 1, n // 2, n, n + 5):
            keep, c, _ = SO.step_select(s, b, 0.0, B)
            np.testing.assert_array_equal(c, s)
            np.testing.assert_array_equal(keep, O.select_top_b(np.zeros(n, np.float32), s, B))


def test_beta_one_is_step_ranking():
    # beta = 1: c = U of the entry's step; a kept entry's step utility is never below
    # an evicted entry's, and the entries of a step are kept in (s desc, slot asc) order
    n = 300
    s = rng.exponential(1.0, n).astype(np.float32)
    b = np.array([0, 20, 21, 90, 90, 150, 260, 300])
    keep, c, u = SO.step_select(s, b, 1.0, 133)
    step_of = np.repeat(np.arange(len(b) - 1), np.diff(b))
    np.testing.assert_array_equal(c, u[step_of])
    assert keep.sum() == 133
    assert u[step_of][keep].min() >= u[step_of][~keep].max()
    for k in range(len(b) - 1):
        idx = np.arange(b[k], b[k + 1])
        kk = keep[idx]
        if kk.any() and not kk.all():
            assert s[idx][kk].min() >= s[idx][~kk].max()


def test_keys_against_exact_rationals():
    # every key recomputed with exact rationals: w = RN(1 - beta), t = RN(w s),
    # U = RN(floor(sum floor(s 2^32) / len) 2^-32), c = RN(beta U + t)
    def rn(x):
        return O.round_fraction_to_f32(Fraction(x))

    for trial in range(30):
        n = int(rng.integers(1, 40))
        s = (rng.exponential(1.0, n) * 10.0 ** rng.integers(-6, 2, n)).astype(np.float32)
        cuts = np.sort(rng.integers(0, n + 1, int(rng.integers(0, 5))))
        b = np.concatenate([[0], cuts, [n]])
        beta = np.float32(rng.choice([0.0, 1.0, rng.random()]))
        c, u = SO.step_keys(s, b, float(beta))
        w = rn(Fraction(1) - Fraction(float(beta)))
        for k in range(len(b) - 1):
            lo, hi = int(b[k]), int(b[k + 1])
            if hi == lo:
                assert u[k] == 0.0
                continue
            tot = sum(int(Fraction(float(x)) * 2 ** 32) for x in s[lo:hi])
            assert u[k] == rn(Fraction(tot // (hi - lo), 2 ** 32))
            for j in range(lo, hi):
                t = rn(Fraction(float(w)) * Fraction(float(s[j])))
                want = rn(Fraction(float(beta)) * Fraction(float(u[k])) + Fraction(float(t)))
                assert c[j] == want, (trial, j)


@pytest.mark.parametrize("a2,expect", [(4, 2 ** 25), (5, 2 ** 25), (12, 2 ** 25 + 8), (8, 2 ** 25 + 4)])
def test_step_mean_rounding(a2, expect):
    # two entries with fixed-point masses 2^26 and a2: U_int = floor((2^26 + a2) / 2);
    # 2^25 + 2 and 2^25 + 6 are halfway between fp32 neighbours (spacing 4) and go to
    # the even one; the odd sum 2^26 + 5 is floored first
    s = np.array([2.0 ** -6, a2 * 2.0 ** -32], np.float32)
    u = SO.step_utility(s, [0, 2])
    assert u[0] == np.float32(expect * 2.0 ** -32)


def test_invariances():
    n = 64
    s = rng.exponential(1.0, n).astype(np.float32)
    b = np.array([0, 10, 30, 64])
    keep, c, u = SO.step_select(s, b, 0.4, 20)
    # permuting entries inside a step changes neither the utility nor which values are kept
    perm = np.arange(n)
    perm[10:30] = 10 + rng.permutation(20)
    keep2, c2, u2 = SO.step_select(s[perm], b, 0.4, 20)
    np.testing.assert_array_equal(u2, u)
    np.testing.assert_array_equal(keep2, keep[perm])
    # a step of constant saliency s0 (on the 2^-32 grid) has utility s0
    s3 = s.copy()
    s3[30:64] = np.float32(0.375)
    assert SO.step_utility(s3, b)[2] == np.float32(0.375)
    # scaling every score by 2 scales every key by 2 (exact in fp32 and on the grid)
    c4, u4 = SO.step_keys(s * np.float32(2), b, 0.4)
    np.testing.assert_array_equal(c4, c * np.float32(2))


def test_bad_inputs():
    s = np.ones(5, np.float32)
    for b in ([0, 4], [1, 5], [0, 3, 2, 5], [0]):
        with pytest.raises(ValueError):
            SO.step_utility(s, b)
    with pytest.raises(ValueError):
        SO.step_keys(s, [0, 5], 1.5)
    with pytest.raises(ValueError):
        SO.step_keys(-s, [0, 5], 0.5)


def test_grid_mean_against_the_plain_mean():
    # reading S3 takes the step mean on the mass cut's 2^-32 grid; against the exact mean
    # of the fp32 scores rounded once it differs by at most 2^-31 plus one fp32 spacing,
    # and the keys by beta times that plus one spacing of the key: so a keep decision
    # can differ only for entries whose plain-mean key lies within that of the K-th key
    from workloads import steps as WS
    r2 = np.random.default_rng(5)
    n_keep_checked = 0
    for trial in range(6):
        n = int(r2.integers(200, 3000))
        _, _, bounds = WS.batch_steps(r2, np.array([n]))
        s = WS.step_scores(r2, bounds[0])
        if trial % 2:
            s = (s * np.float32(1e-3)).astype(np.float32)      # many values below the grid's reach
        u_grid = SO.step_utility(s, bounds[0])
        u_mean = SO.step_utility_mean(s, bounds[0])
        bound = 2.0 ** -31 + np.spacing(np.abs(u_mean)).astype(np.float64)
        assert np.all(np.abs(u_grid.astype(np.float64) - u_mean) <= bound)
        beta, B = 0.5, n // 5
        keep, c, _ = SO.step_select(s, bounds[0], beta, B)
        step_of = np.repeat(np.arange(len(bounds[0]) - 1), np.diff(bounds[0]))
        w = np.float32(np.float32(1.0) - np.float32(beta))
        c_mean = O.fma_f32(np.full(n, np.float32(beta)), u_mean[step_of], (w * s).astype(np.float32))
        keep_mean = O.select_top_b(c_mean, s, B)
        kth = np.sort(c_mean.astype(np.float64))[::-1][B - 1]
        margin = beta * (2.0 ** -31 + float(np.spacing(np.float32(abs(kth))))) + float(np.spacing(np.float32(kth)))
        far = np.abs(c_mean.astype(np.float64) - kth) > 2 * margin
        np.testing.assert_array_equal(keep[far], keep_mean[far])
        n_keep_checked += int(far.sum())
    assert n_keep_checked > 1000
