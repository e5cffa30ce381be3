"""Pins of the confidence-monitor oracle (oracle/confidence_oracle.py) to things
other than itself: closed forms, a route through explicit probabilities on tiny
vocabularies, invariants, a library least-squares fit, and hand-worked series.

A slip in the oracle (a log base, a sign, a mean over the wrong tokens, a window
off by one, a slope normalised wrongly) fails at least one test here.
"""
import math

import numpy as np
import pytest

from oracle import confidence as C
from oracle import ratchet, RATCHET_INITIAL

rng = np.random.default_rng(77)


# ---------------------------------------------------------------------------
# token confidence


@pytest.mark.parametrize("V,k", [(5, 1), (5, 5), (1000, 20), (128256, 20), (4096, 64)])
def test_uniform_logits_give_ln_vocab(V, k):
    # every token has p = 1/V, so every top-k token has -ln p = ln V
    for a in (0.0, -3.25, 17.5):
        assert C.token_confidence(np.full(V, a), k) == pytest.approx(math.log(V), rel=1e-13)


def test_hand_worked_four_tokens():
    # e^z = 1, 2, 3, 4 -> p = 0.1, 0.2, 0.3, 0.4; the two most probable: 0.4 and 0.3
    z = np.log([1.0, 2.0, 3.0, 4.0])
    expect = -(math.log(0.4) + math.log(0.3)) / 2
    assert C.token_confidence(z, 2) == pytest.approx(expect, rel=1e-14)
    # k = 4: all tokens
    expect4 = -(math.log(0.1) + math.log(0.2) + math.log(0.3) + math.log(0.4)) / 4
    assert C.token_confidence(z, 4) == pytest.approx(expect4, rel=1e-14)


@pytest.mark.parametrize("a,V,k", [(8.0, 1000, 20), (0.5, 50, 3), (30.0, 128256, 20)])
def test_one_peak_closed_form(a, V, k):
    # one token at a, V-1 tokens at 0: LSE = ln(e^a + V - 1); the top k are the peak
    # and k-1 zeros, mean logit a/k
    z = np.zeros(V)
    z[rng.integers(V)] = a
    expect = math.log(math.exp(a) + V - 1) - a / k
    assert C.token_confidence(z, k) == pytest.approx(expect, rel=1e-13)


@pytest.mark.parametrize("V", [7, 30, 200])
def test_brute_force_through_probabilities(V):
    # the definition taken literally: probabilities, the k largest of them, mean -ln p
    for _ in range(5):
        z = rng.standard_normal(V) * 3
        p = np.exp(z) / np.sum(np.exp(z))
        for k in (1, 3, min(V, 20)):
            top = sorted(p, reverse=True)[:k]
            expect = sum(-math.log(x) for x in top) / k
            assert C.token_confidence(z, k) == pytest.approx(expect, rel=1e-12)


def test_invariants():
    z = rng.standard_normal(5000) * 2
    c = C.token_confidence(z, 20)
    # a common shift of the logits does not change the distribution
    assert C.token_confidence(z + 11.0, 20) == pytest.approx(c, rel=1e-12)
    # nor does the order of the vocabulary
    assert C.token_confidence(rng.permutation(z), 20) == pytest.approx(c, rel=1e-14)
    # adding less probable tokens to the mean can only raise it
    cs = [C.token_confidence(z, k) for k in range(1, 65)]
    assert all(b >= a - 1e-12 for a, b in zip(cs, cs[1:]))
    # a sharper distribution (logits scaled up) is more confident
    assert C.token_confidence(z * 3, 20) > c
    # and every -ln p is at least -ln p_max >= 0
    assert c >= C.token_confidence(z, 1) >= 0.0


def test_ties_and_masked_tokens():
    # ties across the k-th place: any k-subset gives the same mean
    z = np.array([5.0, 5.0, 5.0, 1.0, 1.0])
    lse = math.log(3 * math.exp(5.0) + 2 * math.exp(1.0))
    assert C.token_confidence(z, 2) == pytest.approx(lse - 5.0, rel=1e-14)
    assert C.token_confidence(z, 4) == pytest.approx(lse - (15.0 + 1.0) / 4, rel=1e-14)
    # -inf logits are tokens of probability 0: they leave the rest unchanged
    zm = np.concatenate([z, [-np.inf, -np.inf]])
    assert C.token_confidence(zm, 4) == pytest.approx(C.token_confidence(z, 4), rel=1e-14)
    with pytest.raises(ValueError):
        C.token_confidence(z, 6)


# ---------------------------------------------------------------------------
# min-pooling, slope, flag


def test_min_pool_hand_worked():
    c = [5, 3, 4, 1, 2, 6, 7, 0]
    # windows of 3 every 2: [5,3,4] [4,1,2] [2,6,7]; [7,0] is not a full window
    np.testing.assert_array_equal(C.min_pool(c, 3, 2), [3, 1, 2])
    np.testing.assert_array_equal(C.min_pool(c, 8, 8), [0])
    assert C.min_pool(c, 9, 1).size == 0


def test_min_pool_pages_parameters_on_ramps():
    T = 64 + 8 * 10
    up = np.arange(T, dtype=np.float64)
    # window starting at 8k: minimum is its first element
    np.testing.assert_array_equal(C.min_pool(up), 8.0 * np.arange(11))
    # descending: minimum is the last element of the window
    np.testing.assert_array_equal(C.min_pool(-up), -(8.0 * np.arange(11) + 63))
    assert C.min_pool(np.ones(63)).size == 0
    assert C.min_pool(np.ones(64)).size == 1
    assert C.min_pool(np.ones(71)).size == 1
    assert C.min_pool(np.ones(72)).size == 2


def test_slope_closed_forms_and_library_fit():
    x = np.arange(12, dtype=np.float64)
    assert C.lsq_slope(3.0 - 0.5 * x) == pytest.approx(-0.5, abs=1e-14)
    assert C.lsq_slope(np.full(9, 2.5)) == pytest.approx(0.0, abs=1e-15)
    assert C.lsq_slope([1.0, 3.0, 2.0]) == pytest.approx(0.5, abs=1e-15)
    assert C.lsq_slope([4.0, 1.0]) == pytest.approx(-3.0, abs=1e-15)
    assert C.lsq_slope([4.0]) is None and C.lsq_slope([]) is None
    for _ in range(5):
        y = rng.standard_normal(int(rng.integers(2, 400)))
        assert C.lsq_slope(y) == pytest.approx(np.polyfit(np.arange(y.size), y, 1)[0], rel=1e-9, abs=1e-12)


def test_flag_follows_the_trend():
    T = 64 + 8 * 20
    t = np.arange(T, dtype=np.float64)
    assert C.trend_flag(10 + 0.01 * t) == (pytest.approx(0.08), 21, False)
    s, n, f = C.trend_flag(10 - 0.01 * t)
    assert f and n == 21 and s == pytest.approx(-0.08)
    # too short for two pooled values: no slope, no flag
    assert C.trend_flag(np.ones(70)) == (None, 1, False)
    assert C.trend_flag(np.ones(10)) == (None, 0, False)
    # a late collapse: the whole-trajectory fit sees it, and so does a fit of the last 4
    c = np.full(T, 12.0)
    c[-20:] = 3.0
    assert C.trend_flag(c)[2]
    s4, _, f4 = C.trend_flag(c, fit_last=4)
    assert f4 and s4 < 0
    # a recovery after a dip: the last pooled values rise, so a short fit does not flag
    c2 = np.full(T, 12.0)
    c2[40:120] = 3.0
    assert not C.trend_flag(c2, fit_last=6)[2]


def test_flags_drive_the_ratchet():
    # Component 2: each flagged round multiplies the budget by 1.75 (integer 7/4), capped
    b = RATCHET_INITIAL
    T = 64 + 8 * 10
    down = 10 - 0.01 * np.arange(T)
    up = 10 + 0.01 * np.arange(T)
    seq = []
    for conf in (up, down, down, up, down):
        b = ratchet(b, C.trend_flag(conf)[2])
        seq.append(b)
    assert seq == [512, 896, 1568, 1568, 2744]
