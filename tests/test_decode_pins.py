"""Pins of the decode-attention oracle (oracle/decode_oracle.py): closed forms, a
library softmax and log-sum-exp on small inputs, invariants, and agreement of its
tally with the observer scorer's definition given the emitted LSE."""
import math

import numpy as np
import pytest
import scipy.special

import oracle as O
from oracle import decode_oracle as DO

rng = np.random.default_rng(99)


def test_two_keys_closed_form():
    q = np.array([[1.0, 0.0]])
    k = np.array([[2.0, 5.0], [-1.0, 3.0]])      # logits (scale 1): 2 and -1
    v = np.array([[1.0, 2.0], [3.0, -4.0]])
    out, lse, p = DO.attend_stream(q, k, v, 1.0)
    p0 = 1.0 / (1.0 + math.exp(-3.0))
    assert p[0, 0] == pytest.approx(p0, rel=1e-14) and p[0, 1] == pytest.approx(1 - p0, rel=1e-13)
    assert lse[0] == pytest.approx(math.log(math.exp(2.0) + math.exp(-1.0)), rel=1e-14)
    np.testing.assert_allclose(out[0], p0 * v[0] + (1 - p0) * v[1], rtol=1e-13)


def test_equal_keys_and_single_key():
    q = rng.standard_normal((3, 8))
    kk = rng.standard_normal(8)
    keys = np.tile(kk, (5, 1))
    vals = rng.standard_normal((5, 8))
    out, lse, p = DO.attend_stream(q, keys, vals, 0.3)
    np.testing.assert_allclose(p, 0.2, rtol=1e-14)
    np.testing.assert_allclose(out, np.tile(vals.mean(0), (3, 1)), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, 0.3 * (q @ kk) + math.log(5), rtol=1e-13)
    out1, lse1, p1 = DO.attend_stream(q, keys[:1], vals[:1], 0.3)
    np.testing.assert_allclose(out1, np.tile(vals[0], (3, 1)), rtol=1e-14)
    np.testing.assert_allclose(lse1, 0.3 * (q @ kk), rtol=1e-14)
    np.testing.assert_allclose(p1, 1.0)


@pytest.mark.parametrize("n", [1, 7, 100])
def test_library_softmax_and_lse(n):
    q = rng.standard_normal((4, 16))
    k = rng.standard_normal((n, 16)) * 2
    v = rng.standard_normal((n, 16))
    out, lse, p = DO.attend_stream(q, k, v, 1 / 4)
    logits = (q @ k.T) / 4
    np.testing.assert_allclose(lse, scipy.special.logsumexp(logits, axis=1), rtol=1e-13)
    ps = scipy.special.softmax(logits, axis=1)
    np.testing.assert_allclose(p, ps, rtol=1e-12)
    np.testing.assert_allclose(out, ps @ v, rtol=1e-11, atol=1e-14)


def test_invariants():
    q = rng.standard_normal((4, 32))
    k = rng.standard_normal((200, 32))
    v = rng.standard_normal((200, 32))
    out, lse, p = DO.attend_stream(q, k, v, 0.2)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-13)
    assert np.all(p >= 0)
    assert np.all(out <= v.max(0) + 1e-12) and np.all(out >= v.min(0) - 1e-12)
    perm = rng.permutation(200)
    out2, lse2, p2 = DO.attend_stream(q, k[perm], v[perm], 0.2)
    np.testing.assert_allclose(out2, out, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)
    np.testing.assert_allclose(p2, p[:, perm], rtol=1e-12)


def test_tally_matches_scorer_given_emitted_lse():
    # Component 3: the scorer recovers p from the LSE that attention emits; the two
    # oracle functions must agree on the per-entry sums
    q = rng.standard_normal((8, 128))
    k = rng.standard_normal((300, 128))
    v = rng.standard_normal((300, 128))
    _, lse, p = DO.attend_stream(q, k, v, 1 / math.sqrt(128))
    s = O.score_stream(q, lse, k, 1 / math.sqrt(128))
    np.testing.assert_allclose(s, p.sum(0).astype(np.float32), rtol=2e-7)


def test_paged_gqa_mapping():
    # heads 0, 1 read KV head 0 and heads 2, 3 read KV head 1; a KV head whose keys and
    # values are constant gives every row that reads it that constant value
    from tests.test_oracle_pins import bf16
    L, P, Hkv, D = 1, 4, 2, 128
    kp = bf16(rng.standard_normal((L, P, Hkv, 16, D)).astype(np.float32))
    vp = bf16(rng.standard_normal((L, P, Hkv, 16, D)).astype(np.float32))
    vp[:, :, 1] = bf16(np.full((16, D), 0.5, np.float32))
    q = bf16(rng.standard_normal((L, 4, 3, D)).astype(np.float32))
    bt = np.array([[2, 0, 3, 1]], np.int32)
    res = DO.decode_attention(kp, vp, q, np.array([0, 3]), bt, np.array([5]), np.array([50]), 4, 0.1)
    np.testing.assert_allclose(res[(0, 0, 1)][0], 0.5, rtol=1e-13)
    assert not np.allclose(res[(0, 0, 0)][0], 0.5)
    for key in res:
        np.testing.assert_allclose(res[key][2].sum(), res[key][0].shape[0], rtol=1e-12)   # 6 rows
