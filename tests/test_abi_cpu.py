"""CPU-only checks of the C ABI: the library loads without a GPU, exports every
function include/kvs.h declares, and its host-side validation rejects bad
arguments before any HIP call.  Host-only entry points (decay, ratchet, pair
capacity, plan host outputs) are checked against the oracle here too."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
from kv_cache_eviction_lse_amd import _lib as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000   # a non-NULL pointer value that no test dereferences


def header_functions():
    txt = open(os.path.join(ROOT, "include", "kvs.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(kvs_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    L = K.lib()
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(K.EXPORTS) <= set(names)


def test_status_strings():
    L = K.lib()
    for code, name in K.STATUS.items():
        assert L.kvs_status_string(code).decode() == name


def _cache(L=1, Hkv=1, P=8, head_dim=128, page=16, k=FAKE, v=FAKE, crf=FAKE):
    return K.Cache(k, v, crf, L, Hkv, head_dim, page, P)


class HostSeqs:
    def __init__(self, bt, start, length, max_pages=None):
        self.bt = np.ascontiguousarray(bt, np.int32)
        self.start = np.ascontiguousarray(start, np.int32)
        self.len = np.ascontiguousarray(length, np.int32)
        self.off = np.zeros(len(self.len) + 1, np.int64)
        self.off[1:] = np.cumsum(self.len)
        mp = self.bt.shape[1] if max_pages is None else max_pages
        self.s = K.Seqs(len(self.len), mp, FAKE, self.bt.ctypes.data, FAKE, self.start.ctypes.data,
                        FAKE, self.len.ctypes.data, FAKE, self.off.ctypes.data)


def _obs(S, Hq=4, O_=4):
    off = np.arange(S + 1, dtype=np.int64) * O_
    o = K.Observers(FAKE, FAKE, FAKE, off.ctypes.data, Hq, int(off[-1]))
    return o, off


def status(code):
    return K.STATUS[code]


def test_score_validation():
    """Every call here is invalid, so none reaches a launch (the pointers are fake)."""
    L = K.lib()
    seqs = HostSeqs([[0, 1, 2]], [0], [40])
    obs, off = _obs(1)
    c = _cache()
    ws = FAKE

    def call(cache=c, s=seqs.s, o=obs, scale=0.1, scores=FAKE, wsb=1 << 20):
        return status(L.kvs_score(C.byref(cache), C.byref(s), C.byref(o), C.c_float(scale),
                                  scores, ws, wsb, None))

    assert call(cache=_cache(head_dim=64)) == "KVS_ERR_UNSUPPORTED"
    assert call(cache=_cache(page=32)) == "KVS_ERR_UNSUPPORTED"
    assert call(cache=_cache(k=0)) == "KVS_ERR_NULL"
    assert call(scores=None) == "KVS_ERR_NULL"
    assert call(scale=float("nan")) == "KVS_ERR_SHAPE"
    # 129 observers x GQA 4 = 516 rows > 512: two row groups, whose partial sums need workspace
    obs129, _ = _obs(1, Hq=4, O_=129)
    assert call(o=obs129, wsb=8) == "KVS_ERR_WORKSPACE"
    obs_bad, _ = _obs(1, Hq=6)   # not a multiple of Hkv = 4? (Hkv = 1 here, use Hkv=4 cache)
    assert call(cache=_cache(Hkv=4), o=obs_bad) == "KVS_ERR_SHAPE"
    bad = HostSeqs([[0, 1, 9]], [0], [40])          # page 9 outside an 8-page pool
    assert call(s=bad.s) == "KVS_ERR_SHAPE"
    bad = HostSeqs([[0, 1, 2]], [16], [20])         # start out of range
    assert call(s=bad.s) == "KVS_ERR_SHAPE"
    bad = HostSeqs([[0, 1]], [0], [40])             # needs 3 pages, table has 2
    assert call(s=bad.s) == "KVS_ERR_SHAPE"
    assert "outside" in K.lib().kvs_last_error().decode() or "pages" in K.lib().kvs_last_error().decode()


def test_inplace_calls_reject_shared_pages():
    L = K.lib()
    seqs = HostSeqs([[0, 1], [1, 2]], [0, 0], [20, 20])     # page 1 in both sequences
    c = _cache()
    r = L.kvs_lrfu_update(C.byref(c), C.byref(seqs.s), FAKE, 9, 10, FAKE, FAKE, None, None)
    assert status(r) == "KVS_ERR_SHAPE"
    bud = np.array([4, 4], np.int32)
    r = L.kvs_compact(C.byref(c), C.byref(seqs.s), bud.ctypes.data, FAKE, FAKE, None)
    assert status(r) == "KVS_ERR_SHAPE"


def test_lrfu_select_validation():
    L = K.lib()
    seqs = HostSeqs([[0, 1]], [3], [20])
    c = _cache()
    assert status(L.kvs_lrfu_update(C.byref(c), C.byref(seqs.s), FAKE, 11, 10, FAKE, FAKE, None, None)) == "KVS_ERR_SHAPE"
    assert status(L.kvs_lrfu_update(C.byref(c), C.byref(seqs.s), FAKE, 9, 0, FAKE, FAKE, None, None)) == "KVS_ERR_SHAPE"
    assert status(L.kvs_lrfu_update(C.byref(_cache(crf=0)), C.byref(seqs.s), FAKE, 9, 10, FAKE, FAKE, None, None)) == "KVS_ERR_NULL"
    bud = np.array([-1], np.int32)
    assert status(L.kvs_select(C.byref(c), C.byref(seqs.s), FAKE, FAKE, bud.ctypes.data, FAKE, None)) == "KVS_ERR_SHAPE"


def test_lrfu_select_compact_validation():
    L = K.lib()
    seqs = HostSeqs([[0, 1]], [3], [20])
    c = _cache()
    bud = np.array([8], np.int32)
    z = np.zeros(4, np.int32)
    n64 = np.zeros(1, np.int64)
    # hit, budget, budget_h (host), keep, pairs, pair_count, then the host plan outputs
    args = (FAKE, FAKE, bud.ctypes.data, FAKE, FAKE, FAKE, z.ctypes.data, z.ctypes.data, z.ctypes.data,
            z.ctypes.data, 4, n64.ctypes.data, None)
    assert status(L.kvs_lrfu_select_compact(C.byref(c), C.byref(seqs.s), FAKE, 11, 10, FAKE, FAKE, *args)) \
        == "KVS_ERR_SHAPE"
    assert status(L.kvs_lrfu_select_compact(C.byref(c), C.byref(seqs.s), FAKE, 9, 0, FAKE, FAKE, *args)) \
        == "KVS_ERR_SHAPE"
    assert status(L.kvs_lrfu_select_compact(None, C.byref(seqs.s), FAKE, 9, 10, FAKE, FAKE, *args)) \
        == "KVS_ERR_NULL"
    assert status(L.kvs_lrfu_select_compact(C.byref(_cache(crf=0)), C.byref(seqs.s), FAKE, 9, 10, FAKE, FAKE,
                                            *args)) == "KVS_ERR_NULL"
    neg = np.array([-1], np.int32)
    args_neg = (FAKE, FAKE, neg.ctypes.data) + args[3:]
    assert status(L.kvs_lrfu_select_compact(C.byref(c), C.byref(seqs.s), FAKE, 9, 10, FAKE, FAKE, *args_neg)) \
        == "KVS_ERR_SHAPE"


def test_lrfu_decay_matches_oracle():
    for lam in (0.5, 0.0, 0.25, 1.0):
        for dt in range(0, 130):
            assert K.kvs_lrfu_decay(lam, dt) == O.lrfu_decay(lam, dt), (lam, dt)


def test_budget_ratchet_matches_oracle_and_golden(golden_dir):
    vals = [int(x) for x in open(os.path.join(golden_dir, "ratchet_sequence.txt"))
            if x.strip() and not x.startswith("#")]
    b = np.array([512], np.int32)
    seq = [512]
    for _ in range(len(vals) - 1):
        b = K.kvs_budget_ratchet(b, np.array([1], np.uint8))
        seq.append(int(b[0]))
    assert seq == vals
    rng = np.random.default_rng(0)
    b = rng.integers(0, 40000, 200).astype(np.int32)
    f = (rng.random(200) < 0.5).astype(np.uint8)
    got = K.kvs_budget_ratchet(b, f)
    exp = [O.ratchet(int(x), bool(y)) for x, y in zip(b, f)]
    assert got.tolist() == exp


def test_pair_capacity_and_plan_host_match_oracle():
    L = K.lib()
    rng = np.random.default_rng(3)
    S = 7
    length = rng.integers(0, 200, S).astype(np.int32)
    length[2] = 0
    start = rng.integers(0, 16, S).astype(np.int32)
    budget = rng.integers(0, 120, S).astype(np.int32)
    budget[4] = 500
    mp = int(((start + length + 15) // 16).max())
    bt = np.arange(S * mp, dtype=np.int32).reshape(S, mp)
    seqs = HostSeqs(bt, start, length)
    P = L.kvs_pair_capacity(C.byref(seqs.s), budget.ctypes.data)
    Ks = np.minimum(budget, length)
    assert P == int(np.max(np.minimum(length - Ks, Ks)))
    shift = np.zeros(S, np.int32); ns = np.zeros(S, np.int32); nl = np.zeros(S, np.int32)
    freed = np.zeros(bt.size, np.int32); nf = np.zeros(1, np.int64)
    r = L.kvs_plan_host(C.byref(seqs.s), budget.ctypes.data, shift.ctypes.data, ns.ctypes.data,
                        nl.ctypes.data, freed.ctypes.data, bt.size, nf.ctypes.data)
    assert status(r) == "KVS_OK"
    w = 0
    for i in range(S):
        sh, st, ln, fr = O.plan_sequence(int(length[i]), int(Ks[i]), int(start[i]), bt[i])
        assert (shift[i], ns[i], nl[i]) == (sh, st, ln)
        np.testing.assert_array_equal(freed[w:w + sh], fr)
        w += sh
    assert nf[0] == w
    # a freed list that does not fit is an error, not an overrun
    r = L.kvs_plan_host(C.byref(seqs.s), budget.ctypes.data, None, None, None, freed.ctypes.data,
                        max(w - 1, 0), nf.ctypes.data)
    assert status(r) == ("KVS_ERR_SHAPE" if w > 0 else "KVS_OK")


def test_empty_batch_is_a_no_op():
    L = K.lib()
    s = K.Seqs(0, 0, None, None, None, None, None, None, None, None)
    c = _cache()
    o = K.Observers(None, None, None, None, 4, 0)
    assert status(L.kvs_score(C.byref(c), C.byref(s), C.byref(o), C.c_float(0.1), None, None, 0, None)) == "KVS_OK"
    assert L.kvs_score_workspace_size(C.byref(c), C.byref(s), C.byref(o)) == 0


# ---------------------------------------------------------------------------
# confidence monitor: validation of kvs_token_confidence (no launch), host trend


def test_token_confidence_validation():
    L = K.lib()
    f = L.kvs_token_confidence
    ok_args = dict(logits=FAKE, dtype=K.KVS_DTYPE_BF16, rows=4, vocab=128256, stride=128256, k=20,
                   conf=FAKE, ws=FAKE, ws_bytes=1 << 30)

    def call(**kw):
        a = dict(ok_args, **kw)
        return f(a["logits"], a["dtype"], a["rows"], a["vocab"], a["stride"], a["k"], a["conf"], a["ws"],
                 a["ws_bytes"], None)

    assert call(dtype=7) == 3                       # unsupported dtype
    assert call(k=0) == 3 and call(k=65) == 3        # k outside [1, 64]
    assert call(vocab=10, stride=10, k=20) == 2      # k > vocab
    assert call(vocab=(1 << 20) + 1, stride=(1 << 20) + 1) == 3
    assert call(vocab=0) == 2
    assert call(stride=1000) == 2                    # row stride below the vocabulary
    assert call(rows=-1) == 2
    assert call(logits=None) == 1 and call(conf=None) == 1
    assert call(ws=None) == 4 and call(ws_bytes=16) == 4
    assert call(rows=0) == 0                         # nothing to do: no launch
    # sized for fp32 rows: chunks of 16 384 logits for k <= 32, else 8 192; (2 + k)
    # floats per (row, chunk)
    need = L.kvs_token_confidence_workspace_size(4, 128256, 20)
    assert need == 4 * 8 * (2 + 20) * 4
    assert L.kvs_token_confidence_workspace_size(4, 16384, 20) == 0
    assert L.kvs_token_confidence_workspace_size(4, 16385, 32) == 4 * 2 * 34 * 4
    assert L.kvs_token_confidence_workspace_size(4, 8192, 33) == 0
    assert L.kvs_token_confidence_workspace_size(4, 8193, 64) == 4 * 2 * 66 * 4


@pytest.mark.parametrize("n", [0, 1, 63, 64, 71, 72, 200, 4096])
@pytest.mark.parametrize("fit_last", [0, 1, 2, 5])
def test_confidence_trend_matches_oracle(n, fit_last):
    from oracle import confidence as CO
    rng = np.random.default_rng(n * 7 + fit_last)
    for shape in ("noise", "down", "up"):
        c = rng.standard_normal(n).astype(np.float32) * 0.3 + 10
        if shape == "down":
            c -= np.linspace(0, 2, n, dtype=np.float32)
        elif shape == "up":
            c += np.linspace(0, 2, n, dtype=np.float32)
        t = K.kvs_confidence_trend(c, 64, 8, fit_last)
        slope, P, flag = CO.trend_flag(c.astype(np.float64), 64, 8, fit_last)
        np.testing.assert_array_equal(t.pooled, CO.min_pool(c.astype(np.float64), 64, 8))
        assert len(t.pooled) == P and t.flag == flag
        if slope is None:
            assert np.isnan(t.slope)
        else:
            assert t.slope == pytest.approx(slope, rel=1e-12, abs=1e-14)


def test_confidence_trend_validation_and_ratchet():
    L = K.lib()
    flag = np.zeros(1, np.int32)
    c = np.ones(100, np.float32)
    assert L.kvs_confidence_trend(c.ctypes.data, 100, 0, 8, 0, None, None, None, flag.ctypes.data) == 2
    assert L.kvs_confidence_trend(c.ctypes.data, 100, 64, 0, 0, None, None, None, flag.ctypes.data) == 2
    assert L.kvs_confidence_trend(None, 100, 64, 8, 0, None, None, None, flag.ctypes.data) == 1
    assert L.kvs_confidence_trend(c.ctypes.data, 100, 64, 8, 0, None, None, None, None) == 1
    # a declining trajectory raises the flag, which grows the budget by 7/4
    down = (12 - 0.01 * np.arange(300)).astype(np.float32)
    t = K.kvs_confidence_trend(down)
    assert t.flag and t.slope < 0
    assert K.kvs_budget_ratchet(np.array([512], np.int32), np.array([t.flag], np.uint8))[0] == 896


def test_decode_attention_validation():
    L = K.lib()
    hs = HostSeqs([[0, 1]], [0], [20])
    c = _cache(P=2)
    off = np.array([0, 5], np.int64)           # 5 tokens x G = 4 rows = 20 > 16
    q = K.Observers(FAKE, None, FAKE, off.ctypes.data, 4, 5)
    st = L.kvs_decode_attention(C.byref(c), C.byref(hs.s), C.byref(q), C.c_float(0.1), FAKE, FAKE, None,
                                FAKE, 1 << 30, None)
    assert st == 3
    off2 = np.array([0, 4], np.int64)          # 16 rows: allowed
    q2 = K.Observers(FAKE, None, FAKE, off2.ctypes.data, 4, 4)
    assert L.kvs_decode_workspace_size(C.byref(c), C.byref(hs.s), C.byref(q2), 1) > 0
    need = L.kvs_decode_workspace_size(C.byref(c), C.byref(hs.s), C.byref(q2), 0)
    assert 0 < need < L.kvs_decode_workspace_size(C.byref(c), C.byref(hs.s), C.byref(q2), 1)
    assert L.kvs_decode_attention(C.byref(c), C.byref(hs.s), C.byref(q2), C.c_float(0.1), None, FAKE, None,
                                  FAKE, 1 << 30, None) == 1
    assert L.kvs_decode_attention(C.byref(c), C.byref(hs.s), C.byref(q2), C.c_float(0.1), FAKE, FAKE, None,
                                  FAKE, 16, None) == 4
    q3 = K.Observers(FAKE, None, FAKE, off2.ctypes.data, 6, 4)   # 6 heads over 4 KV heads? not a multiple
    c4 = _cache(Hkv=4, P=2)
    assert L.kvs_decode_attention(C.byref(c4), C.byref(hs.s), C.byref(q3), C.c_float(0.1), FAKE, FAKE, None,
                                  FAKE, 1 << 30, None) == 2


def test_step_select_validation():
    # every bad argument is refused on the host (status codes), before any HIP call
    L = K.lib()
    hs = HostSeqs([[0, 1], [2, 3]], [0, 3], [20, 9])
    c = _cache(L=2, Hkv=2, P=4)
    bud = np.array([5, 5], np.int32)

    def run(off, first, beta=0.5, budget=bud, ws_bytes=1 << 20, steps=True):
        off = np.ascontiguousarray(off, np.int64)
        first = np.ascontiguousarray(first, np.int32)
        t = K.Steps(FAKE, off.ctypes.data, FAKE, first.ctypes.data)
        return L.kvs_step_select(C.byref(c), C.byref(hs.s), C.byref(t) if steps else None, FAKE,
                                 C.c_float(beta), FAKE, budget.ctypes.data, FAKE, None, FAKE, ws_bytes, None)

    good_off, good_first = [0, 3, 5], [0, 4, 11, 0, 9]       # the last step of sequence 1 is empty
    for beta in (-0.1, 1.5, float("nan")):
        assert run(good_off, good_first, beta=beta) == 2
    assert run(good_off, good_first, steps=False) == 1
    assert run([1, 3, 5], good_first) == 2                     # step_off[0] != 0
    assert run([0, 3, 2], good_first) == 2                     # not monotone
    assert run([0, 0, 2], [0, 3]) == 2                         # live entries without a step
    assert run(good_off, [1, 4, 11, 0, 9]) == 2                # a sequence's steps start at slot 0
    assert run(good_off, [0, 11, 4, 0, 9]) == 2                # boundaries decrease
    assert run(good_off, [0, 4, 21, 0, 9]) == 2                # past the sequence end
    assert run(good_off, good_first, budget=np.array([5, -1], np.int32)) == 2
    off = np.array([0, 3, 5], np.int64)
    first = np.array([0, 4, 11, 0, 9], np.int32)
    t = K.Steps(FAKE, off.ctypes.data, FAKE, first.ctypes.data)
    assert L.kvs_step_select_workspace_size(C.byref(c), C.byref(hs.s), C.byref(t)) == 2 * 2 * 29 * 4
    st = L.kvs_step_select(C.byref(c), C.byref(hs.s), C.byref(t), FAKE, C.c_float(0.5), FAKE,
                           bud.ctypes.data, FAKE, None, FAKE, 100, None)
    assert st == 4 and L.kvs_last_error().decode().startswith("workspace")


def test_beacon_kmeans_validation():
    L = K.lib()
    ok_args = dict(P=4, N=100, k=16, T=5)

    def run(P=4, N=100, k=16, T=5, pts=FAKE, cent=FAKE):
        return L.kvs_beacon_kmeans(pts, P, N, k, T, cent, None, None, None)

    assert run(P=-1) == 2
    assert run(N=0) == 2
    assert run(k=0) == 3 and run(k=17) == 3
    assert run(N=65537) == 3                           # grid sums would leave int64
    assert run(T=-1) == 2
    assert run(pts=None) == 1 and run(cent=None) == 1
    assert run(P=0, pts=None, cent=None) == 0          # nothing to do
    _ = ok_args


def test_eviction_round_validation():
    L = K.lib()
    hs = HostSeqs([[0, 1]], [0], [20])
    c = _cache(P=2)
    o, off = _obs(1)
    bud = np.array([8], np.int32)

    def run(chunks=2, mass=(9, 10), budget=bud, obs=o, ws_bytes=0):
        return L.kvs_eviction_round(C.byref(c), C.byref(hs.s), C.byref(obs), C.c_float(0.1), mass[0], mass[1],
                                    FAKE, FAKE, FAKE, budget.ctypes.data, FAKE, None, FAKE, FAKE, FAKE, None,
                                    ws_bytes, chunks, None, None, None, None, 0, None, None)

    assert run(chunks=0) == 2
    assert run(mass=(11, 10)) == 2 and run(mass=(1, 0)) == 2
    assert run(budget=np.array([-1], np.int32)) == 2
    o2 = K.Observers(FAKE, FAKE, FAKE, off.ctypes.data, 6, int(off[-1]))     # 6 heads over 1 KV head: fine
    c2 = _cache(Hkv=4, P=2)
    assert L.kvs_eviction_round(C.byref(c2), C.byref(hs.s), C.byref(o2), C.c_float(0.1), 9, 10, FAKE, FAKE, FAKE,
                                bud.ctypes.data, FAKE, None, FAKE, FAKE, FAKE, None, 0, 1, None, None, None,
                                None, 0, None, None) == 2


def test_beacon_seed_validation():
    L = K.lib()

    def run(P=4, N=100, k=16, pts=FAKE, u=FAKE, cent=FAKE):
        return L.kvs_beacon_seed(pts, P, N, k, u, cent, None, None)

    assert run(P=-1) == 2 and run(N=0) == 2
    assert run(N=16385) == 3 and run(k=0) == 3 and run(k=17) == 3
    assert run(pts=None) == 1 and run(u=None) == 1 and run(cent=None) == 1
    assert run(P=0, pts=None, u=None, cent=None) == 0


def test_token_confidence_static_validation():
    """The static-buffer confidence call validates before touching a device: bad shapes,
    null pointers and partial results beyond its 16 MiB buffer are rejected."""
    L = K.lib()

    def run(rows=8, V=1000, stride=1000, k=20, x=FAKE, conf=FAKE, dtype=0):
        return status(L.kvs_token_confidence_static(x, dtype, rows, V, stride, k, conf, None))

    assert run(k=0) == "KVS_ERR_SHAPE" or run(k=0) == "KVS_ERR_UNSUPPORTED"
    assert run(x=None) == "KVS_ERR_NULL" and run(conf=None) == "KVS_ERR_NULL"
    assert run(rows=0, x=None, conf=None) == "KVS_OK"
    assert run(rows=4096, V=1 << 20, stride=1 << 20) == "KVS_ERR_UNSUPPORTED"
    assert b"static buffer" in L.kvs_last_error()
