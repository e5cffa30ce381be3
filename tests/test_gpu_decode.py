"""GPU parity of paged decode attention with the LSE and the attention tally
(kvs_decode_attention through the C ABI) against the fp64 oracle on the same bytes.

Tolerances.  Logits are fp32 sums of 128 exact bf16 products; probabilities and the
output accumulate in fp32 over at most a few 10^5 entries with weights <= 1, so the
output is within about 1e-6 of max |v| and the LSE within a few ulp of its value:
|out - ref| <= 1e-4, |lse - ref| <= 1e-5 (1 + |ref|).  The tally is held to the score
bar, 1e-3 relative (it is within about 1e-5), and agrees with kvs_score fed the
emitted LSE to 1e-4: both form 2^(logit log2 e - LSE log2 e) in fp32 from exponent
terms near 20 in magnitude (ulp about 2e-6), summed in different orders (MFMA against
v_dot2), so single terms differ by a few 1e-5 relative.
"""
import numpy as np
import pytest

import oracle as O
from oracle import decode_oracle as DO
from workloads.edge import random_batch

pytestmark = pytest.mark.gpu


def _run(lay, inp, Hq, tally=True, seed=0):
    import torch
    import kv_cache_eviction_lse_amd as K
    from tests.gpu_util import upload
    cache, seqs, _ = upload(lay, inp)
    q = torch.from_numpy(inp.q.view(np.int16)).to("cuda")
    qs = K.DecodeQueries(q, lay.obs_off)
    L, T = inp.q.shape[0], inp.q.shape[2]
    out = torch.full((L, Hq, T, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((L, Hq, T), float("nan"), dtype=torch.float32, device="cuda")
    E = int(lay.entry_off[-1])
    Hkv = inp.k_pool.shape[2]
    s0 = np.random.default_rng(seed).random((L, Hkv, max(E, 1))).astype(np.float32)
    scores = torch.from_numpy(s0.copy()).to("cuda") if tally else None
    ws = torch.empty(max(K.kvs_decode_workspace_size(cache, seqs, qs, tally), 256), dtype=torch.uint8,
                     device="cuda")
    K.kvs_decode_attention(cache, seqs, qs, 1.0 / np.sqrt(128.0), out, lse, scores, ws)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy(), "lse": lse.cpu().numpy()}
    if tally:
        res["tally"] = scores.cpu().numpy() - s0
        res["scores"] = scores.cpu().numpy()
    return res, (cache, seqs, qs, lse)


def _check(lay, inp, Hq, res, tally=True):
    L, P, Hkv = inp.k_pool.shape[:3]
    G = Hq // Hkv
    ref = DO.decode_attention(inp.k_pool, inp.v_pool, inp.q, lay.obs_off, lay.block_table, lay.start,
                              lay.length, Hq, 1.0 / np.sqrt(128.0))
    for (i, l, g), (o, lse, t) in ref.items():
        t0, t1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
        T = t1 - t0
        for r in range(o.shape[0]):
            h, tok = g * G + r // T, t0 + r % T
            got_o, got_l = res["out"][l, h, tok], res["lse"][l, h, tok]
            if lay.length[i] == 0:
                assert np.all(got_o == 0) and got_l == -np.inf
                continue
            assert np.max(np.abs(got_o - o[r])) <= 1e-4, (i, l, g, r)
            assert abs(got_l - lse[r]) <= 1e-5 * (1 + abs(lse[r])), (i, l, g, r, got_l, lse[r])
        if tally and lay.length[i] > 0 and T > 0:
            e0, e1 = int(lay.entry_off[i]), int(lay.entry_off[i + 1])
            got_t = res["tally"][l, g, e0:e1].astype(np.float64)
            # the tally was added to values in [0, 1): compare with that absolute floor
            err = np.abs(got_t - t) / np.maximum(t, 1e-3)
            assert err.max() <= 1e-3, (i, l, g, float(err.max()))


@pytest.mark.parametrize("case", ["ragged", "gqa8_two_tokens", "long", "split_edges"])
def test_decode_attention_parity(case):
    if case == "ragged":
        # G = 4; lengths with partial first pages, an empty sequence, one entry, and
        # sequences with 1, 2 and 4 tokens (4 .. 16 rows per KV head)
        lay, inp = random_batch(31, 2, 2, 8, [700, 333, 0, 1, 16, 5000], [0, 9, 3, 15, 0, 7],
                                [1, 2, 1, 1, 4, 1], prior_crf=False)
        Hq = 8
    elif case == "gqa8_two_tokens":
        lay, inp = random_batch(32, 1, 2, 16, [1029, 4100], [3, 0], [2, 1], prior_crf=False)
        Hq = 16
    elif case == "long":
        lay, inp = random_batch(33, 1, 1, 4, [40000], [11], [1], prior_crf=False, planted=0.02)
        Hq = 4
    else:
        # live ranges that end exactly on a split boundary (1 024 positions), one past
        # it (a split with one key), on the second boundary, and within the first tile
        lay, inp = random_batch(35, 1, 2, 8, [1009, 1010, 2033, 49], [15, 15, 15, 15], [1, 2, 1, 4],
                                prior_crf=False)
        Hq = 8
    print(f"decode parity {case}", flush=True)
    res, _ = _run(lay, inp, Hq)
    _check(lay, inp, Hq, res)


def test_decode_without_tally_and_consistency_with_scorer():
    # the same outputs without a tally; and the tally equals kvs_score fed the LSE that
    # the decode call emitted (both GPU, same definition)
    import torch
    import kv_cache_eviction_lse_amd as K
    lay, inp = random_batch(34, 2, 2, 8, [2000, 777], [5, 0], [1, 3], prior_crf=False)
    print("decode consistency", flush=True)
    res_t, (cache, seqs, qs, lse_dev) = _run(lay, inp, 8, tally=True)
    res_n, _ = _run(lay, inp, 8, tally=False)
    np.testing.assert_array_equal(res_t["out"], res_n["out"])
    np.testing.assert_array_equal(res_t["lse"], res_n["lse"])
    q = torch.from_numpy(inp.q.view(np.int16)).to("cuda")
    obs = K.ObserverSet(q, lse_dev, lay.obs_off)
    E = int(lay.entry_off[-1])
    s = torch.zeros((2, 2, E), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(K.kvs_score_workspace_size(cache, seqs, obs), 256), dtype=torch.uint8, device="cuda")
    K.kvs_score(cache, seqs, obs, 1.0 / np.sqrt(128.0), s, ws)
    torch.cuda.synchronize()
    sv = s.cpu().numpy().astype(np.float64)
    tv = res_t["tally"].astype(np.float64)
    assert np.max(np.abs(tv - sv) / np.maximum(sv, 1e-3)) <= 1e-4
