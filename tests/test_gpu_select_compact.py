"""kvs_lrfu_select_compact (the cut, LRFU update, keep set, slot plan and moves in one
call) against the two calls it fuses, kvs_lrfu_select then kvs_plan_compact: hits, keep
set, the final CRF pool, pairs, pair counts, the moved K/V rows and the host plan match
bit for bit.  The staged calls are themselves checked against the oracle
(tests/gpu_util.check_stages).  Cases cover the fused path (selection and plan in one
kernel for streams up to 32 768 entries: ragged lengths, an empty and a one-entry
sequence, budgets of 0, below n and at least n, start offsets, quantised priors that tie
at the threshold, a stream with 8 000 pairs) and the fallback to the two calls (a
40 000-entry stream)."""
import numpy as np
import pytest

from workloads.edge import quantised_priors, random_batch

pytestmark = pytest.mark.gpu

CASES = {
    # name: (lengths, starts, observers, budgets, quantised priors)
    "ragged": ([700, 333, 0, 1300, 1], [0, 9, 3, 5, 15], [20, 5, 3, 16, 4], [96, 40, 8, 512, 1], False),
    "budgets": ([2000, 2000, 2000, 9], [0, 7, 15, 2], [16, 8, 16, 4], [0, 1999, 5000, 3], False),
    "ties": ([5000, 2048, 777], [3, 0, 11], [16, 16, 5], [512, 300, 100], True),
    "full_stream": ([32768, 513], [0, 4], [16, 8], [512, 200], False),
    "many_pairs": ([20000, 700], [1, 0], [8, 4], [8000, 100], False),
    "long_stream": ([40000, 900], [0, 6], [8, 16], [4096, 64], False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_select_compact_matches_two_calls(name):
    import torch
    import kv_cache_eviction_lse_amd as K
    import oracle as O
    from tests import gpu_util as U
    lengths, starts, observers, budget, quant = CASES[name]
    print(f"select_compact case={name}", flush=True)
    lay, inp = random_batch(97 + len(name), 2, 2, 8, lengths, starts, observers)
    if quant:
        inp.crf_pool[...] = quantised_priors(np.random.default_rng(5), inp.crf_pool.shape)
    budget = np.asarray(budget, np.int32)
    decay = np.array([O.lrfu_decay(0.5, int(d)) for d in lay.dt], np.float32)
    ref = U.run_stages(lay, inp, 8, budget, decay, fused=True)
    if name in ("ragged", "ties"):
        U.check_stages(lay, inp, ref, 8, budget, decay)
    cache, seqs, obs = U.upload(lay, inp)
    bufs = K.RoundBuffers(cache, seqs, obs, budget, keep_hits=True)
    dev = torch.device("cuda", 0)
    dec = torch.from_numpy(decay).to(dev)
    n_prev = torch.from_numpy(np.asarray(lay.n_prev, np.int32)).to(dev)
    K.kvs_score(cache, seqs, obs, 1.0 / np.sqrt(128.0), bufs.scores, bufs.workspace)
    plan = K.kvs_lrfu_select_compact(cache, seqs, bufs.scores, 9, 10, dec, n_prev, bufs.budget, bufs.budget_h,
                                     bufs.keep, bufs.pairs, bufs.pair_count, hit=bufs.hit)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bufs.scores.cpu().numpy(), ref["s"])
    np.testing.assert_array_equal(bufs.hit.cpu().numpy().astype(bool), ref["hit"])
    np.testing.assert_array_equal(bufs.keep.cpu().numpy().astype(bool), ref["keep"])
    np.testing.assert_array_equal(bufs.pair_count.cpu().numpy(), ref["pair_count"])
    pc = ref["pair_count"]
    got_pairs = bufs.pairs.cpu().numpy()
    for idx in np.ndindex(pc.shape):
        n = int(pc[idx])
        np.testing.assert_array_equal(got_pairs[idx][:n], ref["pairs"][idx][:n])
    np.testing.assert_array_equal(cache.k.cpu().numpy().view(np.uint16), ref["k1"])
    np.testing.assert_array_equal(cache.v.cpu().numpy().view(np.uint16), ref["v1"])
    np.testing.assert_array_equal(cache.crf.cpu().numpy().view(np.uint32), ref["crf2"].view(np.uint32))
    for f in ("shift", "new_start", "new_len", "freed"):
        np.testing.assert_array_equal(getattr(plan, f), getattr(ref["plan"], f))
