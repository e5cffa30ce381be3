"""The one-call round (kvs_eviction_round) against the stage calls: with the layers in
1, 2, 3 or 5 chunks (scoring of one chunk overlapped with the cut, keep set and moves
of the previous one), every output matches the staged round bit for bit -- scores,
hits, CRF, keep set, pairs, pair counts, the moved K/V rows and the host plan -- and the
staged round is itself checked against the oracle (tests/gpu_util.check_stages).  The
"short" batch takes the fused selection-and-plan kernel; the "long" batch has a stream of
40 000 entries, so the round takes the long-stream kernels (cut and update, keep set,
plan, then moves)."""
import numpy as np
import pytest

from workloads.edge import random_batch

pytestmark = pytest.mark.gpu


LAYOUTS = {
    # name: (layers, lengths, starts, observers, budgets); Hkv = 2, Hq = 8 (G = 4)
    "short": (5, [700, 333, 0, 1300], [0, 9, 3, 5], [20, 5, 3, 16], [96, 40, 8, 512]),
    "long": (3, [40000, 900, 17], [3, 0, 8], [16, 3, 8], [3000, 64, 20]),
}
CASES = [("short", c) for c in (1, 2, 3, 5)] + [("long", c) for c in (1, 2)]


@pytest.mark.parametrize("layout,chunks", CASES, ids=[f"{n}-{c}" for n, c in CASES])
def test_round_matches_stages(layout, chunks):
    import torch
    import kv_cache_eviction_lse_amd as K
    import oracle as O
    from tests import gpu_util as U
    # MFMA (R >= 16) and VALU (R < 16) scorer paths, ragged batches
    L, lengths, starts, observers, budget = LAYOUTS[layout]
    lay, inp = random_batch(61, L, 2, 8, lengths, starts, observers)
    budget = np.array(budget, np.int32)
    decay = np.array([O.lrfu_decay(0.5, int(d)) for d in lay.dt], np.float32)
    print(f"round {layout} chunks={chunks}", flush=True)
    ref = U.run_stages(lay, inp, 8, budget, decay, fused=True)
    if chunks == 1:
        U.check_stages(lay, inp, ref, 8, budget, decay)
    cache, seqs, obs = U.upload(lay, inp)
    bufs = K.RoundBuffers(cache, seqs, obs, budget, keep_hits=True)
    dev = torch.device("cuda", 0)
    dec = torch.from_numpy(decay).to(dev)
    n_prev = torch.from_numpy(np.asarray(lay.n_prev, np.int32)).to(dev)
    plan = K.eviction_round(cache, seqs, obs, bufs, dec, n_prev, 1.0 / np.sqrt(128.0), layer_chunks=chunks)
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


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
def test_round_repeats_bit_for_bit(layout):
    """Three rounds from identical copies of one state give identical results, bit for
    bit: scores, hits, CRF, keep set, pair counts, pairs and the moved K/V rows.  Every
    reduction and ranking in the kernels runs in a fixed order and the moves' pairs are
    disjoint, so nothing may depend on timing (a race would show up here as a difference
    between the runs)."""
    import torch
    import kv_cache_eviction_lse_amd as K
    import oracle as O
    from tests import gpu_util as U
    L, lengths, starts, observers, budget = LAYOUTS[layout]
    lay, inp = random_batch(83, L, 2, 8, lengths, starts, observers)
    budget = np.array(budget, np.int32)
    dev = torch.device("cuda", 0)
    dec = torch.from_numpy(np.array([O.lrfu_decay(0.5, int(d)) for d in lay.dt], np.float32)).to(dev)
    n_prev = torch.from_numpy(np.asarray(lay.n_prev, np.int32)).to(dev)
    runs = []
    for rep in range(3):
        print(f"repeat {layout} run {rep}", flush=True)
        cache, seqs, obs = U.upload(lay, inp)
        bufs = K.RoundBuffers(cache, seqs, obs, budget, keep_hits=True)
        plan = K.eviction_round(cache, seqs, obs, bufs, dec, n_prev, 1.0 / np.sqrt(128.0))
        torch.cuda.synchronize()
        pc = bufs.pair_count.cpu().numpy()
        pairs = bufs.pairs.cpu().numpy()
        runs.append({
            "s": bufs.scores.cpu().numpy().view(np.uint32), "hit": bufs.hit.cpu().numpy(),
            "keep": bufs.keep.cpu().numpy(), "pc": pc,
            "pairs": [pairs[idx][:int(pc[idx])] for idx in np.ndindex(pc.shape)],
            "k": cache.k.cpu().numpy(), "v": cache.v.cpu().numpy(),
            "crf": cache.crf.cpu().numpy().view(np.uint32), "freed": plan.freed})
    for r in runs[1:]:
        for key in ("s", "hit", "keep", "pc", "k", "v", "crf", "freed"):
            np.testing.assert_array_equal(r[key], runs[0][key], err_msg=key)
        for a, b in zip(r["pairs"], runs[0]["pairs"]):
            np.testing.assert_array_equal(a, b)
