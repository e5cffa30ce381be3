"""The one-call round (kvs_eviction_round) against the stage calls: with the layers in
1, 2, 3 or 5 chunks (scoring of one chunk overlapped with the cut, keep set and moves
of the previous one), every output matches the staged round bit for bit -- scores,
hits, CRF, keep set, pairs, pair counts, the moved K/V rows and the host plan -- and the
staged round is itself checked against the oracle (tests/gpu_util.check_stages)."""
import numpy as np
import pytest

from workloads.edge import random_batch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("chunks", [1, 2, 3, 5])
def test_round_matches_stages(chunks):
    import torch
    import kv_cache_eviction_lse_amd as K
    import oracle as O
    from tests import gpu_util as U
    # 5 layers, G = 4; MFMA (20 observers) and VALU (5) scorer paths, a ragged batch
    lay, inp = random_batch(61, 5, 2, 8, [700, 333, 0, 1300], [0, 9, 3, 5], [20, 5, 3, 16])
    budget = np.array([96, 40, 8, 512], np.int32)
    decay = np.array([O.lrfu_decay(0.5, int(d)) for d in lay.dt], np.float32)
    print(f"round chunks={chunks}", flush=True)
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
