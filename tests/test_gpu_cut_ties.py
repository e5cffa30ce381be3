"""GPU parity of the attention-mass cut, the LRFU update and the keep set on crafted
scores (kvs_lrfu_update + kvs_select, and the fused kvs_lrfu_select, through the C ABI).

ActKV Dissected, Component 1: the entries holding the top 90 % of the tallied action
attention are hits.  The cut is defined on integer masses m = floor(s 2^32) with ties
in s going to the lower slot; the scores here are written straight into the scores
buffer, so exact ties at the threshold, zero mass, masses below the grid, subnormal
scores, one dominant entry and masses near 2^42 all reach the device kernels.  Both the
register-resident kernel (streams up to 32 768 entries) and the global-memory kernels
(longer streams) are covered.  Hits, CRF and keep bits must equal the oracle's bit for
bit on the same fp32 inputs.
"""
import zlib

import numpy as np
import pytest

import oracle as O
from tests import gpu_util as U
from workloads.edge import CRAFTED_KINDS, crafted_scores, quantised_priors, random_batch

pytestmark = pytest.mark.gpu

L, HKV, HQ = 2, 2, 4
LAYOUTS = {
    # every stream fits the register-resident kernel
    "register": ([700, 5000, 32768, 1, 2049], [0, 7, 0, 15, 3]),
    # a stream beyond 32 768 entries: the batch takes the global-memory kernels
    "global": ([40000, 33001, 300, 9], [5, 0, 11, 0]),
}


def _run(name, fused, mass, dt):
    import torch
    import kv_cache_eviction_lse_amd as K
    lengths, starts = LAYOUTS[name]
    seed = zlib.crc32(f"{name}{fused}{mass}{dt}".encode())
    rng = np.random.default_rng(seed)
    S = len(lengths)
    lay, inp = random_batch(seed, L, HKV, HQ, lengths, starts, [1] * S, planted=0.0)
    lay.n_prev[:] = lay.length
    lay.n_prev[0] = max(0, int(lay.length[0]) - 37)          # new entries: prior 0
    E = int(lay.entry_off[-1])
    scores = np.zeros((L, HKV, E), np.float32)
    kinds = {}
    t = 0
    for i in range(S):
        n, e0 = int(lay.length[i]), int(lay.entry_off[i])
        for l in range(L):
            for g in range(HKV):
                kind = CRAFTED_KINDS[(t + seed) % len(CRAFTED_KINDS)]
                t += 1
                kinds[(i, l, g)] = kind
                scores[l, g, e0:e0 + n] = crafted_scores(rng, n, kind)
                if (i + l + g) % 2 == 0:                      # tied priors on half the streams
                    page, row = O.slot_location(lay.block_table[i], lay.start[i], np.arange(n))
                    inp.crf_pool[l, page, g, row] = quantised_priors(rng, n)
    budget = np.array([int(rng.integers(0, n + 2)) if j % 3 else (0 if j % 2 else n)
                       for j, n in enumerate(lay.length.tolist())], np.int32)
    decay_h = np.full(S, O.lrfu_decay(0.5, dt), np.float32)
    dev = torch.device("cuda", 0)
    cache, seqs, obs = U.upload(lay, inp)
    crf0 = cache.crf.cpu().numpy()
    s_dev = torch.from_numpy(scores).to(dev)
    hit = torch.zeros((L, HKV, max(E, 1)), dtype=torch.uint8, device=dev)
    keep = torch.zeros_like(hit)
    decay = torch.from_numpy(decay_h).to(dev)
    n_prev = torch.from_numpy(lay.n_prev.astype(np.int32)).to(dev)
    bud = torch.from_numpy(budget).to(dev)
    print(f"cut ties {name} fused={fused} mass={mass} dt={dt} n={lengths} B={budget.tolist()}", flush=True)
    if fused:
        K.kvs_lrfu_select(cache, seqs, s_dev, mass[0], mass[1], decay, n_prev, bud, budget, keep, hit=hit)
    else:
        K.kvs_lrfu_update(cache, seqs, s_dev, mass[0], mass[1], decay, n_prev, hit)
        K.kvs_select(cache, seqs, s_dev, bud, budget, keep)
    torch.cuda.synchronize()
    hit_g = hit.cpu().numpy().astype(bool)
    keep_g = keep.cpu().numpy().astype(bool)
    crf1 = cache.crf.cpu().numpy()
    ties_at_cut = 0
    for (i, l, g), kind in kinds.items():
        n, e0 = int(lay.length[i]), int(lay.entry_off[i])
        s = scores[l, g, e0:e0 + n]
        want_hit = O.mass_cut(s, *mass)
        np.testing.assert_array_equal(hit_g[l, g, e0:e0 + n], want_hit, err_msg=f"hit {(i, l, g)} {kind}")
        if want_hit.any():
            tau = s[want_hit].min()
            ties_at_cut += int(np.sum(~want_hit & (s == tau)) > 0)
        page, row = O.slot_location(lay.block_table[i], lay.start[i], np.arange(n))
        want_crf = O.lrfu_update(crf0[l, page, g, row], want_hit, decay_h[i], int(lay.n_prev[i]))
        np.testing.assert_array_equal(crf1[l, page, g, row].view(np.uint32), want_crf.view(np.uint32),
                                      err_msg=f"crf {(i, l, g)} {kind}")
        want_keep = O.select_top_b(want_crf, s, int(budget[i]))
        np.testing.assert_array_equal(keep_g[l, g, e0:e0 + n], want_keep, err_msg=f"keep {(i, l, g)} {kind}")
    return ties_at_cut


@pytest.mark.parametrize("name", list(LAYOUTS))
@pytest.mark.parametrize("fused", [False, True])
def test_cut_on_crafted_scores(name, fused):
    # the 90 % cut and the keep set at two decays: dt = 64 makes every hit's CRF round to
    # exactly 1.0 (ties decided by s, then slot); dt = 2 keeps the priors' ties
    ties = _run(name, fused, (9, 10), 64) + _run(name, fused, (9, 10), 2)
    assert ties > 0          # the tie branch of the cut was taken


@pytest.mark.parametrize("mass", [(1, 2), (1, 1)])
def test_cut_other_fractions(mass):
    # half of the mass, and all of it (every entry of positive integer mass is a hit)
    _run("register", False, mass, 8)
    _run("global", True, mass, 8)
