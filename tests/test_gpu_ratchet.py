"""The ratchet loop on the GPU, checked round by round with teacher forcing.

One Llama-3-8B-shaped sequence (32 layers x 8 KV heads x 32 query heads) is prefilled
with 8 192 tokens; each of 387 rounds appends 64 tokens, draws 32 fresh observers per
query head with their LSE over the live entries, draws the budget flag (Bernoulli 0.05,
budget x7/4 capped at 30 000, never shrinking), and runs a full eviction round with
dt = 64.  Freed pages go back to a host free list and appended tokens take pages from
it.  On the checked rounds the oracle's input is the GPU state just before the round
(the sampled streams' pages, CRF, observers and LSE), so one boundary decision cannot
cascade into later rounds.
"""
import numpy as np
import pytest

import oracle as O
from tests import gpu_util as U
from workloads import RATCHET, philox
from workloads.configs import TAG_FLAG
from workloads.host import make_layout, observers

pytestmark = pytest.mark.gpu

CHECK_STREAMS = [(0, 0, 0), (0, 31, 7)]
OBS = 32
APPEND = 64


@pytest.mark.timeout(900)
def test_ratchet_loop_teacher_forced():
    import torch
    import kv_cache_eviction_lse_amd as K
    from workloads import device as DV
    w = RATCHET
    dev = torch.device("cuda", 0)
    L, Hkv, Hq, G, D = w.num_layers, w.num_kv_heads, w.num_q_heads, w.group, w.head_dim
    lay = make_layout(w)
    q0 = observers(w, lay, only_heads=True, heads=set())
    d = DV.fill(w, lay, q0, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.key & 0x7FFFFFFFFFFFFFFF ^ 0x5A5A)
    P = lay.num_pages
    n = int(lay.length[0])
    start = int(lay.start[0])
    npg0 = (start + n + 15) // 16
    pages = [int(p) for p in lay.block_table[0][:npg0]]
    used = set(pages)
    free = [p for p in range(P) if p not in used]
    n_prev = 0                      # the prefill has no LRFU state
    budget = int(w.budget)
    R = w.rounds
    flags = philox.uniform01(philox.words(w.key, TAG_FLAG, np.arange(R, dtype=np.uint64))[0]) < w.flag_prob
    decay_h = np.array([K.kvs_lrfu_decay(0.5, APPEND)], np.float32)
    decay = torch.from_numpy(decay_h).to(dev)
    flag_rounds = [r + 1 for r in np.flatnonzero(flags)[:3]]
    check = sorted({1, 2, 3, R} | set(range(40, R, 40)) | set(flag_rounds))
    cache = K.PagedCache(d.k, d.v, d.crf)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_ms, entries_timed, checked, pinned_total = 0.0, 0, 0, 0
    worst = 0.0
    max_budget = budget
    for r in range(1, R + 1):
        # 1. this round's observers
        q = torch.randn((L, Hq, OBS, D), generator=gen, device=dev).to(torch.bfloat16)
        qf = q.float()
        # 2. append 64 tokens (2 % planted towards one of this round's observer rows)
        pos = start + n + np.arange(APPEND)
        while len(pages) < (pos[-1] // 16) + 1:
            pages.append(free.pop(0))
        pg = torch.from_numpy(np.asarray(pages, np.int64)[pos // 16]).to(dev)
        rw = torch.from_numpy(pos % 16).to(dev)
        for l in range(L):
            z = torch.randn((APPEND, Hkv, D), generator=gen, device=dev)
            qr = qf[l].reshape(Hkv, G * OBS, D)
            qn = qr / qr.norm(dim=2, keepdim=True)
            pm = torch.rand((APPEND, Hkv), generator=gen, device=dev) < w.planted_frac
            rr = torch.randint(0, G * OBS, (APPEND, Hkv), generator=gen, device=dev)
            gi = torch.arange(Hkv, device=dev)[None, :].expand(APPEND, Hkv)
            z = torch.where(pm[:, :, None], 3.0 * qn[gi, rr] + z, z)
            d.k[l][pg, :, rw, :] = z.to(torch.bfloat16).view(torch.int16)
            d.v[l][pg, :, rw, :] = torch.randn((APPEND, Hkv, D), generator=gen, device=dev) \
                .to(torch.bfloat16).view(torch.int16)
        n_prev = n
        n += APPEND
        # 3. LSE of every observer row over the live entries
        live = start + np.arange(n)
        lpg = torch.from_numpy(np.asarray(pages, np.int64)[live // 16]).to(dev)
        lrw = torch.from_numpy(live % 16).to(dev)
        lse = torch.empty((L, Hq, OBS), dtype=torch.float32, device=dev)
        for l in range(L):
            keys = d.k[l][lpg, :, lrw, :].view(torch.bfloat16).float()
            lse[l] = DV.live_lse(keys, qf[l].reshape(Hkv, G * OBS, D), w.scale).reshape(Hq, OBS)
        # 4. the budget flag
        nb = int(K.kvs_budget_ratchet(np.array([budget], np.int32), np.array([flags[r - 1]], np.int32))[0])
        assert nb == O.ratchet(budget, bool(flags[r - 1])), (r, budget, nb)
        budget = nb
        max_budget = max(max_budget, budget)
        # 5. the round
        bt = np.asarray(pages, np.int32)[None, :]
        seqs = K.SeqBatch(bt, np.array([start], np.int32), np.array([n], np.int32), device=dev)
        obs = K.ObserverSet(q.view(torch.int16), lse, np.array([0, OBS], np.int64), device=dev)
        budget_h = np.array([budget], np.int32)
        bufs = K.RoundBuffers(cache, seqs, obs, budget_h, keep_hits=True)
        n_prev_t = torch.tensor([n_prev], dtype=torch.int32, device=dev)
        if r in check:
            pre = {}
            pt = torch.from_numpy(np.asarray(pages, np.int64)).to(dev)
            for (i, l, g) in CHECK_STREAMS:
                pre[(i, l, g)] = {
                    "k": d.k[l][pt, g].cpu().numpy().view(np.uint16),
                    "v": d.v[l][pt, g].cpu().numpy().view(np.uint16),
                    "crf": d.crf[l][pt, g].cpu().numpy(),
                    "q": q[l, g * G:(g + 1) * G].view(torch.int16).cpu().numpy().view(np.uint16),
                    "lse": lse[l, g * G:(g + 1) * G].cpu().numpy(),
                }
            rec = {s: {"crf0": pre[s]["crf"], "kv0": (pre[s]["k"], pre[s]["v"])} for s in CHECK_STREAMS}

            def grab(tag, fn):
                torch.cuda.synchronize()
                for s in CHECK_STREAMS:
                    rec[s][tag] = fn(s)
            K.kvs_score(cache, seqs, obs, w.scale, bufs.scores, bufs.workspace)
            grab("s", lambda s: bufs.scores[s[1], s[2], :n].cpu().numpy())
            K.kvs_lrfu_update(cache, seqs, bufs.scores, 9, 10, decay, n_prev_t, bufs.hit)
            grab("hit", lambda s: bufs.hit[s[1], s[2], :n].cpu().numpy().astype(bool))
            grab("crf1", lambda s: d.crf[s[1]][pt, s[2]].cpu().numpy())
            K.kvs_select(cache, seqs, bufs.scores, bufs.budget, bufs.budget_h, bufs.keep)
            grab("keep", lambda s: bufs.keep[s[1], s[2], :n].cpu().numpy().astype(bool))
            plan = K.kvs_plan(seqs, L, Hkv, bufs.keep, bufs.budget, bufs.budget_h, bufs.pairs, bufs.pair_count)
            grab("pairs", lambda s: bufs.pairs[s[1], s[2], 0, :int(bufs.pair_count[s[1], s[2], 0])].cpu().numpy())
            K.kvs_compact(cache, seqs, bufs.budget_h, bufs.pairs, bufs.pair_count)
            grab("kv1", lambda s: (d.k[s[1]][pt, s[2]].cpu().numpy().view(np.uint16),
                                   d.v[s[1]][pt, s[2]].cpu().numpy().view(np.uint16)))
            grab("crf2", lambda s: d.crf[s[1]][pt, s[2]].cpu().numpy())
            npg = len(pages)
            for s in CHECK_STREAMS:
                p_ = pre[s]
                kp = p_["k"][None, :, None]
                vp = p_["v"][None, :, None]
                cp = p_["crf"][None, :, None].copy()
                res = O.eviction_round(kp.copy(), vp.copy(), cp, p_["q"][None], p_["lse"][None],
                                       np.array([0, OBS], np.int64), np.arange(npg, dtype=np.int32)[None, :],
                                       np.array([start]), np.array([n]), G, w.scale, 0.5, np.array([APPEND]),
                                       np.array([n_prev]), np.array([budget]))
                plan3 = (plan.shift[0], plan.new_start[0], plan.new_len[0])
                w_, pn, bad = U.check_stream_record(res, rec[s], n, start, budget, decay_h[0], n_prev, plan3,
                                                    np.arange(npg), 1e-3, (r, s))
                assert bad == 0, (r, s, bad)
                worst = max(worst, w_)
                pinned_total += pn
            checked += 1
        else:
            ev0.record()
            plan = K.eviction_round(cache, seqs, obs, bufs, decay, n_prev_t, w.scale)
            ev1.record()
            torch.cuda.synchronize()
            t_ms += ev0.elapsed_time(ev1)
            entries_timed += n * L * Hkv
        # 6. the host side of the plan: pages at the front are freed
        shift = int(plan.shift[0])
        assert list(plan.freed) == pages[:shift]
        free.extend(pages[:shift])
        pages = pages[shift:]
        start, n = int(plan.new_start[0]), int(plan.new_len[0])
        assert n == min(budget, n_prev + APPEND)
        if r % 50 == 0:
            print(f"round {r}: budget {budget}, live {n}, pages {len(pages)}", flush=True)
    print(f"ratchet: {R} rounds, {checked} checked (max rel score err {worst:.2e}, {pinned_total} keep bits "
          f"pinned), final budget {budget} (max {max_budget}); amortised {entries_timed / (t_ms / 1e3):.3e} "
          f"entries/s over {R - checked} timed rounds", flush=True)
    assert budget == max_budget
