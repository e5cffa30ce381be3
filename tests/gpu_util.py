"""Shared helpers of the GPU parity tests: upload host-generated inputs, run the
five C-ABI calls one at a time (reading every intermediate back), and compare
each stage with the oracle on identical inputs."""
from __future__ import annotations

import numpy as np

import oracle as O

PAGE = 16


def _dev():
    import torch
    return torch.device("cuda", 0)


def upload(lay, inp):
    import torch
    import kv_cache_eviction_lse_amd as K
    dev = _dev()
    k = torch.from_numpy(inp.k_pool.view(np.int16)).to(dev)
    v = torch.from_numpy(inp.v_pool.view(np.int16)).to(dev)
    crf = torch.from_numpy(inp.crf_pool.copy()).to(dev)
    q = torch.from_numpy(inp.q.view(np.int16)).to(dev)
    lse = torch.from_numpy(inp.lse.copy()).to(dev)
    cache = K.PagedCache(k, v, crf)
    seqs = K.SeqBatch(lay.block_table, lay.start, lay.length, device=dev)
    obs = K.ObserverSet(q, lse, lay.obs_off, device=dev)
    return cache, seqs, obs


def run_stages(lay, inp, Hq, budget, decay_h, mass=(9, 10), scale=None, fused=False):
    """Run the round stage by stage on the GPU; return every intermediate on the host.
    fused: run the cut, LRFU update and keep set through kvs_lrfu_select, and the plan
    and the move through kvs_plan_compact."""
    import torch
    import kv_cache_eviction_lse_amd as K
    dev = _dev()
    cache, seqs, obs = upload(lay, inp)
    bufs = K.RoundBuffers(cache, seqs, obs, np.asarray(budget, np.int32), keep_hits=True)
    decay = torch.from_numpy(np.asarray(decay_h, np.float32)).to(dev)
    n_prev = torch.from_numpy(np.asarray(lay.n_prev, np.int32)).to(dev)
    scale = 1.0 / np.sqrt(128.0) if scale is None else scale
    out = {}
    K.kvs_score(cache, seqs, obs, scale, bufs.scores, bufs.workspace)
    torch.cuda.synchronize()
    out["s"] = bufs.scores.cpu().numpy()
    out["crf0"] = cache.crf.cpu().numpy()
    if fused:
        K.kvs_lrfu_select(cache, seqs, bufs.scores, mass[0], mass[1], decay, n_prev, bufs.budget,
                          bufs.budget_h, bufs.keep, hit=bufs.hit)
        torch.cuda.synchronize()
        out["hit"] = bufs.hit.cpu().numpy().astype(bool)
        out["crf1"] = cache.crf.cpu().numpy()
    else:
        K.kvs_lrfu_update(cache, seqs, bufs.scores, mass[0], mass[1], decay, n_prev, bufs.hit)
        torch.cuda.synchronize()
        out["hit"] = bufs.hit.cpu().numpy().astype(bool)
        out["crf1"] = cache.crf.cpu().numpy()
        K.kvs_select(cache, seqs, bufs.scores, bufs.budget, bufs.budget_h, bufs.keep)
        torch.cuda.synchronize()
    out["keep"] = bufs.keep.cpu().numpy().astype(bool)
    out["k0"] = cache.k.cpu().numpy().view(np.uint16)
    out["v0"] = cache.v.cpu().numpy().view(np.uint16)
    if fused:
        plan = K.kvs_plan_compact(cache, seqs, bufs.keep, bufs.budget, bufs.budget_h, bufs.pairs,
                                  bufs.pair_count)
    else:
        plan = K.kvs_plan(seqs, cache.c.num_layers, cache.c.num_kv_heads, bufs.keep, bufs.budget,
                          bufs.budget_h, bufs.pairs, bufs.pair_count)
    torch.cuda.synchronize()
    out["plan"] = plan
    out["pairs"] = bufs.pairs.cpu().numpy()
    out["pair_count"] = bufs.pair_count.cpu().numpy()
    out["P"] = bufs.P
    if not fused:
        K.kvs_compact(cache, seqs, bufs.budget_h, bufs.pairs, bufs.pair_count)
    torch.cuda.synchronize()
    out["k1"] = cache.k.cpu().numpy().view(np.uint16)
    out["v1"] = cache.v.cpu().numpy().view(np.uint16)
    out["crf2"] = cache.crf.cpu().numpy()
    return out


def streams_of(lay, L, Hkv):
    return [(i, l, g) for i in range(len(lay.length)) for l in range(L) for g in range(Hkv)
            if lay.length[i] > 0]


def check_stages(lay, inp, out, Hq, budget, decay_h, mass=(9, 10), score_rtol=1e-3, scale=None):
    """Component parity: scores within tolerance; every later stage exact on the GPU's
    own inputs.  Returns the largest relative score error."""
    L, P, Hkv = inp.k_pool.shape[:3]
    scale = 1.0 / np.sqrt(128.0) if scale is None else scale
    ora_s = O.score(inp.k_pool, inp.q, inp.lse, lay.obs_off, lay.block_table, lay.start,
                    lay.length, Hq, scale, streams=streams_of(lay, L, Hkv))
    worst = 0.0
    exp_k, exp_v, exp_c = out["k0"].copy(), out["v0"].copy(), out["crf1"].copy()
    for (i, l, g), s_ora in ora_s.items():
        e0, e1 = int(lay.entry_off[i]), int(lay.entry_off[i + 1])
        n = e1 - e0
        s_gpu = out["s"][l, g, e0:e1]
        if n:
            denom = np.maximum(np.abs(s_ora.astype(np.float64)), 1e-30)
            err = np.abs(s_gpu.astype(np.float64) - s_ora.astype(np.float64)) / denom
            nz = s_ora > 0
            if nz.any():
                worst = max(worst, float(err[nz].max()))
                assert err[nz].max() <= score_rtol, (i, l, g, float(err[nz].max()))
            assert np.all(s_gpu[~nz] == 0) if (~nz).any() else True
        # cut + LRFU on the GPU's own scores
        hit = O.mass_cut(s_gpu, *mass)
        np.testing.assert_array_equal(out["hit"][l, g, e0:e1], hit, err_msg=f"hit {(i, l, g)}")
        page, row = O.slot_location(lay.block_table[i], lay.start[i], np.arange(n))
        prior = out["crf0"][l, page, g, row]
        crf_new = O.lrfu_update(prior, hit, np.float32(decay_h[i]), int(lay.n_prev[i]))
        got = out["crf1"][l, page, g, row]
        np.testing.assert_array_equal(got.view(np.uint32), crf_new.view(np.uint32),
                                      err_msg=f"crf {(i, l, g)}")
        # top-B on the GPU's CRF and scores
        keep = O.select_top_b(got, s_gpu, int(budget[i]))
        np.testing.assert_array_equal(out["keep"][l, g, e0:e1], keep, err_msg=f"keep {(i, l, g)}")
        # plan on the GPU's keep mask
        src, dst = O.plan_stream(out["keep"][l, g, e0:e1])
        cnt = int(out["pair_count"][l, g, i])
        assert cnt == len(src), ((i, l, g), cnt, len(src))
        if cnt:
            gp = out["pairs"][l, g, i, :cnt]
            np.testing.assert_array_equal(gp[:, 0], src)
            np.testing.assert_array_equal(gp[:, 1], dst)
        O.compact_stream(exp_k, exp_v, exp_c, l, g, lay.block_table[i], lay.start[i], src, dst)
    # host outputs of the plan
    for i in range(len(lay.length)):
        n = int(lay.length[i])
        K_ = min(int(budget[i]), n)
        sh, ns, nl, fr = O.plan_sequence(n, K_, int(lay.start[i]), lay.block_table[i])
        assert (out["plan"].shift[i], out["plan"].new_start[i], out["plan"].new_len[i]) == (sh, ns, nl)
    fr_all = np.concatenate([O.plan_sequence(int(lay.length[i]), min(int(budget[i]), int(lay.length[i])),
                                             int(lay.start[i]), lay.block_table[i])[3]
                             for i in range(len(lay.length))] or [np.zeros(0, np.int32)])
    np.testing.assert_array_equal(out["plan"].freed, fr_all)
    # compaction: every byte of every pool
    np.testing.assert_array_equal(out["k1"], exp_k)
    np.testing.assert_array_equal(out["v1"], exp_v)
    np.testing.assert_array_equal(out["crf2"].view(np.uint32), exp_c.view(np.uint32))
    return worst


def pinned_keep_check(s_ora, crf_ora, keep_ora, hit_ora, s_gpu, crf_gpu, keep_gpu, tol=1e-3):
    """End-to-end keep parity wherever the oracle's margins exceed the score tolerance.

    tau = smallest oracle score among the hits (cut threshold); b = the oracle's last
    kept entry in (CRF desc, s desc, slot asc) order.  Entry j is pinned when its hit
    bit is unambiguous (|s_j - tau| > tol*tau) and its rank against b is decided by
    CRF by more than tol, or by s by more than tol at bit-equal CRF.
    Returns (number pinned, number of pinned mismatches)."""
    n = len(s_ora)
    assert keep_gpu.sum() == keep_ora.sum()
    if n == 0 or keep_ora.sum() in (0, n):
        return n, int((keep_gpu != keep_ora).sum())
    s64 = s_ora.astype(np.float64)
    tau = s64[hit_ora].min() if hit_ora.any() else None
    order = np.lexsort((np.arange(n), -s64, -crf_ora.astype(np.float64)))
    b = order[int(keep_ora.sum()) - 1]
    cb, sb = float(crf_ora[b]), s64[b]
    c64 = crf_ora.astype(np.float64)
    unamb = np.ones(n, bool) if tau is None else np.abs(s64 - tau) > tol * tau
    by_crf = np.abs(c64 - cb) > tol * cb if cb > 0 else c64 > 0
    same_crf = (crf_ora.view(np.uint32) == np.float32(cb).view(np.uint32)) & \
               (crf_gpu.view(np.uint32) == crf_ora.view(np.uint32))
    by_s = same_crf & (np.abs(s64 - sb) > tol * sb)
    pinned = unamb & (by_crf | by_s)
    return int(pinned.sum()), int((keep_gpu[pinned] != keep_ora[pinned]).sum())


# ---------------------------------------------------------------------------
# full-size workloads: the whole cache on the GPU, sampled streams checked
# ---------------------------------------------------------------------------


def _stream_pages(lay, i):
    n, st = int(lay.length[i]), int(lay.start[i])
    npg = (st + n + 15) // 16
    return lay.block_table[i][:npg].astype(np.int64)


def kmeans_update_mismatches(x, a, c_prev, c_gpu, tiny=2.0 ** -25):
    """Centroids that break the k-means update's bar: bit-equal to the oracle's plain
    member mean of the GPU's assignments wherever no member coordinate is in (0, tiny),
    else within 2^-32 plus one fp32 spacing (the GPU sums on the 2^-32 grid)."""
    want = O.kmeans.update(x, a, c_prev)
    small = (np.abs(x) > 0) & (np.abs(x) < tiny)
    loose = np.zeros(want.shape, bool)
    for k in range(want.shape[0]):
        m = a == k
        if m.any():
            loose[k] = small[m].any(axis=0)
    bad = int(np.sum(c_gpu[~loose] != want[~loose]))
    tol = 2.0 ** -32 + np.spacing(np.abs(want[loose])).astype(np.float64)
    bad += int(np.sum(np.abs(c_gpu[loose].astype(np.float64) - want[loose].astype(np.float64)) > tol))
    return bad


def history_observers(w, lay, heads):
    """Observer sets (bf16 bits) of the history rounds 1..H: counter-based draws for the
    (layer, query head) pairs in `heads`, seeded PCG64 draws for the others."""
    from workloads.host import observers
    return [observers(w, lay, rnd=r, heads=heads, only_heads=True) for r in range(1, w.history_rounds + 1)]


def gpu_history(w, lay, d, cache, seqs, q_hist, exact_streams, scores, workspace, exact_lse=None):
    """The untimed history rounds on the device, in order: kvs_score with that round's
    observers (their LSE over the cache's keys), then kvs_lrfu_update with that round's
    dt; every live entry carries a prior.  exact_lse: {stream: [LSE rows of round r]}
    computed on the host beforehand (else recomputed here)."""
    import torch
    import kv_cache_eviction_lse_amd as K
    from workloads import device as DV
    from workloads.host import history_dt
    dev = _dev()
    dts = history_dt(w)
    n_prev = torch.from_numpy(lay.length.astype(np.int32)).to(dev)
    for r, qh in enumerate(q_hist):
        ex = {s: v[r] for s, v in exact_lse.items()} if exact_lse else None
        q_dev, lse_dev = DV.observer_lse(w, lay, d, qh, dev, exact_streams, ex)
        obs = K.ObserverSet(q_dev, lse_dev, lay.obs_off, device=dev)
        decay = torch.from_numpy(np.array([K.kvs_lrfu_decay(0.5, int(x)) for x in dts[r]], np.float32)).to(dev)
        K.kvs_score(cache, seqs, obs, w.scale, scores, workspace)
        K.kvs_lrfu_update(cache, seqs, scores, 9, 10, decay, n_prev, None)
        torch.cuda.synchronize()
        del obs, q_dev, lse_dev


def oracle_history(w, lay, q_host0, q_hist, stream, mini, tol=1e-3):
    """The oracle's replay of the history rounds of one stream on its host bytes (the
    mini-pools of host_stream_inputs).  Returns (crf_pool after the history,
    unambiguous [n], LSE rows of each round): an entry is unambiguous when its score was
    more than tol away from the cut threshold in every history round, so its hit bits,
    and hence its CRF, do not depend on score rounding."""
    from workloads import device as DV
    from workloads.host import history_dt
    k, v, c, qq, lse, bt, stt, ln, oo = mini
    c = c.copy()
    dts = history_dt(w)
    i = stream[0]
    n = int(ln[0])
    unamb = np.ones(n, bool)
    page, row = O.slot_location(bt[0], stt[0], np.arange(n))
    lse_rows = []
    for r, qh in enumerate(q_hist):
        q_r, lse_r = DV.host_stream_observers(w, lay, q_host0, qh, [stream])
        lse_rows.append(np.concatenate([lse_r[0, hh] for hh in range(w.group)]))
        s = O.score(k, q_r, lse_r, oo, bt, stt, ln, w.group, w.scale)[(0, 0, 0)]
        hit = O.mass_cut(s)
        if hit.any():
            tau = float(s[hit].min())
            unamb &= np.abs(s.astype(np.float64) - tau) > tol * tau
        c[0, page, 0, row] = O.lrfu_update(c[0, page, 0, row], hit, O.lrfu_decay(0.5, int(dts[r][i])), n)
    return c, unamb, lse_rows


def run_config_sampled(w, lay, q_host, sample, scale=None, fused=False):
    """One round of workload w over its whole cache on the GPU (device-drawn data, the
    sampled streams overwritten with host-generated bytes), stage by stage, after the
    workload's history rounds (if any); returns the GPU's intermediates for the sampled
    streams only."""
    import torch
    import kv_cache_eviction_lse_amd as K
    from workloads import device as DV
    dev = _dev()
    d = DV.fill(w, lay, q_host, dev, exact_streams=sample)
    torch.cuda.synchronize()
    L, Hkv = w.num_layers, w.num_kv_heads
    cache = K.PagedCache(d.k, d.v, d.crf)
    seqs = K.SeqBatch(lay.block_table, lay.start, lay.length, device=dev)
    obs = K.ObserverSet(d.q, d.lse, lay.obs_off, device=dev)
    budget_h = np.full(w.num_seqs, w.budget, np.int32)
    bufs = K.RoundBuffers(cache, seqs, obs, budget_h, keep_hits=True)
    if w.history_rounds:
        heads = {(l, h) for (_, l, g) in sample for h in range(g * w.group, (g + 1) * w.group)}
        gpu_history(w, lay, d, cache, seqs, history_observers(w, lay, heads), sample, bufs.scores,
                    bufs.workspace)
    decay_h = np.array([K.kvs_lrfu_decay(0.5, int(x)) for x in lay.dt], np.float32)
    decay = torch.from_numpy(decay_h).to(dev)
    n_prev = torch.from_numpy(lay.n_prev.astype(np.int32)).to(dev)
    scale = w.scale if scale is None else scale
    pages = {s: torch.from_numpy(_stream_pages(lay, s[0])).to(dev) for s in sample}
    rec = {s: {} for s in sample}

    def grab(tag, fn):
        torch.cuda.synchronize()
        for s in sample:
            rec[s][tag] = fn(s)

    def ent(buf, s):
        i, l, g = s
        return buf[l, g, int(lay.entry_off[i]):int(lay.entry_off[i + 1])].cpu().numpy()

    def crf_pages(s):
        i, l, g = s
        return d.crf[l][pages[s], g].cpu().numpy()          # [npg][16]

    def kv_pages(s):
        i, l, g = s
        return (d.k[l][pages[s], g].cpu().numpy().view(np.uint16),
                d.v[l][pages[s], g].cpu().numpy().view(np.uint16))

    grab("crf0", crf_pages)
    K.kvs_score(cache, seqs, obs, scale, bufs.scores, bufs.workspace)
    grab("s", lambda s: ent(bufs.scores, s))
    if fused:
        K.kvs_lrfu_select(cache, seqs, bufs.scores, 9, 10, decay, n_prev, bufs.budget, bufs.budget_h,
                          bufs.keep, hit=bufs.hit)
    else:
        K.kvs_lrfu_update(cache, seqs, bufs.scores, 9, 10, decay, n_prev, bufs.hit)
    grab("hit", lambda s: ent(bufs.hit, s).astype(bool))
    grab("crf1", crf_pages)
    if not fused:
        K.kvs_select(cache, seqs, bufs.scores, bufs.budget, bufs.budget_h, bufs.keep)
    grab("keep", lambda s: ent(bufs.keep, s).astype(bool))
    grab("kv0", kv_pages)
    if fused:
        plan = K.kvs_plan_compact(cache, seqs, bufs.keep, bufs.budget, bufs.budget_h, bufs.pairs, bufs.pair_count)
    else:
        plan = K.kvs_plan(seqs, L, Hkv, bufs.keep, bufs.budget, bufs.budget_h, bufs.pairs, bufs.pair_count)
    grab("pairs", lambda s: bufs.pairs[s[1], s[2], s[0], :max(int(bufs.pair_count[s[1], s[2], s[0]]), 0)]
         .cpu().numpy())
    if not fused:
        K.kvs_compact(cache, seqs, bufs.budget_h, bufs.pairs, bufs.pair_count)
    grab("kv1", kv_pages)
    grab("crf2", crf_pages)
    torch.cuda.synchronize()
    out = {"rec": rec, "plan": plan, "decay": decay_h}
    del bufs, cache, d
    torch.cuda.empty_cache()
    return out


def check_config_sampled(w, lay, q_host, sample, out, score_rtol=1e-3):
    """Sampled-stream parity of a full-size round: scores against the oracle on the same
    bytes; cut, LRFU, keep set, pairs and moved bytes exact on the GPU's own inputs; the
    end-to-end keep set exact wherever the oracle's margins pin it.  Returns
    (worst relative score error, pinned entries, pinned mismatches)."""
    from workloads.device import host_stream_inputs
    G = w.group
    worst, pinned_all, bad_all = 0.0, 0, 0
    if w.history_rounds:
        heads = {(l, h) for (_, l, g) in sample for h in range(g * w.group, (g + 1) * w.group)}
        q_hist = history_observers(w, lay, heads)
    for s in sample:
        i, l, g = s
        n, st = int(lay.length[i]), int(lay.start[i])
        B = int(w.budget)
        mini = host_stream_inputs(w, lay, q_host, [s])
        k, v, c, qq, lse, bt, stt, ln, oo = mini
        if w.history_rounds:
            # the history: the GPU's CRF before the measured round equals the oracle's
            # replay wherever no history round's cut was within the score tolerance;
            # the measured round then starts from the GPU's state (teacher forcing)
            c_hist, unamb, _ = oracle_history(w, lay, q_host, q_hist, s, mini)
            pos = st + np.arange(n)
            gpu0 = out["rec"][s]["crf0"][pos // 16, pos % 16]
            ora0 = c_hist[0, pos // 16, 0, pos % 16]
            hist_bad = int(np.sum(gpu0[unamb].view(np.uint32) != ora0[unamb].view(np.uint32)))
            print(f"history {s}: {int(unamb.sum())} of {n} entries unambiguous in every round, "
                  f"{hist_bad} CRF mismatches", flush=True)
            assert hist_bad == 0 and unamb.sum() > n // 2, (s, hist_bad)
            c = c.copy()
            c[0, pos // 16, 0, pos % 16] = gpu0
        res = O.eviction_round(k.copy(), v.copy(), c.copy(), qq, lse, oo, bt, stt, ln, G, w.scale, 0.5,
                               np.array([lay.dt[i]]), np.array([lay.n_prev[i]]), np.array([B]))
        plan3 = (out["plan"].shift[i], out["plan"].new_start[i], out["plan"].new_len[i])
        w_, pn, nb = check_stream_record(res, out["rec"][s], n, st, B, out["decay"][i], int(lay.n_prev[i]),
                                         plan3, lay.block_table[i], score_rtol, s)
        worst = max(worst, w_)
        pinned_all += pn
        bad_all += nb
    return worst, pinned_all, bad_all


def check_stream_record(res, r, n, st, B, decay, n_prev, plan3, bt_row, score_rtol=1e-3, tag=None):
    """One stream's GPU record r (scores, hit, keep, pairs; crf0/crf1/crf2 and kv0/kv1 as
    the stream's pages) against the oracle round res on the same input bytes: scores
    within score_rtol, every later stage exact on the GPU's own inputs, the keep set
    exact where pinned.  Returns (worst relative score error, pinned, mismatches)."""
    s_ora = res["s"][(0, 0, 0)]
    s_gpu = r["s"]
    worst = 0.0
    nz = s_ora > 0
    err = np.abs(s_gpu.astype(np.float64) - s_ora) / np.maximum(np.abs(s_ora.astype(np.float64)), 1e-30)
    if nz.any():
        worst = float(err[nz].max())
        assert worst <= score_rtol, (tag, worst)
    # components on the GPU's own inputs
    pos = st + np.arange(n)
    pi, row = pos // 16, pos % 16
    hit = O.mass_cut(s_gpu)
    np.testing.assert_array_equal(r["hit"], hit, err_msg=f"hit {tag}")
    prior = r["crf0"][pi, row]
    crf_new = O.lrfu_update(prior, hit, np.float32(decay), int(n_prev))
    got = r["crf1"][pi, row]
    np.testing.assert_array_equal(got.view(np.uint32), crf_new.view(np.uint32), err_msg=f"crf {tag}")
    keep = O.select_top_b(got, s_gpu, B)
    np.testing.assert_array_equal(r["keep"], keep, err_msg=f"keep {tag}")
    src, dst = O.plan_stream(r["keep"])
    assert len(r["pairs"]) == len(src), (tag, len(r["pairs"]), len(src))
    if len(src):
        np.testing.assert_array_equal(r["pairs"][:, 0], src)
        np.testing.assert_array_equal(r["pairs"][:, 1], dst)
    # moved bytes: the stream's pages after = before with the pairs applied
    k0, v0 = r["kv0"]
    c0 = r["crf1"].copy()
    ek, ev, ec = k0.copy(), v0.copy(), c0.copy()
    sp, sr = (st + src) // 16, (st + src) % 16
    dp, dr = (st + dst) // 16, (st + dst) % 16
    ek[dp, dr] = k0[sp, sr]
    ev[dp, dr] = v0[sp, sr]
    ec[dp, dr] = c0[sp, sr]
    np.testing.assert_array_equal(r["kv1"][0], ek, err_msg=f"K bytes {tag}")
    np.testing.assert_array_equal(r["kv1"][1], ev, err_msg=f"V bytes {tag}")
    np.testing.assert_array_equal(r["crf2"].view(np.uint32), ec.view(np.uint32), err_msg=f"CRF {tag}")
    # host plan outputs
    sh, ns, nl, _ = O.plan_sequence(n, min(B, n), st, bt_row)
    assert tuple(int(x) for x in plan3) == (sh, ns, nl), (tag, plan3, (sh, ns, nl))
    # end to end against the oracle's own round
    pn, nb = pinned_keep_check(s_ora, res["crf"][(0, 0, 0)], res["keep"][(0, 0, 0)], res["hit"][(0, 0, 0)],
                               s_gpu, got, r["keep"])
    return worst, pn, nb
