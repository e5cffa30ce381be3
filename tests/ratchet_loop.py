"""The ratchet-loop workload driver shared by its GPU test and `bench.py --workload
ratchet` (test and benchmark plumbing: it only calls the library and draws inputs).

One Llama-3-8B-shaped sequence (32 layers x 8 KV heads x 32 query heads) is prefilled
with 8 192 tokens; each round appends 64 tokens (the round's decode steps), draws 32
fresh observers per query head with their LSE over the live entries (what the decode
kernel would hand over), takes the budget flag, and runs one eviction round with
dt = 64.  Freed pages go back to a host free list; appended tokens take pages from it.

Flags: "bernoulli" is the configuration's seeded Bernoulli(0.05) per round.
"confidence" closes ActKV's loop (Component 2): the round's 64 decode steps have
synthetic logits over the Llama-3 vocabulary whose sharpness follows a trajectory
(slow drift, noise and short collapses: hesitation); kvs_token_confidence gives each
step's confidence, kvs_confidence_trend min-pools the trajectory so far (window 64,
stride 8) and fits a line over the last FIT_LAST pooled values, and a negative slope
is the flag for kvs_budget_ratchet.
"""
from __future__ import annotations

import numpy as np

from workloads import RATCHET, philox
from workloads.configs import TAG_FLAG
from workloads.host import make_layout, observers

OBS = 32
APPEND = 64
CHECK_STREAMS = [(0, 0, 0), (0, 31, 7)]
FIT_LAST = 16          # pooled windows in the fitted line: the last 64 + 15 * 8 = 184 steps
CONF_K = 20


def trajectory_boost(rounds: int, seed: int = 31) -> np.ndarray:
    """Per-step sharpness of the whole decode trajectory (rounds x 64 steps): 12 +
    N(0, 0.8^2) noise rising by 4 over the trajectory, with a 16-step collapse to 1
    every 40 rounds (the agent hesitates)."""
    from workloads import logits as LG
    steps = rounds * APPEND
    return LG.trajectory_boost(seed, steps, 4.0, collapses=tuple(range(20 * APPEND, steps, 40 * APPEND)))


def boosted_rows_device(seed: int, boost: np.ndarray, vocab: int, device, dtype):
    """Logit rows on the device with the lm_rows recipe and a given per-row boost."""
    import torch
    rows = boost.shape[0]
    g = torch.Generator(device=device).manual_seed(seed)
    z = torch.randn((rows, vocab), generator=g, device=device, dtype=torch.float32).mul_(1.5).sub_(6.0)
    pos = torch.randint(0, vocab, (rows, 8), generator=g, device=device)
    val = torch.rand((rows, 8), generator=g, device=device) * 2.0 - 1.0
    val[:, 0] = torch.from_numpy(boost.astype(np.float32)).to(device)
    z.scatter_(1, pos, val)
    return z.to(dtype)


class RatchetLoop:
    def __init__(self, dev, flags: str = "bernoulli", rounds: int | None = None):
        import torch
        import kv_cache_eviction_lse_amd as K
        from workloads import device as DV
        self.K, self.torch, self.dev = K, torch, dev
        w = self.w = RATCHET
        self.R = w.rounds if rounds is None else rounds
        self.L, self.Hkv, self.Hq, self.G, self.D = w.num_layers, w.num_kv_heads, w.num_q_heads, w.group, w.head_dim
        lay = make_layout(w)
        q0 = observers(w, lay, only_heads=True, heads=set())
        self.d = DV.fill(w, lay, q0, dev)
        self.gen = torch.Generator(device=dev)
        self.gen.manual_seed(w.key & 0x7FFFFFFFFFFFFFFF ^ 0x5A5A)
        self.n = int(lay.length[0])
        self.start = int(lay.start[0])
        npg0 = (self.start + self.n + 15) // 16
        self.pages = [int(p) for p in lay.block_table[0][:npg0]]
        used = set(self.pages)
        self.free = [p for p in range(lay.num_pages) if p not in used]
        self.n_prev = 0                       # the prefill has no LRFU state
        self.budget = int(w.budget)
        self.flag_mode = flags
        self.bern = philox.uniform01(philox.words(w.key, TAG_FLAG, np.arange(w.rounds, dtype=np.uint64))[0]) \
            < w.flag_prob
        self.boost = trajectory_boost(self.R) if flags == "confidence" else None
        self.conf_hist = np.zeros(0, np.float32)
        self.decay_h = np.array([K.kvs_lrfu_decay(0.5, APPEND)], np.float32)
        self.decay = torch.from_numpy(self.decay_h).to(dev)
        self.cache = K.PagedCache(self.d.k, self.d.v, self.d.crf)
        from workloads import logits as LG
        self.vocab = LG.LLAMA3_VOCAB
        self.conf_ws = None

    def prepare(self, r: int):
        """Append the round's tokens and draw its observers and their LSE; returns
        (q, lse) on the device."""
        q = self.append(r)
        lse = self.torch.empty((self.L, self.Hq, OBS), dtype=self.torch.float32, device=self.dev)
        self.observer_lse(q, lse)
        return q, lse

    def append(self, r: int):
        """Append the round's 64 tokens (K with planted keys aligned to the round's
        observers, V) and draw the observers; returns q (bf16 [L][Hq][OBS][D], device)."""
        torch, dev, d = self.torch, self.dev, self.d
        L, Hkv, Hq, G, D = self.L, self.Hkv, self.Hq, self.G, self.D
        q = torch.randn((L, Hq, OBS, D), generator=self.gen, device=dev).to(torch.bfloat16)
        qf = q.float()
        pos = self.start + self.n + np.arange(APPEND)
        while len(self.pages) < (pos[-1] // 16) + 1:
            self.pages.append(self.free.pop(0))
        pg = torch.from_numpy(np.asarray(self.pages, np.int64)[pos // 16]).to(dev)
        rw = torch.from_numpy(pos % 16).to(dev)
        for l in range(L):
            z = torch.randn((APPEND, Hkv, D), generator=self.gen, device=dev)
            qr = qf[l].reshape(Hkv, G * OBS, D)
            qn = qr / qr.norm(dim=2, keepdim=True)
            pm = torch.rand((APPEND, Hkv), generator=self.gen, device=dev) < self.w.planted_frac
            rr = torch.randint(0, G * OBS, (APPEND, Hkv), generator=self.gen, device=dev)
            gi = torch.arange(Hkv, device=dev)[None, :].expand(APPEND, Hkv)
            z = torch.where(pm[:, :, None], 3.0 * qn[gi, rr] + z, z)
            d.k[l][pg, :, rw, :] = z.to(torch.bfloat16).view(torch.int16)
            d.v[l][pg, :, rw, :] = torch.randn((APPEND, Hkv, D), generator=self.gen, device=dev) \
                .to(torch.bfloat16).view(torch.int16)
        self.n_prev = self.n
        self.n += APPEND
        return q

    def observer_lse(self, q, lse) -> None:
        """The observers' LSE over the live entries into lse (fp32 [L][Hq][OBS], device):
        what the decode kernel hands over.  Its host-to-device copies come first, so
        after they return the rest is device work enqueued on the current stream."""
        torch, dev, d = self.torch, self.dev, self.d
        from workloads import device as DV
        L, Hkv, Hq, G, D = self.L, self.Hkv, self.Hq, self.G, self.D
        qf = q.float()
        live = self.start + np.arange(self.n)
        lpg = torch.from_numpy(np.asarray(self.pages, np.int64)[live // 16]).to(dev)
        lrw = torch.from_numpy(live % 16).to(dev)
        for l in range(L):
            keys = d.k[l][lpg, :, lrw, :].view(torch.bfloat16).float()
            lse[l] = DV.live_lse(keys, qf[l].reshape(Hkv, G * OBS, D), self.w.scale).reshape(Hq, OBS)

    def step_logits(self, r: int):
        """The round's 64 decode steps' logits (bf16, device)."""
        b = self.boost[(r - 1) * APPEND:r * APPEND]
        return boosted_rows_device(1000 + r, b, self.vocab, self.dev, self.torch.bfloat16)

    def flag(self, r: int, logits=None, conf=None):
        """The round's budget flag.  With confidence flags, `logits` are the round's
        decode-step rows and `conf` a device float32 [64] buffer: the library computes
        the confidences, the trend over the trajectory so far, and its flag."""
        if self.flag_mode == "bernoulli":
            return bool(self.bern[r - 1])
        K, torch = self.K, self.torch
        if self.conf_ws is None:
            need = K.kvs_token_confidence_workspace_size(APPEND, self.vocab, CONF_K)
            self.conf_ws = torch.empty(max(need, 4), dtype=torch.uint8, device=self.dev)
        K.kvs_token_confidence(logits, conf, k=CONF_K, workspace=self.conf_ws)
        self.conf_hist = np.concatenate([self.conf_hist, conf.cpu().numpy()])   # waits for the kernel
        return K.kvs_confidence_trend(self.conf_hist, 64, 8, FIT_LAST).flag

    def batch(self):
        """(seqs, budget_h) of the current round."""
        K = self.K
        bt = np.asarray(self.pages, np.int32)[None, :]
        seqs = K.SeqBatch(bt, np.array([self.start], np.int32), np.array([self.n], np.int32), device=self.dev)
        return seqs, np.array([self.budget], np.int32)

    def ratchet(self, flag: bool) -> int:
        self.budget = int(self.K.kvs_budget_ratchet(np.array([self.budget], np.int32),
                                                    np.array([flag], np.int32))[0])
        return self.budget

    def finish(self, plan) -> None:
        """The host side of the plan: the pages at the front are freed."""
        shift = int(plan.shift[0])
        assert list(plan.freed) == self.pages[:shift]
        self.free.extend(self.pages[:shift])
        self.pages = self.pages[shift:]
        self.start, self.n = int(plan.new_start[0]), int(plan.new_len[0])


def checked_round(lp, r, q, lse, seqs, bufs):
    """Run round r stage by stage and compare the sampled streams with the oracle's
    round from the same pre-round state.  Returns (plan, worst score error, pinned,
    oracle seconds, oracle entries)."""
    import time
    import torch
    import oracle as O
    from tests import gpu_util as U
    K, d, L, Hkv, G = lp.K, lp.d, lp.L, lp.Hkv, lp.G
    n, start, budget, n_prev = lp.n, lp.start, lp.budget, lp.n_prev
    n_prev_t = torch.tensor([n_prev], dtype=torch.int32, device=lp.dev)
    pt = torch.from_numpy(np.asarray(lp.pages, np.int64)).to(lp.dev)
    pre = {}
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
    cache = lp.cache
    obs = K.ObserverSet(q.view(torch.int16), lse, np.array([0, OBS], np.int64), device=lp.dev)
    K.kvs_score(cache, seqs, obs, lp.w.scale, bufs.scores, bufs.workspace)
    grab("s", lambda s: bufs.scores[s[1], s[2], :n].cpu().numpy())
    K.kvs_lrfu_update(cache, seqs, bufs.scores, 9, 10, lp.decay, n_prev_t, bufs.hit)
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
    npg = len(lp.pages)
    worst, pinned, t_ora = 0.0, 0, 0.0
    for s in CHECK_STREAMS:
        p_ = pre[s]
        t0 = time.perf_counter()
        res = O.eviction_round(p_["k"][None, :, None].copy(), p_["v"][None, :, None].copy(),
                               p_["crf"][None, :, None].copy(), p_["q"][None], p_["lse"][None],
                               np.array([0, OBS], np.int64), np.arange(npg, dtype=np.int32)[None, :],
                               np.array([start]), np.array([n]), G, lp.w.scale, 0.5, np.array([APPEND]),
                               np.array([n_prev]), np.array([budget]))
        t_ora += time.perf_counter() - t0
        plan3 = (plan.shift[0], plan.new_start[0], plan.new_len[0])
        w_, pn, bad = U.check_stream_record(res, rec[s], n, start, budget, lp.decay_h[0], n_prev, plan3,
                                            np.arange(npg), 1e-3, (r, s))
        assert bad == 0, (r, s, bad)
        worst = max(worst, w_)
        pinned += pn
    return plan, worst, pinned, t_ora, n * len(CHECK_STREAMS)
