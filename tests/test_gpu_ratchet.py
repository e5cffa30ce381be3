"""The ratchet loop on the GPU, checked round by round with teacher forcing.

One Llama-3-8B-shaped sequence (32 layers x 8 KV heads x 32 query heads) is prefilled
with 8 192 tokens; each of 387 rounds appends 64 tokens, draws 32 fresh observers per
query head with their LSE over the live entries, takes the budget flag (x7/4 capped at
30 000, never shrinking), and runs a full eviction round with dt = 64 (driver:
tests/ratchet_loop.py).  On the checked rounds the oracle's input is the GPU state just
before the round (the sampled streams' pages, CRF, observers and LSE), so one boundary
decision cannot cascade into later rounds.

The configuration's flag is a seeded Bernoulli(0.05).  The closed loop (ActKV
Dissected, Component 2) takes it from the model's hesitation instead: each round's 64
decode steps have synthetic logits, kvs_token_confidence scores them, the host trend
over the trajectory so far gives the flag.  There every round's confidences are checked
against the oracle on the same bf16 bytes, the flag against the oracle's trend of the
GPU's confidences, the budget against the oracle's ratchet, and sampled rounds by
teacher forcing as above.
"""
import numpy as np
import pytest

import oracle as O
from tests.ratchet_loop import APPEND, CONF_K, FIT_LAST, OBS, RatchetLoop, checked_round

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_ratchet_loop_teacher_forced():
    import torch
    import kv_cache_eviction_lse_amd as K
    lp = RatchetLoop(torch.device("cuda", 0), flags="bernoulli")
    R = lp.R
    flag_rounds = [r + 1 for r in np.flatnonzero(lp.bern)[:3]]
    check = sorted({1, 2, 3, R} | set(range(40, R, 40)) | set(flag_rounds))
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_ms, entries_timed, checked, pinned_total, worst = 0.0, 0, 0, 0, 0.0
    max_budget = lp.budget
    for r in range(1, R + 1):
        q, lse = lp.prepare(r)
        old = lp.budget
        nb = lp.ratchet(lp.flag(r))
        assert nb == O.ratchet(old, bool(lp.bern[r - 1])), (r, old, nb)
        max_budget = max(max_budget, nb)
        seqs, budget_h = lp.batch()
        obs = K.ObserverSet(q.view(torch.int16), lse, np.array([0, OBS], np.int64), device=lp.dev)
        bufs = K.RoundBuffers(lp.cache, seqs, obs, budget_h, keep_hits=True)
        n_prev = lp.n_prev
        if r in check:
            plan, w_, pn, _, _ = checked_round(lp, r, q, lse, seqs, bufs)
            worst, pinned_total, checked = max(worst, w_), pinned_total + pn, checked + 1
        else:
            n_prev_t = torch.tensor([n_prev], dtype=torch.int32, device=lp.dev)
            ev0.record()
            plan = K.eviction_round(lp.cache, seqs, obs, bufs, lp.decay, n_prev_t, lp.w.scale)
            ev1.record()
            torch.cuda.synchronize()
            t_ms += ev0.elapsed_time(ev1)
            entries_timed += lp.n * lp.L * lp.Hkv
        lp.finish(plan)
        assert lp.n == min(nb, n_prev + APPEND)
        if r % 50 == 0:
            print(f"round {r}: budget {lp.budget}, live {lp.n}, pages {len(lp.pages)}", flush=True)
    print(f"ratchet: {R} rounds, {checked} checked (max rel score err {worst:.2e}, {pinned_total} keep bits "
          f"pinned), final budget {lp.budget} (max {max_budget}); amortised {entries_timed / (t_ms / 1e3):.3e} "
          f"entries/s over {R - checked} timed rounds", flush=True)
    assert lp.budget == max_budget


# confidence bound of the monitor's kernel against the fp64 oracle (derived in
# tests/test_gpu_confidence.py for logits below 100 in magnitude)
def _conf_tol(ref):
    return 5e-5 + 1e-6 * np.abs(ref)


@pytest.mark.timeout(900)
def test_ratchet_closed_loop_confidence():
    import torch
    import kv_cache_eviction_lse_amd as K
    from workloads import logits as LG
    R = 100
    lp = RatchetLoop(torch.device("cuda", 0), flags="confidence", rounds=R)
    conf = torch.empty(APPEND, dtype=torch.float32, device=lp.dev)
    budget, flags_seen, checked = lp.budget, 0, 0
    check = {1, 21, 22, 61, 62, R}
    for r in range(1, R + 1):
        q, lse = lp.prepare(r)
        x = lp.step_logits(r)
        f = lp.flag(r, x, conf)
        # this round's confidences against the oracle on the same bf16 bytes
        got = lp.conf_hist[-APPEND:].astype(np.float64)
        bits = x.view(torch.int16).cpu().numpy().view(np.uint16)
        z = LG.bf16_bits_to_f64(bits)
        for row in range(0, APPEND, 8 if r not in check else 1):
            ref = O.confidence.token_confidence(z[row], CONF_K)
            assert abs(got[row] - ref) <= _conf_tol(ref), (r, row, got[row], ref)
        # the flag: the oracle's trend of the GPU's confidences (same fp32 inputs)
        slope, _, want = O.confidence.trend_flag(lp.conf_hist, 64, 8, FIT_LAST)
        if slope is None or abs(slope) > 1e-9:
            assert f == want, (r, slope)
        flags_seen += int(f)
        nb = lp.ratchet(f)
        assert nb == O.ratchet(budget, f), (r, budget, nb)
        budget = nb
        seqs, budget_h = lp.batch()
        obs = K.ObserverSet(q.view(torch.int16), lse, np.array([0, OBS], np.int64), device=lp.dev)
        bufs = K.RoundBuffers(lp.cache, seqs, obs, budget_h, keep_hits=True)
        n_prev = lp.n_prev
        if r in check:
            plan = checked_round(lp, r, q, lse, seqs, bufs)[0]
            checked += 1
        else:
            n_prev_t = torch.tensor([n_prev], dtype=torch.int32, device=lp.dev)
            plan = K.eviction_round(lp.cache, seqs, obs, bufs, lp.decay, n_prev_t, lp.w.scale)
        lp.finish(plan)
        assert lp.n == min(budget, n_prev + APPEND)
    print(f"closed loop: {R} rounds, {flags_seen} flags from the confidence trend, final budget {budget}, "
          f"{checked} rounds teacher-forced", flush=True)
    assert flags_seen > 0 and budget > 512
