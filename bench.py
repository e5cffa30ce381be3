#!/usr/bin/env python3
"""Throughput of one attention-guided eviction round on one MI355X.

A step is one full round over the Llama-3-8B-shaped cache (32 layers x 8 KV heads,
32 query heads, 32,768 live entries per stream in 16-token pages scattered over a
4,096-page pool, 64 observers per sequence, budget 512):

    kvs_score -> kvs_lrfu_select_compact
    (with --separate: kvs_score -> kvs_lrfu_update -> kvs_select -> kvs_plan -> kvs_compact)

all enqueued on one stream with inputs resident in HBM.  Every step re-runs the
round on the same 32K-entry layout (the evicted slots stand for freshly appended
tokens), so the work per step is constant.  Prints one JSON line.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

`--workload decode_llama3_8b_32k` times paged decode attention with the LSE and the
attention tally (one decode token over the 8B-shaped cache), and `--workload
token_confidence` times the confidence monitor that drives the
budget ratchet: kvs_token_confidence over one round's decode steps (64 sequences x
64 steps = 4 096 rows of bf16 logits over the Llama-3 vocabulary, 128 256 tokens),
and prints its own JSON line.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import platform
import sys
import time

import numpy as np
from threadpoolctl import threadpool_limits

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV entries scored+compacted/sec; achieved HBM GB/s vs peak (8B shape, 32K ctx)"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
D = 128


# ---------------------------------------------------------------------------
# the oracle leg of the round benchmark: host bytes of sampled streams, the oracle's
# replay of the workload's LRFU history, then the oracle's measured round timed over a
# process pool (one BLAS thread per worker); all of it before the GPU is touched
# ---------------------------------------------------------------------------

_ORACLE_INPUTS: list = []


def _prepare_stream(args):
    """Host bytes of one sampled stream (mini-pools) and, for a workload with history
    rounds, the oracle's replay of that history."""
    from threadpoolctl import threadpool_limits
    from workloads import ALL
    from workloads.device import host_stream_inputs
    from workloads.host import make_layout, observers
    from tests.gpu_util import oracle_history
    wname, (i, l, g) = args
    w = ALL[wname]
    lay = make_layout(w)
    G = w.num_q_heads // w.num_kv_heads
    heads = {(l, h) for h in range(g * G, (g + 1) * G)}
    with threadpool_limits(1):
        q0 = observers(w, lay, heads=heads, only_heads=True, rest_zero=True)
        mini = host_stream_inputs(w, lay, q0, [(i, l, g)])
        hist = None
        if w.history_rounds:
            qh = [observers(w, lay, rnd=r, heads=heads, only_heads=True, rest_zero=True)
                  for r in range(1, w.history_rounds + 1)]
            hist = oracle_history(w, lay, q0, qh, (i, l, g), mini)
    return mini, hist


def _oracle_round(idx):
    """The oracle's measured round (score, cut, LRFU, keep set, plan, moves) on sampled
    stream idx, from its own post-history state, on one BLAS thread; timed."""
    import oracle as O
    G, scale, dt, n_prev, budget, mini, hist = _ORACLE_INPUTS[idx]
    k, v, c, qq, lse, bt, stt, ln, oo = mini
    c0 = hist[0] if hist is not None else c
    with threadpool_limits(1):
        t = time.perf_counter()
        res = O.eviction_round(k.copy(), v.copy(), c0.copy(), qq, lse, oo, bt, stt, ln, G, scale, 0.5,
                               np.array([dt]), np.array([n_prev]), np.array([budget]))
        t = time.perf_counter() - t
    return {"s": res["s"][(0, 0, 0)], "hit": res["hit"][(0, 0, 0)], "t": t}


def oracle_leg(w, lay, sample, workers, min_cpu_s):
    """Prepare the sampled streams, then time the oracle's round over them with a pool of
    `workers` processes (fork, before any GPU work), in passes over the sample until the
    processes have spent min_cpu_s in the oracle.  Returns the first pass's per-stream
    results and the totals of the timed passes."""
    import multiprocessing as mp
    global _ORACLE_INPUTS
    ctx = mp.get_context("fork")
    nw = max(1, min(workers, len(sample)))
    t0 = time.perf_counter()
    with cf.ProcessPoolExecutor(max_workers=nw, mp_context=ctx) as ex:
        prep = list(ex.map(_prepare_stream, [(w.name, s) for s in sample]))
    t_prep = time.perf_counter() - t0
    G = w.num_q_heads // w.num_kv_heads
    _ORACLE_INPUTS = [(G, w.scale, int(lay.dt[i]), int(lay.n_prev[i]), int(w.budget), mini, hist)
                      for (i, _, _), (mini, hist) in zip(sample, prep)]
    rounds, wall, cpu_s, passes = None, 0.0, 0.0, 0
    with cf.ProcessPoolExecutor(max_workers=nw, mp_context=ctx) as ex:
        while passes == 0 or (cpu_s < min_cpu_s and passes < 20):
            t0 = time.perf_counter()
            res = list(ex.map(_oracle_round, range(len(sample))))
            wall += time.perf_counter() - t0
            cpu_s += sum(r["t"] for r in res)
            passes += 1
            rounds = rounds or res
    return {"hist": [h for (_, h) in prep], "minis": [m for (m, _) in prep], "rounds": rounds, "wall": wall,
            "cpu_s": cpu_s, "passes": passes, "workers": nw, "prep_s": t_prep}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def copy_peak_gbps(dev, mib: int = 1024, reps: int = 10) -> float:
    """A measured HBM reference: a plain device-to-device copy of `mib` MiB, timed with HIP
    events over `reps` copies (bytes read plus bytes written per second)."""
    import torch
    src = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    gbps = 2.0 * (mib << 20) * reps / (t0.elapsed_time(t1) / 1000.0) / 1e9
    del src, dst
    return gbps


def score_kernels(w, lay) -> str:
    """The kvs_score kernels this workload launches (by the rows R = O G of its sequences)."""
    G = w.num_q_heads // w.num_kv_heads
    names = set()
    for O in lay.obs.tolist():
        R = O * G
        if R < 16:
            names.add("score_valu_kernel")
        elif R <= 128:
            names.add("score_mfma_kernel")
        else:
            names.add("score_pipe_kernel<4>" if R <= 256 else "score_pipe_kernel<8>")
    return " + ".join(sorted(names))


def load_traffic(workload, name="score", source="score.hip"):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter summary
    profiles/<name>_<workload>_traffic.json, if it was taken on the current source of
    that kernel; else None."""
    from kv_cache_eviction_lse_amd.profiling import source_sha
    p = os.path.join(ROOT, "profiles", f"{name}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    t = json.load(open(p))
    if t.get("source_sha", t.get("score_source_sha")) != source_sha(source):
        return None
    return float(t["hbm_bytes_per_launch"])


CONF_METRIC = ("decode-step logit rows scored (top-20 mean NLL confidence)/sec; achieved HBM GB/s vs peak "
               "(Llama-3 vocabulary)")


def bench_confidence(args) -> None:
    """kvs_token_confidence over 4 096 rows x 128 256 bf16 logits (one JSON line)."""
    import torch
    import kv_cache_eviction_lse_amd as K
    from workloads import logits as LG
    import oracle as O

    rows, V, k = 4096, LG.LLAMA3_VOCAB, 20
    dev = torch.device("cuda", 0)
    x = LG.lm_rows_device(7, rows, V, dev, torch.bfloat16)
    conf = torch.empty(rows, dtype=torch.float32, device=dev)
    ws = torch.empty(max(K.kvs_token_confidence_workspace_size(rows, V, k), 4), dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream()
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(20):
            K.kvs_token_confidence(x, conf, k=k, workspace=ws)
        torch.cuda.synchronize()
    t_settle = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        K.kvs_token_confidence(x, conf, k=k, workspace=ws)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(st)
        K.kvs_token_confidence(x, conf, k=k, workspace=ws)
        e1.record(st)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    ev_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    byts = rows * V * 2 + rows * 4          # logits read once, one fp32 per row written
    gbps = byts / (ev_ms / 1000.0) / 1e9
    out = {
        "metric": CONF_METRIC, "value": rows / (ms / 1000.0), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "token_confidence", "rows": rows, "vocab": V, "k": k, "logits": "bf16",
                   "rows_are": "64 sequences x 64 decode steps"},
        "hbm_gbps": byts / (ms / 1000.0) / 1e9, "hbm_frac": byts / (ms / 1000.0) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"kernel": "conf_chunk_kernel (+ conf_merge_kernel)", "bound": "hbm", "achieved": gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": load_traffic("token_confidence", "conf_chunk", "confidence.hip"),
                     "ms": ev_ms, "bytes_per_launch": byts},
    }
    if not args.no_cpu_baseline:
        got = conf.cpu().numpy()
        pick = np.random.default_rng(0).permutation(rows)
        t_cpu, n_done, worst = 0.0, 0, 0.0
        for r in pick:
            bits = x[int(r)].view(torch.int16).cpu().numpy().view(np.uint16)
            z = LG.bf16_bits_to_f64(bits)
            ta = time.perf_counter()
            want = O.confidence.token_confidence(z, k)
            t_cpu += time.perf_counter() - ta
            n_done += 1
            worst = max(worst, abs(float(got[int(r)]) - want))
            if t_cpu >= args.cpu_seconds:
                break
        out["cpu_baseline"] = {"value": n_done / t_cpu, "unit": "rows/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n_done} of {rows} rows of the same batch, {t_cpu:.1f} s of fp64 "
                                         f"numpy oracle time (one thread)"}
        out["parity"] = {"rows": n_done, "max_abs_conf_err": worst}
    if args.calibration_copy:
        src = torch.empty(args.calibration_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    out["setup_s"] = {"settle_s": round(t_settle, 2)}
    print(json.dumps(out), flush=True)


DEC_METRIC = ("KV entries attended by paged decode attention with LSE and attention tally/sec; achieved HBM "
              "GB/s vs peak (8B shape, 32K ctx)")


def bench_decode(args) -> None:
    """kvs_decode_attention for one decode token over the 8B-shaped cache, with the
    attention tally into the scores (the token is an action token); one JSON line."""
    import torch
    import kv_cache_eviction_lse_amd as K
    from workloads import ALL
    from workloads.host import make_layout, observers
    from workloads import device as DV
    import oracle as O

    w = ALL["llama3_8b_32k"]
    lay = make_layout(w)
    L, Hkv, Hq = w.num_layers, w.num_kv_heads, w.num_q_heads
    dev = torch.device("cuda", 0)
    q_obs = observers(w, lay, heads=set(), only_heads=True)
    d = DV.fill(w, lay, q_obs, dev)
    T = 1                                                    # one decode token per sequence
    g = torch.Generator(device=dev).manual_seed(5)
    q = torch.randn((L, Hq, T * w.num_seqs, D), generator=g, device=dev).to(torch.bfloat16)
    tok_off = np.arange(w.num_seqs + 1, dtype=np.int64) * T
    cache = K.PagedCache(d.k, d.v, d.crf)
    seqs = K.SeqBatch(lay.block_table, lay.start, lay.length, device=dev)
    qs = K.DecodeQueries(q, tok_off, device=dev)
    out = torch.empty((L, Hq, T * w.num_seqs, D), dtype=torch.float32, device=dev)
    lse = torch.empty((L, Hq, T * w.num_seqs), dtype=torch.float32, device=dev)
    E = int(lay.entry_off[-1])
    scores = torch.zeros((L, Hkv, E), dtype=torch.float32, device=dev)
    ws = torch.empty(K.kvs_decode_workspace_size(cache, seqs, qs, True), dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream()
    run = lambda: K.kvs_decode_attention(cache, seqs, qs, w.scale, out, lse, scores, ws)  # noqa: E731
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(20):
            run()
        torch.cuda.synchronize()
    t_settle = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in evs:
        e0.record(st)
        run()
        e1.record(st)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    ev_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    entries = E * L * Hkv
    R = Hq // Hkv * T
    # K and V rows read once, the tally's logits written and read (4 B per row), scores
    # read and written, queries read and outputs written
    byts = entries * (2 * 2 * D + 2 * 4 * R + 8) + L * Hq * T * (2 * D + 4 * D + 4)
    gbps = byts / (ev_ms / 1000.0) / 1e9
    res = {
        "metric": DEC_METRIC, "value": entries / (ms / 1000.0), "unit": "entries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode_llama3_8b_32k", "layers": L, "kv_heads": Hkv, "q_heads": Hq,
                   "head_dim": D, "context": int(lay.length[0]), "decode_tokens": T, "tally": True,
                   "entries_per_step": entries},
        "hbm_gbps": byts / (ms / 1000.0) / 1e9, "hbm_frac": byts / (ms / 1000.0) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"kernel": "decode_split_kernel (+ combine, tally)", "bound": "hbm", "achieved": gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": load_traffic("decode_llama3_8b_32k", "decode_split", "decode.hip"),
                     "traffic_of": "decode_split_kernel",
                     "ms": ev_ms, "bytes_per_launch": byts},
    }
    if not args.no_cpu_baseline:
        # parity and the oracle's rate on sampled streams (one call, tally from zero)
        scores.zero_()
        run()
        torch.cuda.synchronize()
        o_gpu, l_gpu, s_gpu = out.cpu().numpy(), lse.cpu().numpy(), scores.cpu().numpy()
        rng = np.random.default_rng(0)
        t_cpu, n_done, worst_o, worst_t = 0.0, 0, 0.0, 0.0
        G = Hq // Hkv
        n = int(lay.length[0])
        pos = int(lay.start[0]) + np.arange(n)
        pg = torch.from_numpy(lay.block_table[0][pos // 16].astype(np.int64)).to(dev)
        rw = torch.from_numpy((pos % 16).astype(np.int64)).to(dev)
        # up to 16 distinct streams are gathered to the host once and checked against the
        # oracle; the oracle then runs over them in turn (one BLAS thread) until it has
        # spent --cpu-seconds
        host = []
        for (l, gg) in {(int(rng.integers(L)), int(rng.integers(Hkv))) for _ in range(16)}:
            # the pools hold bf16 bit patterns in int16 storage
            kk = d.k[l][pg, gg, rw].view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
            vv = d.v[l][pg, gg, rw].view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
            qq = q[l, gg * G:(gg + 1) * G, 0].float().cpu().numpy().astype(np.float64)
            host.append((l, gg, qq, kk, vv))
        with threadpool_limits(1):
            while t_cpu < args.cpu_seconds:
                for (l, gg, qq, kk, vv) in host:
                    ta = time.perf_counter()
                    o_ref, l_ref, p_ref = O.decode.attend_stream(qq, kk, vv, w.scale)
                    t_cpu += time.perf_counter() - ta
                    if n_done < len(host) * n:
                        worst_o = max(worst_o, float(np.max(np.abs(o_gpu[l, gg * G:(gg + 1) * G, 0] - o_ref))))
                        tref = p_ref.sum(0)
                        worst_t = max(worst_t, float(np.max(np.abs(s_gpu[l, gg] - tref) / np.maximum(tref, 1e-6))))
                    n_done += n
        res["cpu_baseline"] = {"value": n_done / t_cpu, "unit": "entries/s", "cores": 1, "kind": "oracle",
                               "sample": f"{len(host)} of {L * Hkv} streams (layer, KV head), each "
                                         f"{n} entries, evaluated {n_done // n} times in {t_cpu:.1f} s of fp64 "
                                         f"numpy oracle time (one BLAS thread)"}
        res["parity"] = {"streams": len(host), "max_abs_out_err": worst_o, "max_rel_tally_err": worst_t}
    if args.calibration_copy:
        src = torch.empty(args.calibration_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    res["setup_s"] = {"settle_s": round(t_settle, 2)}
    print(json.dumps(res), flush=True)


SK_METRIC = ("KV entries ranked by step-aware selection (step utility + token saliency -> top-B keep "
             "set)/sec; achieved HBM GB/s vs peak (8B shape, 32K ctx)")


def bench_stepkv(args) -> None:
    """kvs_step_select over the 8B-shaped batch (32 layers x 8 KV heads x 32 768 entries)
    with an agent-trajectory step structure; one JSON line."""
    import torch
    import kv_cache_eviction_lse_amd as K
    from workloads import ALL
    from workloads import steps as WS
    from workloads.host import make_layout
    import oracle as O

    w = ALL["llama3_8b_32k"]
    lay = make_layout(w)
    L, Hkv = w.num_layers, w.num_kv_heads
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(7)
    step_off, first, bounds = WS.batch_steps(rng, lay.length)
    E = int(lay.entry_off[-1])
    s_h = np.empty((L, Hkv, E), np.float32)
    for i in range(w.num_seqs):
        e0, e1 = int(lay.entry_off[i]), int(lay.entry_off[i + 1])
        for l in range(L):
            for g in range(Hkv):
                s_h[l, g, e0:e1] = WS.step_scores(rng, bounds[i])
    beta = 0.5
    cache = K.CacheShape(L, Hkv, lay.num_pages)
    seqs = K.SeqBatch(lay.block_table, lay.start, lay.length, device=dev)
    steps = K.StepSet(step_off, first, device=dev)
    scores = torch.from_numpy(s_h).to(dev)
    budget_h = np.full(w.num_seqs, w.budget, np.int32)
    budget = torch.from_numpy(budget_h).to(dev)
    keep = torch.empty((L, Hkv, E), dtype=torch.uint8, device=dev)
    M = steps.num_steps
    util = torch.empty((L, Hkv, M), dtype=torch.float32, device=dev)
    need = K.kvs_step_select_workspace_size(cache, seqs, steps)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream()
    run = lambda: K.kvs_step_select(cache, seqs, steps, scores, beta, budget, budget_h, keep, util, ws)  # noqa: E731
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(20):
            run()
        torch.cuda.synchronize()
    t_settle = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        run()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0_, e1_ in evs:
        e0_.record(st)
        run()
        e1_.record(st)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    ev_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    entries = E * L * Hkv
    # scores read and keep bits written once per entry; per step its first slot and its
    # utility per stream
    byts = entries * (4 + 1) + M * (4 + 4 * L * Hkv) + 8 * (w.num_seqs + 1)
    gbps = byts / (ev_ms / 1000.0) / 1e9
    res = {
        "metric": SK_METRIC, "value": entries / (ms / 1000.0), "unit": "entries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "stepkv_llama3_8b_32k", "layers": L, "kv_heads": Hkv, "context": int(lay.length[0]),
                   "reasoning_steps": M, "budget": int(w.budget), "beta": beta,
                   "entries_per_step": entries},
        "hbm_gbps": gbps, "hbm_frac": gbps / HBM_PEAK_GBPS,
        "roofline": {"kernel": "step_key_kernel + stream_reg_kernel (keys from the step utilities)",
                     "bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": load_traffic("stepkv_llama3_8b_32k", "stream_reg", "stream.hip"),
                     "traffic_of": "stream_reg_kernel", "ms": ev_ms, "bytes_per_launch": byts},
        "setup_s": {"settle_s": round(t_settle, 2)},
    }
    if not args.no_cpu_baseline:
        keep_g, util_g = keep.cpu().numpy(), util.cpu().numpy()
        pick = np.random.default_rng(1).permutation(L * Hkv)
        t_cpu, n_done, streams, mism = 0.0, 0, 0, 0
        while t_cpu < args.cpu_seconds:
            for p in pick:
                l, g = divmod(int(p), Hkv)
                for i in range(w.num_seqs):
                    e0, e1 = int(lay.entry_off[i]), int(lay.entry_off[i + 1])
                    ta = time.perf_counter()
                    kw, _, uw = O.stepkv.step_select(s_h[l, g, e0:e1], bounds[i], beta, int(budget_h[i]))
                    t_cpu += time.perf_counter() - ta
                    n_done += e1 - e0
                    if streams < L * Hkv:
                        mism += int(np.sum(kw != keep_g[l, g, e0:e1].astype(bool)))
                        mism += int(np.sum(uw != util_g[l, g, step_off[i]:step_off[i + 1]]))
                if streams < L * Hkv:
                    streams += 1
                if t_cpu >= args.cpu_seconds:
                    break
        res["cpu_baseline"] = {"value": n_done / t_cpu, "unit": "entries/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n_done} entries ({streams} distinct streams of {L * Hkv}) in "
                                         f"{t_cpu:.1f} s of oracle time (numpy and exact integer sums)"}
        res["parity"] = {"streams": streams, "mismatches": mism}
    if args.calibration_copy:
        src = torch.empty(args.calibration_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(res), flush=True)


RATCHET_METRIC = ("KV entries scored+compacted/sec, amortised over the ratchet loop (one 8B-shape sequence "
                  "growing 8192 -> 33000 tokens, a round every 64 tokens); achieved HBM GB/s vs peak")


def bench_ratchet(args) -> None:
    """The ratchet loop: 387 rounds of (append 64 tokens, 32 observers, flag, eviction
    round).  Each round's eviction round is timed with HIP events on its stream; the
    appends, observers and their LSE (inputs the decode kernel would hand over) are
    prepared between rounds, untimed.  With --flags confidence the flag comes from the
    confidence monitor (ActKV Dissected, Component 2), whose call is timed apart.  One
    JSON line."""
    import torch
    import kv_cache_eviction_lse_amd as K
    from tests.ratchet_loop import APPEND, OBS, RatchetLoop, checked_round

    dev = torch.device("cuda", 0)
    lp = RatchetLoop(dev, flags=args.flags)
    R = lp.R
    L, Hkv, Hq = lp.L, lp.Hkv, lp.Hq
    check = set() if args.no_cpu_baseline else {1, R // 4, R // 2, 3 * R // 4, R}
    conf = torch.empty(APPEND, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream()
    t_round, t_score, t_conf = [], [], []
    entries, score_bytes, req_bytes, timed_entries = 0, 0, 0, 0
    worst, pinned, t_ora, n_ora, expansions = 0.0, 0, 0.0, 0, 0
    budgets = []
    t_wall = time.perf_counter()
    for r in range(1, R + 1):
        # the round's tokens and observers; their LSE (the decode kernel's hand-over) is
        # computed below, right before the round, except on the checked rounds
        q = lp.append(r)
        lse = torch.empty((L, Hq, OBS), dtype=torch.float32, device=dev)
        if r in check:
            lp.observer_lse(q, lse)
        if args.flags == "confidence":
            x = lp.step_logits(r)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            f = lp.flag(r, x, conf)           # confidence kernel, then the host trend
            e1.record(st)
            torch.cuda.synchronize()
            t_conf.append(e0.elapsed_time(e1))
        else:
            f = lp.flag(r)
        old = lp.budget
        expansions += int(lp.ratchet(f) != old)
        budgets.append(lp.budget)
        seqs, budget_h = lp.batch()
        obs = K.ObserverSet(q.view(torch.int16), lse, np.array([0, OBS], np.int64), device=dev)
        bufs = K.RoundBuffers(lp.cache, seqs, obs, budget_h, keep_hits=r in check)
        n, n_prev = lp.n, lp.n_prev
        if r in check:
            plan, w_, pn, to, no = checked_round(lp, r, q, lse, seqs, bufs)
            worst, pinned, t_ora, n_ora = max(worst, w_), pinned + pn, t_ora + to, n_ora + no
        else:
            n_prev_t = torch.tensor([n_prev], dtype=torch.int32, device=dev)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            torch.cuda.synchronize()
            # The LSE is device work on this stream (after its own host-to-device copies):
            # the round's calls are enqueued while it runs, as they would be behind the
            # decode kernel, so the events time the round's kernels and not the host's
            # enqueue on an idle GPU.
            lp.observer_lse(q, lse)
            ev[0].record(st)
            K.kvs_score(lp.cache, seqs, obs, lp.w.scale, bufs.scores, bufs.workspace)
            ev[1].record(st)
            plan = K.kvs_lrfu_select_compact(lp.cache, seqs, bufs.scores, 9, 10, lp.decay, n_prev_t, bufs.budget,
                                             bufs.budget_h, bufs.keep, bufs.pairs, bufs.pair_count)
            ev[2].record(st)
            torch.cuda.synchronize()
            t_round.append(ev[0].elapsed_time(ev[2]))
            t_score.append(ev[0].elapsed_time(ev[1]))
            e = n * L * Hkv
            pairs = int(bufs.pair_count.sum().item())
            timed_entries += e
            score_bytes += e * (2 * D + 4) + Hq * OBS * L * (2 * D + 4)
            req_bytes += e * (2 * D + 8) + Hq * OBS * L * (2 * D + 4) + pairs * (4 * 2 * D + 8)
        lp.finish(plan)
    t_wall = time.perf_counter() - t_wall
    ms_round = float(np.sum(t_round))
    ms_score = float(np.sum(t_score))
    gbps = score_bytes / (ms_score / 1000.0) / 1e9
    res = {
        "metric": RATCHET_METRIC, "value": timed_entries / (ms_round / 1000.0), "unit": "entries/s",
        "n_gpus": 1, "steps": len(t_round), "warmup": 0, "ms_per_step": ms_round / len(t_round),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "ratchet", "layers": L, "kv_heads": Hkv, "q_heads": Hq, "head_dim": D,
                   "prefill": 8192, "append_per_round": APPEND, "observers": OBS, "rounds": R,
                   "timed_rounds": len(t_round), "flags": args.flags, "budget_start": 512,
                   "budget_final": lp.budget, "budget_expansions": expansions,
                   "timing": "HIP events around each round's kvs_score -> kvs_lrfu_select_compact, "
                             "enqueued behind the device work that computes the round's observer LSE; "
                             "appends, observers and their LSE are untimed; "
                             "value = sum of entries / sum of round times"},
        "hbm_gbps": req_bytes / (ms_round / 1000.0) / 1e9,
        "hbm_frac": req_bytes / (ms_round / 1000.0) / 1e9 / HBM_PEAK_GBPS,
        "round_ms": {"median": float(np.median(t_round)), "min": float(np.min(t_round)),
                     "max": float(np.max(t_round)), "first_timed": t_round[0], "last_timed": t_round[-1]},
        "roofline": {"kernel": "kvs_score kernels over the loop", "bound": "hbm", "achieved": gbps,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "ms": ms_score / len(t_score), "bytes_per_launch": score_bytes / len(t_score)},
        "wall_s": round(t_wall, 1),
    }
    if t_conf:
        res["confidence_ms"] = {"median": float(np.median(t_conf)), "max": float(np.max(t_conf)),
                                "includes": "kvs_token_confidence over the round's 64 steps, the copy of 64 "
                                            "floats to the host and kvs_confidence_trend"}
    if check:
        res["cpu_baseline"] = {"value": n_ora / t_ora, "unit": "entries/s", "cores": 1, "kind": "oracle",
                               "sample": f"{len(check)} rounds x 2 streams (layer, KV head) run by the fp64 oracle "
                                         f"from the GPU's pre-round state: {n_ora} entries in {t_ora:.1f} s"}
        res["parity"] = {"rounds_checked": sorted(check), "max_rel_score_err": worst, "keep_pinned": pinned,
                         "keep_pinned_mismatch": 0}
    print(json.dumps(res), flush=True)


KM_METRIC = ("history-query passes of beacon maintenance (k-means++ seeding, then Lloyd k-means: assignment + "
             "exact update)/sec; achieved HBM GB/s vs peak (70B shape: 80 layers x 64 query heads, 4096 "
             "queries, k = 16, 25 iterations)")


def bench_kmeans(args) -> None:
    """kvs_beacon_seed then kvs_beacon_kmeans for every (layer, query head) of the 70B
    shape; one JSON line."""
    import torch
    import kv_cache_eviction_lse_amd as K
    from workloads import ALL
    from workloads.logits import bf16_bits_to_f64
    import oracle as O
    from tests.gpu_util import kmeans_update_mismatches

    w = ALL["llama3_70b_128k"]
    L, Hq, N, Kc, T = w.num_layers, w.num_q_heads, w.beacon_history, w.beacons, w.kmeans_iters
    P = L * Hq
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev).manual_seed(11)
    pts = torch.randn((P, N, 128), generator=g, device=dev).to(torch.bfloat16)
    uni = torch.rand((P, Kc), generator=g, device=dev)          # the k-means++ draws
    cent = torch.empty((P, Kc, 128), dtype=torch.float32, device=dev)
    asg = torch.empty((P, N), dtype=torch.int32, device=dev)
    bcn = torch.empty((P, Kc, 128), dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream()

    def run():
        K.kvs_beacon_seed(pts, uni, cent)
        K.kvs_beacon_kmeans(pts, cent, T, assign=asg, beacons=bcn)

    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        run()
        torch.cuda.synchronize()
    t_settle = time.perf_counter() - t_settle
    for _ in range(args.warmup):
        run()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0_, e1_, e2_ in evs:
        e0_.record(st)
        K.kvs_beacon_seed(pts, uni, cent)
        e1_.record(st)
        K.kvs_beacon_kmeans(pts, cent, T, assign=asg, beacons=bcn)
        e2_.record(st)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / args.steps
    seed_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in evs]))
    km_ms = float(np.mean([b.elapsed_time(c) for _, b, c in evs]))
    passes = P * N * (Kc - 1 + T)
    # each Lloyd iteration and each seeding round reads every history row once; the
    # centroids, beacons and assignments are written once
    km_bytes = P * N * 128 * 2 * T + P * Kc * 128 * (4 + 4 + 2) + P * N * 4
    seed_bytes = P * N * 128 * 2 * (Kc - 1) + P * Kc * (128 * 4 + 4)
    gbps = km_bytes / (km_ms / 1000.0) / 1e9
    flops = 2.0 * 2 * 128 * 16 * P * N * T          # two bf16 centroid parts x 16 groups (MFMA)
    res = {
        "metric": KM_METRIC, "value": passes / (ms / 1000.0), "unit": "point-passes/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "beacon_kmeans_llama3_70b", "layers": L, "q_heads": Hq, "problems": P,
                   "history": N, "k": Kc, "iters": T, "init": "k-means++ (device, seeded uniforms)"},
        "hbm_gbps": (km_bytes + seed_bytes) / (ms / 1000.0) / 1e9,
        "hbm_frac": (km_bytes + seed_bytes) / (ms / 1000.0) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"kernel": "kmeans_kernel", "bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": load_traffic("beacon_kmeans_llama3_70b", "kmeans", "kmeans.hip"),
                     "traffic_of": "kmeans_kernel", "ms": km_ms, "bytes_per_launch": km_bytes,
                     "mfma_tflops": flops / (km_ms / 1000.0) / 1e12},
        "seed": {"kernel": "kmeanspp_kernel", "ms": seed_ms, "bytes_per_launch": seed_bytes,
                 "gbps": seed_bytes / (seed_ms / 1000.0) / 1e9},
        "setup_s": {"settle_s": round(t_settle, 2)},
    }
    if not args.no_cpu_baseline:
        # parity on sampled problems: every seeding draw is a valid k-means++ step of the
        # oracle's fp64 distances; then one Lloyd iteration from the GPU's seeds gives a
        # valid argmin (within the fp32 bound) and the oracle's update bit for bit
        rows_dev = torch.empty((P, Kc), dtype=torch.int32, device=dev)
        K.kvs_beacon_seed(pts, uni, cent, rows=rows_dev)
        c_seed = cent.clone()
        K.kvs_beacon_kmeans(pts, cent, 1, assign=asg)
        torch.cuda.synchronize()
        pick = [0, P // 2 + 7, P - 1]
        mism, flips = 0, 0
        xs = {}
        for p in pick:
            x = bf16_bits_to_f64(pts[p].view(torch.int16).cpu().numpy().view(np.uint16))
            xs[p] = x
            up = uni[p].cpu().numpy()
            rows = rows_dev[p].cpu().numpy()
            mism += int(rows[0] != O.kmeans.seed_index(up[0], N))
            mism += sum(int(not O.kmeans.seed_step_valid(x, rows[:c], up[c], int(rows[c]), 3e-4))
                        for c in range(1, Kc))
            cp = c_seed[p].cpu().numpy()
            mism += int(np.sum(cp != x[rows].astype(np.float32)))
            a = asg[p].cpu().numpy()
            _, sc = O.kmeans.assign(x, cp)
            cmax = float(np.sqrt((cp.astype(np.float64) ** 2).sum(1)).max())
            tol = 1e-4 * (cmax ** 2 + np.sqrt((x * x).sum(1)) * cmax)
            mism += int(np.sum(sc[np.arange(N), a] > sc.min(axis=1) + tol))
            flips += int(np.sum(a != np.argmin(sc, axis=1)))
            mism += kmeans_update_mismatches(x, a, cp, cent[p].cpu().numpy())
        t_cpu, n_it = 0.0, 0
        cc = {p: c_seed[p].cpu().numpy() for p in pick}
        while t_cpu < args.cpu_seconds:
            for p in pick:
                ta = time.perf_counter()
                a, _ = O.kmeans.assign(xs[p], cc[p])
                cc[p] = O.kmeans.update(xs[p], a, cc[p])
                t_cpu += time.perf_counter() - ta
                n_it += 1
                if t_cpu >= args.cpu_seconds:
                    break
        res["cpu_baseline"] = {"value": n_it * N / t_cpu, "unit": "point-passes/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"{n_it} Lloyd iterations over {len(pick)} of {P} problems "
                                         f"({N} queries each) in {t_cpu:.1f} s of oracle time"}
        res["parity"] = {"problems": len(pick), "invalid": mism, "argmin_flips_within_bound": flips}
    if args.calibration_copy:
        src = torch.empty(args.calibration_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(res), flush=True)


# Measured by the default invocation too (one child process each, before this process
# touches the GPU), so that their figures come from the same run as the headline.
OTHER_WORKLOADS = (("ragged64", 5), ("llama3_70b_128k", 5), ("ratchet", 1), ("decode_llama3_8b_32k", 20),
                   ("token_confidence", 20), ("stepkv_llama3_8b_32k", 20), ("beacon_kmeans_llama3_70b", 5))


def run_other_workloads() -> dict:
    """One JSON summary per other workload, each from `bench.py --workload W` in a child
    process (its own GPU memory, freed when it exits)."""
    import subprocess
    res = {}
    for wname, steps in OTHER_WORKLOADS:
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", wname, "--no-cpu-baseline", "--no-others",
               "--steps", str(steps), "--warmup", "1"]
        t0 = time.perf_counter()
        try:
            p = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
            lines = [ln for ln in p.stdout.splitlines() if ln.startswith("{")]
            if p.returncode == 0 and lines:
                d = json.loads(lines[-1])
                r = {k: d[k] for k in ("metric", "value", "unit", "ms_per_step", "steps", "dtype") if k in d}
                if isinstance(d.get("roofline"), dict):
                    r["roofline"] = {k: d["roofline"].get(k) for k in ("kernel", "bound", "achieved", "peak",
                                                                          "unit", "frac")}
                res[wname] = r
            else:
                res[wname] = {"error": f"exit status {p.returncode}", "stderr_tail": p.stderr[-400:]}
        except subprocess.TimeoutExpired:
            res[wname] = {"error": "timed out after 300 s"}
        res[wname]["wall_s"] = round(time.perf_counter() - t0, 1)
        print(f"[bench] {wname}: {json.dumps(res[wname])}", file=sys.stderr, flush=True)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_32k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flags", choices=("bernoulli", "confidence"), default="bernoulli",
                    help="ratchet workload: the configuration's Bernoulli(0.05) flag, or the confidence "
                         "monitor's trend")
    ap.add_argument("--cpu-streams", type=int, default=48, help="streams in the oracle sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle CPU time")
    ap.add_argument("--separate", action="store_true",
                    help="run cut/LRFU, keep set, plan and move as four calls instead of two fused ones")
    ap.add_argument("--layer-chunks", type=int, default=0,
                    help="time rounds as one kvs_eviction_round call pipelined over this many layer "
                         "chunks (1: one call, no overlap); 0 (default): the stage calls in turn, with "
                         "the scorer timed by events inside the timed rounds")
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MiB",
                    help="after timing, copy MiB of device memory 3 times (counter calibration)")
    ap.add_argument("--settle", type=float, default=0.5, metavar="SECONDS",
                    help="untimed full rounds for SECONDS before the warmup steps, so that the "
                         "GPU's clocks have left their idle state (reported as settle_s)")
    ap.add_argument("--hold", type=float, default=0.0, metavar="SECONDS",
                    help="after timing, keep running full rounds for SECONDS (sustained rate, "
                         "e.g. for a power/clock sampler); reported under \"hold\"")
    ap.add_argument("--no-others", action="store_true",
                    help="the default run also measures the other workloads (ragged64, 70B, ratchet, "
                         "decode, confidence, step-aware, k-means) in child processes and reports them "
                         "under \"other_workloads\"; this skips that")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the eviction path "
              "shards over sequences, layers or KV heads with no exchange step, but this build "
              "runs and reports a single MI355X.", file=sys.stderr)
        sys.exit(2)

    if args.workload == "token_confidence":
        bench_confidence(args)
        return
    if args.workload == "decode_llama3_8b_32k":
        bench_decode(args)
        return
    if args.workload == "stepkv_llama3_8b_32k":
        bench_stepkv(args)
        return
    if args.workload == "beacon_kmeans_llama3_70b":
        bench_kmeans(args)
        return
    if args.workload == "ratchet":
        bench_ratchet(args)
        return
    others = None
    if (args.workload == "llama3_8b_32k" and not args.no_others and not args.no_cpu_baseline
            and not args.separate and args.layer_chunks == 0 and not args.hold and not args.calibration_copy):
        others = run_other_workloads()
    from workloads import ALL
    from workloads.host import make_layout, observers
    w = ALL[args.workload]
    chunks = 0 if args.separate else args.layer_chunks
    lay = make_layout(w)
    L, Hkv, Hq = w.num_layers, w.num_kv_heads, w.num_q_heads
    G = Hq // Hkv
    # sampled streams: spread over sequences, layers and heads
    rng = np.random.default_rng(0)
    all_streams = [(i, l, g) for i in range(w.num_seqs) if lay.length[i] > 0
                   for l in range(L) for g in range(Hkv)]
    pick = rng.choice(len(all_streams), size=min(args.cpu_streams, len(all_streams)), replace=False)
    sample = [all_streams[int(p)] for p in sorted(pick)]
    # counter-based draws for the sampled streams' observer heads, seeded PCG64 for the rest
    heads = {(l, h) for (_, l, g) in sample for h in range(g * G, (g + 1) * G)}
    q_host = observers(w, lay, heads=heads, only_heads=True)
    q_hist = [observers(w, lay, rnd=r, heads=heads, only_heads=True) for r in range(1, w.history_rounds + 1)]
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(16, cores))
    t0 = time.perf_counter()
    ora = oracle_leg(w, lay, sample, workers, args.cpu_seconds) if not args.no_cpu_baseline else None
    t_host = time.perf_counter() - t0

    import torch
    import kv_cache_eviction_lse_amd as K
    from workloads import device as DV
    import oracle as O
    from tests.gpu_util import gpu_history, pinned_keep_check

    dev = torch.device("cuda", 0)
    t0 = time.perf_counter()
    exact = sample if ora is not None else ()
    pre = {s: DV.mini_stream_bytes(m, G) for s, m in zip(sample, ora["minis"])} if ora is not None else None
    d = DV.fill(w, lay, q_host, dev, exact_streams=exact, exact_bytes=pre)
    seqs = K.SeqBatch(lay.block_table, lay.start, lay.length, device=dev)
    obs = K.ObserverSet(d.q, d.lse, lay.obs_off, device=dev)
    budget_h = np.full(w.num_seqs, w.budget, np.int32)
    bufs = K.RoundBuffers(K.PagedCache(d.k, d.v, d.crf), seqs, obs, budget_h, keep_hits=True)
    if w.history_rounds:
        # the LRFU history: untimed score -> LRFU rounds with fresh observers
        ex_lse = {s: h[2] for s, h in zip(sample, ora["hist"])} if ora is not None else None
        gpu_history(w, lay, d, K.PagedCache(d.k, d.v, d.crf), seqs, q_hist, exact, bufs.scores,
                    bufs.workspace, exact_lse=ex_lse)
    torch.cuda.synchronize()
    t_fill = time.perf_counter() - t0
    # Each step starts from the workload's prior LRFU state (after its history): steps
    # use their own copy of that CRF pool (prepared before timing), so every step evicts
    # from the same ranking instead of re-keeping what the previous step kept.
    # (warmup rounds cycle over at most 8 copies: their results are not used)
    n_warm = min(args.warmup, 8)
    n_copies = n_warm + args.steps + 2   # [0] parity round, [-1] settle and hold rounds
    crfs = [d.crf.clone() for _ in range(n_copies)]
    # The moves write kept K rows into evicted slots, which changes what the next round
    # on the same pool scores.  Each timed step therefore gets its own copy of the K pool
    # as well (V rows only travel, their contents decide nothing), when they fit in
    # device memory; otherwise the timed steps share the K pool and say so.
    k_bytes = d.k.numel() * d.k.element_size()
    fresh_k = k_bytes * (args.steps + 1) < torch.cuda.mem_get_info()[0] * 0.8
    k_steps = [d.k.clone() for _ in range(args.steps)] if fresh_k else [d.k] * args.steps
    caches = [K.PagedCache(d.k, d.v, c) for c in crfs]
    for k in range(args.steps):
        caches[1 + n_warm + k] = K.PagedCache(k_steps[k], d.v, crfs[1 + n_warm + k])
    decay_h = np.array([K.kvs_lrfu_decay(0.5, int(x)) for x in lay.dt], np.float32)
    decay = torch.from_numpy(decay_h).to(dev)
    n_prev = torch.from_numpy(lay.n_prev.astype(np.int32)).to(dev)
    scale = w.scale
    st = torch.cuda.current_stream()

    # first round, stage by stage: keep the sampled streams' intermediates for parity
    rec = {}
    if ora is not None:
        c = caches[0]
        pages = {s: torch.from_numpy(lay.block_table[s[0]][:(int(lay.start[s[0]]) + int(lay.length[s[0]]) + 15)
                                                          // 16].astype(np.int64)).to(dev) for s in sample}

        def crf_of(s):
            return c.crf[s[1]][pages[s], s[2]].cpu().numpy()

        def ent(buf, s):
            i, l, g = s
            return buf[l, g, int(lay.entry_off[i]):int(lay.entry_off[i + 1])].cpu().numpy()

        torch.cuda.synchronize()
        for s in sample:
            rec[s] = {"crf0": crf_of(s)}
        K.kvs_score(c, seqs, obs, scale, bufs.scores, bufs.workspace)
        if args.separate:
            K.kvs_lrfu_update(c, seqs, bufs.scores, 9, 10, decay, n_prev, bufs.hit)
            K.kvs_select(c, seqs, bufs.scores, bufs.budget, bufs.budget_h, bufs.keep)
        else:
            K.kvs_lrfu_select(c, seqs, bufs.scores, 9, 10, decay, n_prev, bufs.budget, bufs.budget_h, bufs.keep,
                              hit=bufs.hit)
        torch.cuda.synchronize()
        for s in sample:
            rec[s].update(s=ent(bufs.scores, s), hit=ent(bufs.hit, s).astype(bool),
                          keep=ent(bufs.keep, s).astype(bool), crf1=crf_of(s))
        K.kvs_plan_compact(c, seqs, bufs.keep, bufs.budget, bufs.budget_h, bufs.pairs, bufs.pair_count)
        torch.cuda.synchronize()
    # The hit bytes are an optional inspection output (the CRF carries the hits into the
    # next round); the parity round above asked for them, the timed rounds do not.
    bufs.hit = None
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle:
        for _ in range(20):
            K.eviction_round(caches[-1], seqs, obs, bufs, decay, n_prev, scale, fused=not args.separate,
                             layer_chunks=chunks)
        torch.cuda.synchronize()
    t_settle = time.perf_counter() - t_settle
    for wi in range(args.warmup):
        K.eviction_round(caches[1 + wi % max(n_warm, 1)], seqs, obs, bufs, decay, n_prev, scale,
                         fused=not args.separate, layer_chunks=chunks)
    torch.cuda.synchronize()

    # per step: events before the scorer, after it, and after the round's last call
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        c = caches[1 + n_warm + k]
        if chunks > 0:
            # the whole round in one call, scoring overlapped with the cut, keep set and
            # moves of the previous layer chunk (the scorer is timed alone below)
            evs[k][0].record(st)
            K.eviction_round(c, seqs, obs, bufs, decay, n_prev, scale, layer_chunks=chunks)
            evs[k][2].record(st)
            continue
        # (a round ends where the next one's first event is recorded: each event record
        # leaves the GPU idle for a few microseconds, so a round carries two, not three)
        evs[k][0].record(st)
        K.kvs_score(c, seqs, obs, scale, bufs.scores, bufs.workspace)
        evs[k][1].record(st)
        if args.separate:
            K.kvs_lrfu_update(c, seqs, bufs.scores, 9, 10, decay, n_prev, None)
            K.kvs_select(c, seqs, bufs.scores, bufs.budget, bufs.budget_h, bufs.keep)
            K.kvs_plan(seqs, L, Hkv, bufs.keep, bufs.budget, bufs.budget_h, bufs.pairs, bufs.pair_count)
            K.kvs_compact(c, seqs, bufs.budget_h, bufs.pairs, bufs.pair_count)
        else:
            K.kvs_lrfu_select_compact(c, seqs, bufs.scores, 9, 10, decay, n_prev, bufs.budget, bufs.budget_h,
                                      bufs.keep, bufs.pairs, bufs.pair_count)
        if k == args.steps - 1:
            evs[k][2].record(st)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1000.0 / args.steps
    if chunks > 0:
        round_ev = [a.elapsed_time(c_) for a, _, c_ in evs]
    else:
        round_ev = [evs[k][0].elapsed_time(evs[k + 1][0] if k + 1 < args.steps else evs[k][2])
                    for k in range(args.steps)]
    if chunks > 0:
        # the dominant kernel's launch time, live with HIP events on its stream: the scorer
        # alone on the same inputs, as many launches as timed steps
        for k in range(args.steps):
            evs[k][0].record(st)
            K.kvs_score(caches[1 + n_warm + k], seqs, obs, scale, bufs.scores, bufs.workspace)
            evs[k][1].record(st)
        torch.cuda.synchronize()
    score_ev = [a.elapsed_time(b) for a, b, _ in evs]
    score_ms = float(np.mean(score_ev))

    entries = int(lay.entry_off[-1]) * L * Hkv
    rows = int(sum((lay.obs_off[i + 1] - lay.obs_off[i]) for i in range(w.num_seqs))) * Hq * L
    pairs = int(bufs.pair_count.sum().item())
    hold = None
    if args.hold > 0:
        # sustained full rounds, untimed by the contract: the rate once the GPU has settled
        # (at its power limit).  Each round first restores the prior CRF pool with a
        # device copy (33.5 MB at 8B), so that every round evicts from the same ranking;
        # the copy is inside the reported time.
        c = caches[-1]
        n_hold = 0
        th0 = time.perf_counter()
        while time.perf_counter() - th0 < args.hold:
            for _ in range(50):
                c.crf.copy_(d.crf)
                K.eviction_round(c, seqs, obs, bufs, decay, n_prev, scale, fused=not args.separate,
                                 layer_chunks=chunks)
            torch.cuda.synchronize()
            n_hold += 50
        hold = {"seconds": round(time.perf_counter() - th0, 2), "steps": n_hold,
                "ms_per_step": (time.perf_counter() - th0) * 1000.0 / n_hold,
                "includes": "a CRF-pool reset copy per round; the K pool is not reset, so these "
                            "rounds score rows earlier moves wrote"}
    req_bytes = entries * (2 * D + 8) + rows * (2 * D + 4) + pairs * (4 * 2 * D + 8)
    gbps = req_bytes / (ms_per_step / 1000.0) / 1e9
    copy_gbps = copy_peak_gbps(dev)
    score_bytes = entries * (2 * D + 4) + rows * (2 * D + 4)
    score_gbps = score_bytes / (score_ms / 1000.0) / 1e9
    # MFMA work of the scorer: 2 * D flops per (observer row, entry) pair of a stream
    score_flops = sum(2.0 * D * float(lay.obs[i]) * Hq * int(lay.length[i]) * L for i in range(w.num_seqs))
    score_tflops = score_flops / (score_ms / 1000.0) / 1e12
    traffic = load_traffic(w.name)
    # the bound by the published peaks: whichever takes longer at its peak
    if score_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > score_bytes / (HBM_PEAK_GBPS * 1e9):
        roofline = {"kernel": score_kernels(w, lay), "bound": "mfma", "achieved": score_tflops,
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": score_tflops / MFMA_BF16_PEAK_TFLOPS,
                    "traffic": traffic, "ms": score_ms, "ms_median": float(np.median(score_ev)),
                    "flops_per_launch": score_flops, "hbm_gbps": score_gbps}
    else:
        roofline = {"kernel": score_kernels(w, lay), "bound": "hbm", "achieved": score_gbps,
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": score_gbps / HBM_PEAK_GBPS,
                    "traffic": traffic, "ms": score_ms, "ms_median": float(np.median(score_ev)),
                    "bytes_per_launch": score_bytes, "mfma_tflops": score_tflops,
                    "frac_of_copy": score_gbps / copy_gbps}

    out = {
        "metric": METRIC if w.name == "llama3_8b_32k" else METRIC.replace("(8B shape, 32K ctx)", f"({w.name})"),
        "value": entries / (ms_per_step / 1000.0),
        "unit": "entries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "kv_heads": Hkv, "q_heads": Hq,
                   "head_dim": D, "page_size": 16, "context": int(lay.length[0]),
                   "pool_pages": lay.num_pages, "observers": int(lay.obs[0]), "budget": w.budget,
                   "entries_per_step": entries, "layer_chunks": chunks,
                   "history_rounds": w.history_rounds,
                   "step_state": ("each timed step starts from its own copy of the post-history CRF pool "
                                  "and of the K pool" if fresh_k else
                                  "each timed step starts from its own copy of the CRF pool; the K pool is "
                                  "shared, so later steps score the rows earlier moves wrote")},
        "hbm_gbps": gbps,
        "hbm_frac": gbps / HBM_PEAK_GBPS,
        # the same rate against a measured plain device copy (1 GiB, read + written)
        "copy_peak_gbps": copy_gbps,
        "hbm_frac_of_copy": gbps / copy_gbps,
        "required_bytes_per_step": req_bytes,
        "pairs_per_step": pairs,
        # per-step round times from HIP events (the events add a few microseconds)
        "round_events_ms": {"mean": float(np.mean(round_ev)), "median": float(np.median(round_ev)),
                            "min": float(np.min(round_ev)), "max": float(np.max(round_ev))},
        "roofline": roofline,
    }
    if hold is not None:
        hold["entries_per_s"] = entries / (hold["ms_per_step"] / 1000.0)
        out["hold"] = hold

    if ora is not None:
        # parity of the first round on the sampled streams: scores against the oracle on
        # the same bytes; cut, LRFU and keep set exact on the GPU's own inputs; the keep
        # set end to end (the oracle's round from the GPU's pre-round CRF) wherever the
        # oracle's margins pin it; the history's CRF exact wherever no history cut was
        # within the score tolerance
        worst, comp_bad, pinned_total, bad, hist_bad, hist_unamb = 0.0, 0, 0, 0, 0, 0
        for idx, s in enumerate(sample):
            i, l, g = s
            n, stt = int(lay.length[i]), int(lay.start[i])
            pos = stt + np.arange(n)
            pi, row = pos // 16, pos % 16
            r, o = rec[s], ora["rounds"][idx]
            so, ho = o["s"], o["hit"]
            sg, hg, kg = r["s"], r["hit"], r["keep"]
            c0, c1 = r["crf0"][pi, row], r["crf1"][pi, row]
            nz = so > 0
            if nz.any():
                worst = max(worst, float(np.max(np.abs(sg[nz].astype(np.float64) - so[nz]) / so[nz])))
            comp_bad += int(np.sum(hg != O.mass_cut(sg)))
            want1 = O.lrfu_update(c0, hg, np.float32(decay_h[i]), int(lay.n_prev[i]))
            comp_bad += int(np.sum(c1.view(np.uint32) != want1.view(np.uint32)))
            comp_bad += int(np.sum(kg != O.select_top_b(c1, sg, int(w.budget))))
            crf_tf = O.lrfu_update(c0, ho, O.lrfu_decay(0.5, int(lay.dt[i])), int(lay.n_prev[i]))
            keep_tf = O.select_top_b(crf_tf, so, int(w.budget))
            pn, nb = pinned_keep_check(so, crf_tf, keep_tf, ho, sg, c1, kg)
            pinned_total += pn
            bad += nb
            if ora["hist"][idx] is not None:
                c_hist, unamb, _ = ora["hist"][idx]
                ch = c_hist[0, pi, 0, row]
                hist_bad += int(np.sum(c0[unamb].view(np.uint32) != ch[unamb].view(np.uint32)))
                hist_unamb += int(unamb.sum())
        n_ent = int(sum(int(lay.length[i]) for (i, _, _) in sample)) * ora["passes"]
        t_sum = ora["cpu_s"]
        try:
            from threadpoolctl import threadpool_info
            blas = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
        except Exception:
            blas = None
        out["cpu_baseline"] = {
            "value": n_ent / ora["wall"], "unit": "entries/s", "cores": ora["workers"], "kind": "oracle",
            "sample": f"{len(sample)} of {len(all_streams)} streams (sequence, layer, KV head) of the same "
                      f"workload, {ora['passes']} oracle rounds each (score, cut, LRFU, keep set, plan, moves; "
                      f"fp64 numpy) over a pool of {ora['workers']} processes with one BLAS thread each: "
                      f"{ora['wall']:.2f} s wall, {t_sum:.1f} s of process time",
            "host_cores": cores, "cpu_model": cpu_model(), "blas_threads_per_process": 1,
            "blas_threads_available": blas, "per_process_entries_per_s": n_ent / t_sum,
        }
        out["parity"] = {"streams": len(sample), "max_rel_score_err": worst,
                         "component_mismatches": comp_bad,
                         "keep_pinned": pinned_total, "keep_pinned_mismatch": bad}
        if w.history_rounds:
            out["parity"].update(history_unambiguous=hist_unamb, history_crf_mismatch=hist_bad)
    if args.calibration_copy:
        # a plain device copy of known size, for scaling the HBM byte counters
        src = torch.empty(args.calibration_copy << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    out["setup_s"] = {"oracle_leg": round(t_host, 2), "oracle_prep": round(ora["prep_s"], 2) if ora else None,
                      "device_fill_and_history": round(t_fill, 2), "settle_s": round(t_settle, 2)}
    if others is not None:
        out["other_workloads"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
