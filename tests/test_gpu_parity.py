"""GPU parity of the five C-ABI calls against the fp64 oracle on identical inputs.

Scores: within 1e-3 relative.  Cut, LRFU, select, plan and compaction: exact,
each given the GPU's own previous-stage output (identical inputs).  End to end:
the keep set matches the oracle wherever the oracle's margins exceed 1e-3."""
import zlib

import numpy as np
import pytest

import oracle as O
from tests import gpu_util as U
from workloads import TINY
from workloads.edge import random_batch
from workloads.host import full_inputs, make_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_eviction_lse_amd as K
    K.lib()


def test_tiny_stages():
    w = TINY
    lay = make_layout(w)
    inp = full_inputs(w, lay)
    budget = np.full(w.num_seqs, w.budget, np.int32)
    decay = np.array([O.lrfu_decay(0.5, int(d)) for d in lay.dt], np.float32)
    print(f"tiny: L{w.num_layers} Hkv{w.num_kv_heads} Hq{w.num_q_heads} n={lay.length.tolist()}", flush=True)
    out = U.run_stages(lay, inp, w.num_q_heads, budget, decay)
    worst = U.check_stages(lay, inp, out, w.num_q_heads, budget, decay)
    print(f"tiny: max relative score error {worst:.3e}")
    assert out["keep"].sum() == w.budget


def test_tiny_end_to_end_pinned():
    w = TINY
    lay = make_layout(w)
    inp = full_inputs(w, lay)
    budget = np.full(w.num_seqs, w.budget, np.int32)
    decay = np.array([O.lrfu_decay(0.5, int(d)) for d in lay.dt], np.float32)
    out = U.run_stages(lay, inp, w.num_q_heads, budget, decay)
    k, v, c = inp.k_pool.copy(), inp.v_pool.copy(), inp.crf_pool.copy()
    res = O.eviction_round(k, v, c, inp.q, inp.lse, lay.obs_off, lay.block_table, lay.start,
                           lay.length, w.num_q_heads, w.scale, 0.5, lay.dt, lay.n_prev, budget)
    n = int(lay.length[0])
    page, row = O.slot_location(lay.block_table[0], lay.start[0], np.arange(n))
    pinned, bad = U.pinned_keep_check(res["s"][(0, 0, 0)], res["crf"][(0, 0, 0)], res["keep"][(0, 0, 0)],
                                      res["hit"][(0, 0, 0)], out["s"][0, 0, :n],
                                      out["crf1"][0, page, 0, row], out["keep"][0, 0, :n])
    print(f"tiny end-to-end: {pinned} of {n} entries pinned, {bad} mismatches")
    assert bad == 0 and pinned > n // 2


EDGE_CASES = [
    # name, L, Hkv, Hq, lengths, starts, observers, budgets
    ("one_entry", 1, 1, 4, [1], [0], [16], [1]),
    ("page_edges_mfma", 1, 2, 8, [15, 16, 17, 33], [0, 0, 15, 7], [16, 17, 20, 32], [4, 16, 3, 40]),
    # the VALU scorer takes R = O G < 16 rows, the MFMA scorer 16 <= R <= 128
    ("few_observers", 2, 2, 8, [100, 37, 300], [3, 0, 9], [1, 8, 15], [10, 0, 64]),
    ("valu_rows", 2, 2, 4, [100, 300, 65], [3, 9, 0], [1, 3, 7], [10, 64, 20]),
    ("mfma_rows_16", 1, 2, 4, [300, 97], [5, 0], [8, 9], [40, 30]),
    ("mixed_paths", 1, 2, 8, [200, 513, 70], [5, 0, 15], [3, 16, 15], [50, 100, 80]),
    ("big_group", 1, 1, 8, [777], [11], [40], [300]),
    ("two_row_groups", 1, 1, 4, [1000], [2], [65], [256]),
    ("three_row_groups", 1, 2, 16, [600, 250], [0, 4], [40, 33], [128, 7]),
    ("empty_and_no_obs", 1, 1, 4, [0, 64, 50], [0, 0, 3], [16, 0, 16], [5, 5, 100]),
    ("budget_all", 2, 1, 4, [129, 64], [1, 15], [20, 16], [129, 1000]),
    ("long_multi_chunk", 1, 1, 4, [5000, 3333], [0, 13], [24, 18], [700, 1000]),
    ("gqa1", 1, 4, 4, [300, 300], [0, 8], [16, 16], [30, 30]),
    ("pipe8_g32", 1, 1, 32, [300], [0], [15], [40]),
    # streams longer than the register-resident per-stream kernels hold (32768 entries)
    ("long_stream", 1, 1, 4, [40000, 2000], [5, 0], [16, 16], [3000, 700]),
    # the pipelined scorer: 128 < R <= 256 rows on 4 waves (3 or 4 of them with rows),
    # R > 256 on 8 waves in row groups of 512 (one or two groups, the second nearly empty)
    ("pipe4_rows", 1, 2, 8, [1000, 333, 70], [3, 0, 15], [33, 48, 64], [100, 50, 70]),
    ("pipe8_rows", 1, 1, 8, [900, 401], [5, 9], [40, 64], [200, 100]),
    ("pipe8_two_groups", 1, 1, 8, [600], [7], [128], [128]),
    ("pipe8_ragged_groups", 1, 1, 4, [500], [0], [129], [64]),
    ("all_paths", 2, 2, 8, [300, 300, 300, 300], [0, 5, 10, 15], [3, 20, 50, 100], [50, 50, 50, 50]),
    # chunks long enough that the LDS rings wrap (9 and 19 steps per chunk)
    ("pipe4_long_chunks", 2, 8, 32, [40000], [3], [50], [5000]),
    ("pipe8_long_chunks", 2, 8, 64, [40000], [3], [50], [5000]),
    # the largest GQA group (G = 64): R = 576 rows, two row groups of the 8-wave scorer
    ("max_group", 1, 1, 64, [500], [3], [9], [100]),
    # the register-resident per-stream kernels' limit (32 768 entries) and one past it
    ("reg_boundary", 1, 1, 4, [32768, 32769], [0, 7], [16, 16], [1000, 32768]),
    # more than 255 sequences: item tables built on the device
    ("many_seqs", 1, 1, 4, [(37 * i) % 90 + 1 for i in range(300)], [(5 * i) % 16 for i in range(300)],
     [16 + (i % 3) * 7 if i % 4 else 6 for i in range(300)], [(11 * i) % 50 for i in range(300)]),
]


@pytest.mark.parametrize("case", EDGE_CASES, ids=[c[0] for c in EDGE_CASES])
def test_edge_stages(case):
    name, L, Hkv, Hq, lengths, starts, obs, budgets = case
    print(f"edge {name}: L{L} Hkv{Hkv} Hq{Hq} n={lengths} start={starts} O={obs} B={budgets}", flush=True)
    lay, inp = random_batch(zlib.crc32(name.encode()), L, Hkv, Hq, lengths, starts, obs)
    budget = np.asarray(budgets, np.int32)
    decay = np.array([O.lrfu_decay(0.5, int(d)) for d in lay.dt], np.float32)
    out = U.run_stages(lay, inp, Hq, budget, decay)
    worst = U.check_stages(lay, inp, out, Hq, budget, decay)
    print(f"edge {name}: max relative score error {worst:.3e}")


FUSED_CASES = ["page_edges_mfma", "mixed_paths", "empty_and_no_obs", "budget_all", "long_multi_chunk",
               "long_stream", "many_seqs", "all_paths", "pipe8_two_groups"]


@pytest.mark.parametrize("name", FUSED_CASES)
def test_fused_lrfu_select(name):
    """kvs_lrfu_select and kvs_plan_compact give the same CRF, hits, keep set, pairs and
    moved bytes as the separate calls."""
    case = next(c for c in EDGE_CASES if c[0] == name)
    _, L, Hkv, Hq, lengths, starts, obs, budgets = case
    print(f"fused {name}: L{L} Hkv{Hkv} Hq{Hq} n={lengths}", flush=True)
    lay, inp = random_batch(zlib.crc32(name.encode()), L, Hkv, Hq, lengths, starts, obs)
    budget = np.asarray(budgets, np.int32)
    decay = np.array([O.lrfu_decay(0.5, int(d)) for d in lay.dt], np.float32)
    out = U.run_stages(lay, inp, Hq, budget, decay, fused=True)
    U.check_stages(lay, inp, out, Hq, budget, decay)


def test_lrfu_denormal_and_exact_values():
    """CRF arithmetic on the GPU keeps subnormals (gradual underflow) and rounds once."""
    lay, inp = random_batch(77, 1, 1, 4, [64], [0], [16], prior_crf=True)
    # priors that exercise subnormal results and fma rounding
    vals = np.array([2.0 ** -100, 2.0 ** -120, 1.0, 1.9999999, 0.75, 2.0 ** -96, 3e-39, 0.0] * 8,
                    np.float32)
    page, row = O.slot_location(lay.block_table[0], 0, np.arange(64))
    inp.crf_pool[0, page, 0, row] = vals
    budget = np.array([8], np.int32)
    for dt in (1, 2, 33, 64):
        decay = np.array([O.lrfu_decay(0.5, dt)], np.float32)
        out = U.run_stages(lay, inp, 4, budget, decay)
        U.check_stages(lay, inp, out, 4, budget, decay)
