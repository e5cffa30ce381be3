"""The five seeded synthetic workloads (shapes follow the ActKV and BeaconKV pages).

Shapes: ActKV's agent trajectories are ~31-33K tokens (ActKV Dissected, "Start
with the numbers"); observers (action tokens) are under 1 % of entries.  BeaconKV
combines a few cluster-representative historical queries with recent queries
(BeaconKV, Key ideas).  No dataset is used: every tensor is drawn from a
counter-based generator keyed by (seed, config name, tensor kind, index).
"""
from __future__ import annotations

import zlib
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    num_layers: int
    num_kv_heads: int
    num_q_heads: int
    num_seqs: int
    # context length: fixed, or uniform in [len_lo, len_hi]
    len_lo: int
    len_hi: int
    # observers per sequence: fixed, or uniform in [obs_lo, obs_hi]
    obs_lo: int
    obs_hi: int
    budget: int
    planted_frac: float
    page_placement: str          # "in_order" | "random" | "interleaved" | "permutation"
    pool_pages: int              # 0: exactly the pages the sequences need
    prior_crf: bool              # True: a prior CRF in [0, 2) for every live entry
    dt_lo: int = 64
    dt_hi: int = 64
    beacons: int = 0             # leading observers that are k-means centroids
    beacon_history: int = 0      # history queries per (layer, query head) clustered
    kmeans_iters: int = 25
    head_dim: int = 128
    page_size: int = 16
    seed: int = 0
    # ratchet loop
    rounds: int = 0
    append_per_round: int = 0
    flag_prob: float = 0.0
    budget_cap: int = 30000
    # untimed score -> LRFU rounds (fresh observers, dt uniform in [dt_lo, dt_hi]) that
    # build the LRFU history before the measured round
    history_rounds: int = 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / (self.head_dim ** 0.5)

    @property
    def key(self) -> int:
        """64-bit Philox key: (crc32(name), seed)."""
        return (zlib.crc32(self.name.encode()) << 32) | (self.seed & 0xFFFFFFFF)


TINY = Workload(
    name="tiny", num_layers=1, num_kv_heads=1, num_q_heads=4, num_seqs=1,
    len_lo=4096, len_hi=4096, obs_lo=32, obs_hi=32, budget=512, planted_frac=0.05,
    page_placement="in_order", pool_pages=256, prior_crf=False)

LLAMA8B = Workload(
    name="llama3_8b_32k", num_layers=32, num_kv_heads=8, num_q_heads=32, num_seqs=1,
    len_lo=32768, len_hi=32768, obs_lo=64, obs_hi=64, budget=512, planted_frac=0.02,
    page_placement="random", pool_pages=4096, prior_crf=True, dt_lo=8, dt_hi=64, history_rounds=4)

RAGGED = Workload(
    name="ragged64", num_layers=32, num_kv_heads=8, num_q_heads=32, num_seqs=64,
    len_lo=8192, len_hi=33000, obs_lo=8, obs_hi=128, budget=2048, planted_frac=0.02,
    page_placement="interleaved", pool_pages=0, prior_crf=False)

RATCHET = Workload(
    name="ratchet", num_layers=32, num_kv_heads=8, num_q_heads=32, num_seqs=1,
    len_lo=8192, len_hi=8192, obs_lo=32, obs_hi=32, budget=512, planted_frac=0.02,
    page_placement="random", pool_pages=2 * ((33000 + 64 + 15) // 16), prior_crf=False,
    rounds=387, append_per_round=64, flag_prob=0.05, budget_cap=30000)

LLAMA70B = Workload(
    name="llama3_70b_128k", num_layers=80, num_kv_heads=8, num_q_heads=64, num_seqs=1,
    len_lo=131072, len_hi=131072, obs_lo=128, obs_hi=128, budget=4096, planted_frac=0.0,
    page_placement="permutation", pool_pages=8192, prior_crf=False,
    beacons=16, beacon_history=4096)

ALL = {w.name: w for w in (TINY, LLAMA8B, RAGGED, RATCHET, LLAMA70B)}

# Philox tensor tags
TAG_K, TAG_V, TAG_Q, TAG_CRF, TAG_PLANT, TAG_HIST, TAG_LAYOUT, TAG_LEN, TAG_OBS, \
    TAG_DT, TAG_FLAG, TAG_KMPP, TAG_HDT = range(1, 14)

# index strides (element index = ((((seq*L + l)*Hkv + g)*TOKENS + t)*D + d)
TOKENS_MAX = 1 << 20
OBS_MAX = 1 << 10
