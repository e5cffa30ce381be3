"""One eviction round over a batch: score -> mass cut + LRFU -> top-B -> plan -> compact.

A thin driver over the C ABI: it owns the per-round device buffers (scores, keep,
pairs, workspace) and enqueues the five calls on one stream.  It never synchronizes;
the host outputs of the plan (freed pages, new start/len) are available at once.
"""
from __future__ import annotations

import numpy as np

from . import _lib as K


class RoundBuffers:
    """Per-round device buffers sized for a (cache, batch, observers, budget) shape."""

    def __init__(self, cache: K.PagedCache, seqs: K.SeqBatch, obs: K.ObserverSet,
                 budget_h: np.ndarray, keep_hits: bool = False):
        import torch
        dev = cache.k.device
        L, Hkv = cache.c.num_layers, cache.c.num_kv_heads
        E = seqs.entries
        S = seqs.num_seqs
        self.scores = torch.empty((L, Hkv, max(E, 1)), dtype=torch.float32, device=dev)
        self.keep = torch.empty((L, Hkv, max(E, 1)), dtype=torch.uint8, device=dev)
        self.hit = torch.empty((L, Hkv, max(E, 1)), dtype=torch.uint8, device=dev) if keep_hits else None
        ws = K.kvs_score_workspace_size(cache, seqs, obs)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.P = K.kvs_pair_capacity(seqs, budget_h)
        self.pairs = torch.empty((L, Hkv, S, max(self.P, 1), 2), dtype=torch.int32, device=dev)
        self.pair_count = torch.empty((L, Hkv, max(S, 1)), dtype=torch.int32, device=dev)
        self.budget_h = np.ascontiguousarray(budget_h, np.int32)
        self.budget = torch.from_numpy(self.budget_h).to(dev)


def eviction_round(cache: K.PagedCache, seqs: K.SeqBatch, obs: K.ObserverSet, bufs: RoundBuffers,
                   decay, n_prev, scale: float, mass_num: int = 9, mass_den: int = 10,
                   stream=None, fused: bool = True, layer_chunks: int = 0) -> K.PlanHost:
    """Enqueue one full round; returns the host-side plan (shift, new start/len, freed pages).
    fused: the cut, LRFU update, keep set, plan and moves as one call (same results).
    layer_chunks > 0: the whole round as one kvs_eviction_round call, pipelined over that
    many layer chunks (1: no overlap)."""
    L, Hkv = cache.c.num_layers, cache.c.num_kv_heads
    if layer_chunks > 0:
        return K.kvs_eviction_round(cache, seqs, obs, scale, mass_num, mass_den, decay, n_prev, bufs.budget,
                                    bufs.budget_h, bufs.scores, bufs.hit, bufs.keep, bufs.pairs, bufs.pair_count,
                                    bufs.workspace, layer_chunks, stream)
    K.kvs_score(cache, seqs, obs, scale, bufs.scores, bufs.workspace, stream)
    if fused:
        return K.kvs_lrfu_select_compact(cache, seqs, bufs.scores, mass_num, mass_den, decay, n_prev, bufs.budget,
                                         bufs.budget_h, bufs.keep, bufs.pairs, bufs.pair_count, bufs.hit, stream)
    K.kvs_lrfu_update(cache, seqs, bufs.scores, mass_num, mass_den, decay, n_prev, bufs.hit, stream)
    K.kvs_select(cache, seqs, bufs.scores, bufs.budget, bufs.budget_h, bufs.keep, stream)
    plan = K.kvs_plan(seqs, L, Hkv, bufs.keep, bufs.budget, bufs.budget_h, bufs.pairs,
                      bufs.pair_count, stream)
    K.kvs_compact(cache, seqs, bufs.budget_h, bufs.pairs, bufs.pair_count, stream)
    return plan
