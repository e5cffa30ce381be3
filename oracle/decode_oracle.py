"""Plain, slow CPU oracle for paged decode attention that emits the log-sum-exp and
tallies the attention each cached entry receives.

TEST INFRASTRUCTURE ONLY. Nothing in the product library may import, call or
execute this module; the tests, the smoke check and the benchmark's CPU baseline
use it.  It shares no code with the HIP path.

Source: "ActKV Dissected: 99% of an Agent's KV Cache Is Scratch Work, and the
Budget Follows Hesitation" (zhichai.net), Component 3: paged attention produces
each query row's log-sum-exp as a byproduct, and the attention a row puts on an
entry is recovered from that row's logit minus its LSE, block by block, without
gathering or recomputing the attention matrix; Component 1: an entry's signal is
the attention it receives from the action tokens, summed.

Readings (stated here and in the design notes):
  D1. The decode queries of one call are rows r = (query head h, token o) of a
      sequence, like observer rows; query head h reads KV head h // G.
  D2. Every row attends to all n live entries of its sequence (the tokens of one
      call are appended to the cache after it; no mask among the live entries).
  D3. Logits are scale * <q_r, k_j> with the caller's scale; the LSE is natural.
  D4. The tally for the eviction scores is s_j += sum over the rows of the entry's
      KV group of p_rj, p_rj = exp(logit_rj - LSE_r) -- the same quantity the
      observer scorer computes from a given LSE.

Precision: fp64 from the exact stored bf16 values.
"""
from __future__ import annotations

import numpy as np

from .kvs_oracle import bf16_bits_to_f64, gather_stream_rows


def attend_stream(q_rows: np.ndarray, keys: np.ndarray, values: np.ndarray, scale: float):
    """(out [R][D], lse [R], p [R][n]) of rows q_rows over one stream's entries.

    logit_rj = scale <q_r, k_j>;  LSE_r = ln sum_j exp(logit_rj);
    p_rj = exp(logit_rj - LSE_r);  out_r = sum_j p_rj v_j.
    """
    logits = float(scale) * (q_rows @ keys.T)                      # [R][n]
    m = logits.max(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(np.exp(logits - m).sum(axis=1))
    p = np.exp(logits - lse[:, None])
    return p @ values, lse, p


def decode_attention(k_pool, v_pool, q, tok_off, block_table, start, length, num_q_heads, scale,
                     streams=None):
    """Every (or the listed) stream (i, l, g): dict -> (out [G*T][D], lse [G*T], tally [n]).

    q: bf16 bits [L][Hq][T_tot][D]; tokens of sequence i are rows tok_off[i]..tok_off[i+1].
    Rows of a stream are ordered head-major (h = gG .. gG+G-1, then token).
    """
    L, _, Hkv = k_pool.shape[:3]
    G = num_q_heads // Hkv
    out = {}
    todo = streams if streams is not None else [
        (i, l, g) for i in range(len(length)) for l in range(L) for g in range(Hkv)]
    for (i, l, g) in todo:
        n = int(length[i])
        t0, t1 = int(tok_off[i]), int(tok_off[i + 1])
        rows = np.concatenate([bf16_bits_to_f64(q[l, h, t0:t1]) for h in range(g * G, (g + 1) * G)], axis=0)
        if n == 0 or rows.shape[0] == 0:
            out[(i, l, g)] = (np.zeros((rows.shape[0], q.shape[-1])), np.full(rows.shape[0], -np.inf),
                              np.zeros(n))
            continue
        keys = bf16_bits_to_f64(gather_stream_rows(k_pool, l, g, block_table[i], start[i], n))
        vals = bf16_bits_to_f64(gather_stream_rows(v_pool, l, g, block_table[i], start[i], n))
        o, lse, p = attend_stream(rows, keys, vals, scale)
        out[(i, l, g)] = (o, lse, p.sum(axis=0))
    return out
