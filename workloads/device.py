"""Device-side filling of large synthetic workloads (test and benchmark plumbing).

Large pools (the 8B shape is 8.6 GB of K+V) are drawn on the GPU with torch's
seeded generator: N(0,1) keys and values, planted keys k = 3 q/|q| + z for a
Bernoulli(f) subset of slots, a prior CRF in [0, 2), and the log-sum-exp of every
observer row over its stream's live keys (fp32 logits, as a paged decode kernel
would produce it).  Streams listed in `exact_streams` are then overwritten with
the host generator's values (workloads.host) and their LSE rows recomputed in
fp64 on the host, so that the oracle and the GPU see identical bytes for them
without the host ever touching the device-drawn data.
"""
from __future__ import annotations

import numpy as np

from . import host as H
from .configs import Workload

PAGE = 16


def _bf16_dev(a: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)


class DeviceInputs:
    def __init__(self, k, v, crf, q, lse):
        self.k, self.v, self.crf, self.q, self.lse = k, v, crf, q, lse   # k, v, q: int16 storage of bf16


def fill(w: Workload, lay: H.Layout, q_host: np.ndarray, device, exact_streams=(),
         seed_offset: int = 0, exact_bytes=None) -> DeviceInputs:
    import torch
    L, Hkv, Hq, D = w.num_layers, w.num_kv_heads, w.num_q_heads, w.head_dim
    G = w.group
    P = lay.num_pages
    gen = torch.Generator(device=device)
    gen.manual_seed((w.key + seed_offset) & 0x7FFFFFFFFFFFFFFF)
    k = torch.empty((L, P, Hkv, PAGE, D), dtype=torch.bfloat16, device=device)
    v = torch.empty_like(k)
    for l in range(L):
        k[l] = torch.randn((P, Hkv, PAGE, D), generator=gen, device=device).to(torch.bfloat16)
        v[l] = torch.randn((P, Hkv, PAGE, D), generator=gen, device=device).to(torch.bfloat16)
    crf = torch.zeros((L, P, Hkv, PAGE), dtype=torch.float32, device=device)
    if w.prior_crf:
        crf.copy_(2.0 * torch.rand((L, P, Hkv, PAGE), generator=gen, device=device))
    q = _bf16_dev(q_host, device).view(torch.bfloat16)
    O_tot = q.shape[2]
    lse = torch.zeros((L, Hq, O_tot), dtype=torch.float32, device=device)
    scale = w.scale
    for i in range(w.num_seqs):
        n = int(lay.length[i])
        st = int(lay.start[i])
        o0, o1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
        O = o1 - o0
        if n == 0 or O == 0:
            continue
        pos = st + np.arange(n)
        page = torch.from_numpy(lay.block_table[i][pos // PAGE].astype(np.int64)).to(device)
        row = torch.from_numpy((pos % PAGE).astype(np.int64)).to(device)
        R = O * G
        for l in range(L):
            keys = k[l][page, :, row, :].float()                         # [n][Hkv][D]
            qr = q[l, :, o0:o1, :].float().reshape(Hkv, R, D)           # head-major rows per KV head
            if w.planted_frac > 0:
                pm = torch.rand((n, Hkv), generator=gen, device=device) < w.planted_frac
                r = torch.randint(0, R, (n, Hkv), generator=gen, device=device)
                qn = qr / qr.norm(dim=2, keepdim=True)
                gi = torch.arange(Hkv, device=device)[None, :].expand(n, Hkv)
                planted = 3.0 * qn[gi, r] + keys
                keys = torch.where(pm[:, :, None], planted, keys)
                k[l][page, :, row, :] = keys.to(torch.bfloat16)
                keys = k[l][page, :, row, :].float()
            kt = keys.permute(1, 2, 0).contiguous()                         # [Hkv][D][n]
            for r0 in range(0, R, 256):
                r1 = min(R, r0 + 256)
                logits = torch.bmm(qr[:, r0:r1, :].contiguous(), kt) * scale  # [Hkv][r][n] fp32
                lr = torch.logsumexp(logits, dim=2)                          # [Hkv][r]
                rows = torch.arange(r0, r1, device=device)
                hh = rows // O
                oo = rows % O
                for g in range(Hkv):
                    lse[l, g * G + hh, o0 + oo] = lr[g]
    out = DeviceInputs(k.view(torch.int16), v.view(torch.int16), crf, q.view(torch.int16), lse)
    for (i, l, g) in exact_streams:
        pre = exact_bytes.get((i, l, g)) if exact_bytes else None
        write_exact_stream(w, lay, q_host, out, i, l, g, device, pre)
    return out


def observer_lse(w: Workload, lay: H.Layout, d: DeviceInputs, q_host: np.ndarray, device,
                 exact_streams=(), exact_lse=None):
    """(q, lse) on the device for another observer set (bf16 bits q_host) over the
    cache's live keys: fp32 logits for every row, then the rows of `exact_streams`
    recomputed in fp64 on the host from their keys (read back: they are host bytes), or
    taken from exact_lse[stream] (the same fp64 rows, computed beforehand)."""
    import torch
    L, Hkv, Hq, D = w.num_layers, w.num_kv_heads, w.num_q_heads, w.head_dim
    G = w.group
    q = _bf16_dev(q_host, device).view(torch.bfloat16)
    lse = torch.zeros((L, Hq, q.shape[2]), dtype=torch.float32, device=device)
    kb16 = d.k.view(torch.bfloat16)
    for i in range(w.num_seqs):
        n, st = int(lay.length[i]), int(lay.start[i])
        o0, o1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
        O = o1 - o0
        if n == 0 or O == 0:
            continue
        pos = st + np.arange(n)
        page = torch.from_numpy(lay.block_table[i][pos // PAGE].astype(np.int64)).to(device)
        row = torch.from_numpy((pos % PAGE).astype(np.int64)).to(device)
        R = O * G
        for l in range(L):
            keys = kb16[l][page, :, row, :].float()
            qr = q[l, :, o0:o1, :].float().reshape(Hkv, R, D)
            lr = live_lse(keys, qr, w.scale)
            rows = torch.arange(R, device=device)
            for g in range(Hkv):
                lse[l, g * G + rows // O, o0 + rows % O] = lr[g]
    for (i, l, g) in exact_streams:
        if exact_lse is not None and (i, l, g) in exact_lse:
            lr = exact_lse[(i, l, g)]
        else:
            n, st = int(lay.length[i]), int(lay.start[i])
            pos = st + np.arange(n)
            page = torch.from_numpy(lay.block_table[i][pos // PAGE].astype(np.int64)).to(device)
            row = torch.from_numpy((pos % PAGE).astype(np.int64)).to(device)
            kb = d.k[l][page, g, row, :].cpu().numpy().view(np.uint16)
            lr = H.lse_rows(H.stream_observer_rows(w, lay, q_host, i, l, g), kb, w.scale)
        o0, o1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
        O = o1 - o0
        for hh in range(G):
            lse[l, g * G + hh, o0:o1] = torch.from_numpy(lr[hh * O:(hh + 1) * O].copy()).to(device)
    return q.view(torch.int16), lse


def host_stream_observers(w: Workload, lay: H.Layout, q_host0: np.ndarray, q_host: np.ndarray, streams):
    """(q, lse) of another observer set for the mini-pools of host_stream_inputs (same
    stream order and offsets): the LSE over each stream's host keys, fp64 rounded to
    fp32.  q_host0 is the measured round's observer set (it decides the planted keys)."""
    G = w.group
    Os = [int(lay.obs_off[i + 1] - lay.obs_off[i]) for (i, _, _) in streams]
    obs_off = np.zeros(len(streams) + 1, np.int64)
    obs_off[1:] = np.cumsum(Os)
    q = np.zeros((1, G, int(obs_off[-1]), w.head_dim), np.uint16)
    lse = np.zeros((1, G, int(obs_off[-1])), np.float32)
    for s, (i, l, g) in enumerate(streams):
        n = int(lay.length[i])
        tokens = lay.tok0[i] + np.arange(n)
        kb = H.stream_keys(w, H.stream_observer_rows(w, lay, q_host0, i, l, g), i, l, g, tokens)
        lr = H.lse_rows(H.stream_observer_rows(w, lay, q_host, i, l, g), kb, w.scale)
        o0, o1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
        O = o1 - o0
        for hh in range(G):
            q[0, hh, obs_off[s]:obs_off[s + 1]] = q_host[l, g * G + hh, o0:o1]
            lse[0, hh, obs_off[s]:obs_off[s + 1]] = lr[hh * O:(hh + 1) * O]
    return q, lse


def host_stream(w: Workload, lay: H.Layout, q_host: np.ndarray, i: int, l: int, g: int):
    """Host-generated K, V, prior CRF (logical slot order) and LSE rows of one stream."""
    n = int(lay.length[i])
    tokens = lay.tok0[i] + np.arange(n)
    qr = H.stream_observer_rows(w, lay, q_host, i, l, g)
    kb = H.stream_keys(w, qr, i, l, g, tokens)
    vb = H.stream_values(w, i, l, g, tokens)
    crf = H.stream_prior_crf(w, i, l, g, tokens) if w.prior_crf else np.zeros(n, np.float32)
    lr = H.lse_rows(qr, kb, w.scale) if (qr.shape[0] and n) else np.zeros(qr.shape[0], np.float32)
    return kb, vb, crf, lr


def mini_stream_bytes(mini, G: int):
    """(K rows, V rows, prior CRF, LSE rows) of the single stream of a host_stream_inputs
    mini-batch, in logical order: the same bytes host_stream returns."""
    k_pool, v_pool, crf_pool, q, lse, bt, start, length, obs_off = mini
    n, st = int(length[0]), int(start[0])
    pos = st + np.arange(n)
    pg, rw = bt[0][pos // PAGE], pos % PAGE
    lr = np.concatenate([lse[0, hh, obs_off[0]:obs_off[1]] for hh in range(G)])
    return k_pool[0, pg, 0, rw], v_pool[0, pg, 0, rw], crf_pool[0, pg, 0, rw], lr


def write_exact_stream(w: Workload, lay: H.Layout, q_host: np.ndarray, d: DeviceInputs,
                       i: int, l: int, g: int, device, pre=None) -> None:
    """Overwrite stream (i, l, g) with the host generator's bytes (pre: those bytes,
    already generated, as mini_stream_bytes returns them)."""
    import torch
    kb, vb, crf, lr = pre if pre is not None else host_stream(w, lay, q_host, i, l, g)
    n = int(lay.length[i])
    st = int(lay.start[i])
    pos = st + np.arange(n)
    page = torch.from_numpy(lay.block_table[i][pos // PAGE].astype(np.int64)).to(device)
    row = torch.from_numpy((pos % PAGE).astype(np.int64)).to(device)
    d.k[l][page, g, row, :] = torch.from_numpy(kb.view(np.int16)).to(device)
    d.v[l][page, g, row, :] = torch.from_numpy(vb.view(np.int16)).to(device)
    d.crf[l][page, g, row] = torch.from_numpy(crf).to(device)
    G = w.group
    o0, o1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
    O = o1 - o0
    for hh in range(G):
        d.lse[l, g * G + hh, o0:o1] = torch.from_numpy(lr[hh * O:(hh + 1) * O].copy()).to(device)


def host_stream_inputs(w: Workload, lay: H.Layout, q_host: np.ndarray, streams):
    """Mini-pools holding only the given streams, for the oracle.

    Returns (k_pool, v_pool, crf_pool, q, lse, block_table, start, length, obs_off,
    index) where stream s of the list becomes sequence s of a one-layer, one-head
    batch whose pages are numbered 0.. in logical order.
    """
    D = w.head_dim
    G = w.group
    S = len(streams)
    npg = [(int(lay.start[i]) + int(lay.length[i]) + PAGE - 1) // PAGE for (i, _, _) in streams]
    P = int(sum(npg))
    k_pool = np.zeros((1, P, 1, PAGE, D), np.uint16)
    v_pool = np.zeros((1, P, 1, PAGE, D), np.uint16)
    crf_pool = np.zeros((1, P, 1, PAGE), np.float32)
    mp = max(npg) if npg else 1
    bt = np.full((S, mp), -1, np.int32)
    Os = [int(lay.obs_off[i + 1] - lay.obs_off[i]) for (i, _, _) in streams]
    obs_off = np.zeros(S + 1, np.int64)
    obs_off[1:] = np.cumsum(Os)
    q = np.zeros((1, G, int(obs_off[-1]), D), np.uint16)
    lse = np.zeros((1, G, int(obs_off[-1])), np.float32)
    start = np.array([int(lay.start[i]) for (i, _, _) in streams], np.int32)
    length = np.array([int(lay.length[i]) for (i, _, _) in streams], np.int32)
    nxt = 0
    for s, (i, l, g) in enumerate(streams):
        kb, vb, crf, lr = host_stream(w, lay, q_host, i, l, g)
        bt[s, :npg[s]] = np.arange(nxt, nxt + npg[s])
        nxt += npg[s]
        pos = int(lay.start[i]) + np.arange(int(lay.length[i]))
        pg, rw = bt[s][pos // PAGE], pos % PAGE
        k_pool[0, pg, 0, rw] = kb
        v_pool[0, pg, 0, rw] = vb
        crf_pool[0, pg, 0, rw] = crf
        o0, o1 = int(lay.obs_off[i]), int(lay.obs_off[i + 1])
        O = o1 - o0
        for hh in range(G):
            q[0, hh, obs_off[s]:obs_off[s + 1]] = q_host[l, g * G + hh, o0:o1]
            lse[0, hh, obs_off[s]:obs_off[s + 1]] = lr[hh * O:(hh + 1) * O]
    return k_pool, v_pool, crf_pool, q, lse, bt, start, length, obs_off


def live_lse(keys_f32, q_rows_f32, scale, chunk=256):
    """Natural-log LSE of observer rows over live keys, fp32 logits as a paged decode
    kernel would produce them.  keys_f32: [n][Hkv][D]; q_rows_f32: [Hkv][R][D] with the
    rows of KV head g head-major.  Returns [Hkv][R] float32 (torch)."""
    import torch
    kt = keys_f32.permute(1, 2, 0).contiguous()                      # [Hkv][D][n]
    R = q_rows_f32.shape[1]
    out = torch.empty((q_rows_f32.shape[0], R), dtype=torch.float32, device=keys_f32.device)
    for r0 in range(0, R, chunk):
        r1 = min(R, r0 + chunk)
        logits = torch.bmm(q_rows_f32[:, r0:r1, :].contiguous(), kt) * scale
        out[:, r0:r1] = torch.logsumexp(logits, dim=2)
    return out
