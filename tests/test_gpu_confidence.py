"""GPU parity of the confidence monitor (kvs_token_confidence through the C ABI)
against the fp64 oracle on the same bytes, and of the trend flag built on it.

Tolerance.  conf = ln S + (1/k) sum (M - z_j) in fp32.  S is a sum of at most 2^20
terms exp(z - M) <= 1, each within a few ulp (2^(-24) relative) of exact plus the
rounding of its exponent (z - M) log2 e, which is at most 2^(-24) |z - M| log2 e in
absolute terms; the partial sums in a fixed tree add about (64 + 9 + 5) ulp.  For
logits of magnitude below 100 this bounds the error of ln S by about 2e-5, and the
top-k term adds a few ulp of values below 200: |conf - oracle| <= 5e-5 + 1e-6 |oracle|.
"""
import numpy as np
import pytest

from oracle import confidence as CO
from workloads import logits as LG

pytestmark = pytest.mark.gpu

ATOL, RTOL = 5e-5, 1e-6


def _K():
    import kv_cache_eviction_lse_amd as K
    return K


def gpu_conf(x_dev, k, vocab=None):
    import torch
    K = _K()
    rows = x_dev.shape[0]
    V = x_dev.shape[1] if vocab is None else vocab
    conf = torch.full((rows,), float("nan"), dtype=torch.float32, device=x_dev.device)
    ws_n = K.kvs_token_confidence_workspace_size(rows, V, k)
    ws = torch.empty(max(ws_n, 4), dtype=torch.uint8, device=x_dev.device)
    K.kvs_token_confidence(x_dev, conf, k=k, vocab=V, workspace=ws)
    torch.cuda.synchronize()
    return conf.cpu().numpy()


def device_rows(z32, dtype):
    """(device tensor, exact fp64 values of what the device holds)."""
    import torch
    if dtype == "bf16":
        bits = LG.to_bf16_bits(z32)
        t = torch.from_numpy(bits.view(np.int16)).to("cuda").view(torch.bfloat16)
        return t, LG.bf16_bits_to_f64(bits)
    t = torch.from_numpy(np.ascontiguousarray(z32, np.float32)).to("cuda")
    return t, z32.astype(np.float64)


def check(got, exact, k, tag):
    for r in range(exact.shape[0]):
        want = CO.token_confidence(exact[r], k)
        if np.isinf(want):
            assert np.isinf(got[r]) and got[r] > 0, (tag, r, got[r])
            continue
        assert abs(got[r] - want) <= ATOL + RTOL * abs(want), (tag, r, float(got[r]), want)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [64, 100, 4097, 32768, 32769, 65536, 128256, 151936])
@pytest.mark.parametrize("k", [1, 20, 64])
def test_confidence_parity(dtype, V, k):
    if k > V:
        pytest.skip("k > vocab")
    z = np.concatenate([LG.lm_rows(V * 3 + k, 5, V), LG.special_rows(V + k, V)])
    print(f"confidence parity dtype={dtype} V={V} k={k} rows={z.shape[0]}", flush=True)
    x, exact = device_rows(z, dtype)
    check(gpu_conf(x, k), exact, k, (dtype, V, k))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_confidence_strided_and_unaligned(dtype):
    # rows padded to a longer stride, and a view that starts one element in, so that
    # the rows are not 16-byte aligned (element-wise loads)
    import torch
    V, pad = 40000, 40007
    z = LG.lm_rows(5, 6, pad)
    x, exact = device_rows(z, dtype)
    print(f"confidence strided dtype={dtype}", flush=True)
    check(gpu_conf(x, 20, vocab=V), exact[:, :V], 20, "strided")
    xs = x[:, 1:V + 1]
    assert xs.stride(0) == pad and xs.stride(1) == 1
    check(gpu_conf(xs, 20, vocab=V), exact[:, 1:V + 1], 20, "unaligned")
    _ = torch


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_confidence_largest_vocabulary(dtype):
    # 2^20 logits: 64 bf16 chunks (one-wave merge) or 128 fp32 chunks (ranked merge)
    V = 1 << 20
    z = np.concatenate([LG.lm_rows(11, 2, V), LG.special_rows(12, V)[[0, 1, 3, 4]]])
    print(f"confidence V=2^20 {dtype}", flush=True)
    x, exact = device_rows(z, dtype)
    check(gpu_conf(x, 64), exact, 64, "2^20")
    check(gpu_conf(x, 20), exact, 20, "2^20")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("V", [4097, 32768])
def test_confidence_signed_zeros_at_the_kth(dtype, V):
    # rows whose k-th largest logit is a zero, with +0 and -0 spread over many threads
    # (the chunk kernel compares candidates against M_k as floats, where +0 and -0 are
    # level; both add the same zero to the top-k sum)
    rng = np.random.default_rng(11)
    rows = []
    for n_pos, n_pz, n_nz in [(0, 15, 15), (5, 10, 20), (0, 0, 25), (0, 25, 0), (19, 1, 1), (3, 40, 40)]:
        z = (-1.0 - 3.0 * rng.random(V)).astype(np.float32)
        pos = rng.choice(V, n_pos + n_pz + n_nz, replace=False)
        z[pos[:n_pos]] = (1.0 + rng.random(n_pos)).astype(np.float32)
        z[pos[n_pos:n_pos + n_pz]] = np.float32(0.0)
        z[pos[n_pos + n_pz:]] = np.float32(-0.0)
        rows.append(z)
    z = np.stack(rows)
    assert np.signbit(z).any() and (z == 0).sum() > 0
    print(f"confidence signed zeros dtype={dtype} V={V}", flush=True)
    x, exact = device_rows(z, dtype)
    check(gpu_conf(x, 20), exact, 20, ("zeros", dtype, V))
    check(gpu_conf(x, 1), exact, 1, ("zeros k=1", dtype, V))


def test_confidence_bench_shape_sampled():
    # the benchmark's shape (4096 steps x 128 256 bf16 logits, drawn on the device);
    # a sample of rows is read back and checked against the oracle
    import torch
    rows, V = 4096, LG.LLAMA3_VOCAB
    print("confidence bench shape", flush=True)
    x = LG.lm_rows_device(3, rows, V, "cuda", torch.bfloat16)
    conf = gpu_conf(x, 20)
    pick = np.random.default_rng(0).choice(rows, 24, replace=False)
    bits = x[torch.from_numpy(pick).to("cuda")].view(torch.int16).cpu().numpy().view(np.uint16)
    exact = LG.bf16_bits_to_f64(bits)
    check(conf[pick], exact, 20, "bench")
    assert np.all(np.isfinite(conf))


def test_trend_flag_on_gpu_confidence():
    # a decode trajectory of 1 024 steps: the GPU's per-step confidence, the library's
    # trend on it, and the oracle's trend on the same fp32 values decide the same flag
    K = _K()
    steps, V = 1024, 32000
    for declining in (True, False):
        # declining: sharpness 12 -> 6 with an early collapse; rising: 12 -> 16
        boost = LG.trajectory_boost(21 if declining else 22, steps, -6.0 if declining else 4.0,
                                    collapses=(100,) if declining else (40,))
        z = LG.lm_rows(23, steps, V, boost=boost)
        x, exact = device_rows(z, "bf16")
        print(f"trend declining={declining}", flush=True)
        conf = gpu_conf(x, 20)
        check(conf[::37], exact[::37], 20, "trajectory")
        t = K.kvs_confidence_trend(conf, 64, 8, 0)
        slope, P, flag = CO.trend_flag(conf.astype(np.float64), 64, 8, 0)
        assert t.flag == flag and len(t.pooled) == P == (steps - 64) // 8 + 1
        assert t.slope == pytest.approx(slope, rel=1e-12)
        assert t.flag == declining
