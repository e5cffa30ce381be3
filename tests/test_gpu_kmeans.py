"""GPU parity of beacon k-means (kvs_beacon_kmeans through the C ABI) against the
oracle.

The assignment is taken in fp32 on the GPU and in fp64 by the oracle, so where two
groups are nearly equidistant either choice is correct: a GPU choice passes when its
exact score is within the GPU's error bound of the exact minimum.  The bound: ||c||^2
is a sum of 128 fp32 squares (error <= 128 u ||c||^2, u = 2^-24); <x, c> is a sum of
256 exact bf16 products (the centroid in two bf16 parts, residual <= 2^-17 |c|)
accumulated in fp32, so its error is <= (2^-17 + 257 u) |x| |c| <= 2.3e-5 |x| |c|;
two scores are compared, so tol = 2 (128 u max||c||^2 + 2 2.3e-5 |x| max|c|), taken
here as 1e-4 (max||c||^2 + |x| max|c|).  Given the GPU's assignments the update is integer
arithmetic and a defined rounding sequence: the centroids must match bit for bit.
"""
import numpy as np
import pytest

from oracle import kmeans_oracle as KO
from workloads import beacons as WB
from workloads.logits import bf16_bits_to_f64

pytestmark = pytest.mark.gpu


def _K():
    import kv_cache_eviction_lse_amd as K
    return K


def run(xb, c0, iters, sentinel=-7):
    """xb: bf16 bits [P][N][128]; c0: fp32 [P][K][128] -> (centroids, assign, beacons)."""
    import torch
    K = _K()
    dev = torch.device("cuda", 0)
    P, N, _ = xb.shape
    pts = torch.from_numpy(xb.view(np.int16)).to(dev)
    cent = torch.from_numpy(np.ascontiguousarray(c0, np.float32)).to(dev)
    asg = torch.full((P, N), sentinel, dtype=torch.int32, device=dev)
    bcn = torch.zeros((P, c0.shape[1], 128), dtype=torch.int16, device=dev)
    K.kvs_beacon_kmeans(pts, cent, iters, assign=asg, beacons=bcn)
    torch.cuda.synchronize()
    return cent.cpu().numpy(), asg.cpu().numpy(), bcn.cpu().numpy().view(np.uint16)


def check_assignment(x, c, a):
    _, sc = KO.assign(x, c)
    cc = c.astype(np.float64)
    cmax = np.sqrt((cc * cc).sum(1)).max()
    tol = 1e-4 * (cmax ** 2 + np.sqrt((x * x).sum(1)) * cmax)
    got = sc[np.arange(len(a)), a]
    assert np.all(got <= sc.min(axis=1) + tol), float(np.max(got - sc.min(axis=1) - tol))
    return int(np.sum(a != np.argmin(sc, axis=1)))


@pytest.mark.parametrize("N,K", [(4096, 16), (1000, 7), (37, 16), (16, 1), (5, 3)])
def test_kmeans_chained_iterations(N, K):
    # iteration by iteration: each assignment is a valid argmin and each update matches
    # the oracle's update of the GPU's assignments bit for bit; then one call of 6
    # iterations equals the chain
    rng = np.random.default_rng(N * 31 + K)
    P = 3
    xb = WB.normal_history(rng, P, N)
    x = bf16_bits_to_f64(xb)
    c0 = np.stack([x[p, WB.initial_rows(rng, N, K)] for p in range(P)]).astype(np.float32)
    print(f"kmeans chained N={N} K={K}", flush=True)
    c = c0
    for it in range(6):
        c_new, a, bcn = run(xb, c, 1)
        for p in range(P):
            check_assignment(x[p], c[p], a[p])
            np.testing.assert_array_equal(c_new[p], KO.update(x[p], a[p], c[p]), err_msg=f"iter {it} problem {p}")
        np.testing.assert_array_equal(bcn, KO.to_bf16_bits(c_new))
        c = c_new
    c6, a6, _ = run(xb, c0, 6)
    np.testing.assert_array_equal(c6, c)
    np.testing.assert_array_equal(a6, a)


def test_kmeans_separated_groups_match_oracle_exactly():
    # well separated groups: no near ties, so the whole run (assignments and centroids
    # after 10 iterations) equals the oracle's
    rng = np.random.default_rng(5)
    P, N, K = 4, 3000, 16
    xs, labs = zip(*[WB.grouped_history(rng, N, K) for _ in range(P)])
    xb = np.stack(xs)
    x = bf16_bits_to_f64(xb)
    c0 = np.stack([x[p, [int(np.nonzero(labs[p] == k)[0][-1]) for k in range(K)]] for p in range(P)])
    c0 = c0.astype(np.float32)
    print("kmeans separated groups", flush=True)
    c, a, bcn = run(xb, c0, 10)
    for p in range(P):
        cw, aw = KO.lloyd(x[p], c0[p], 10)
        np.testing.assert_array_equal(a[p], aw)
        np.testing.assert_array_equal(a[p], labs[p])
        np.testing.assert_array_equal(c[p], cw)
    np.testing.assert_array_equal(bcn, KO.to_bf16_bits(c))


def test_kmeans_zero_iterations_and_empty_groups():
    # iters = 0 leaves the centroids and the assignments alone; a group far from every
    # point keeps its centroid
    rng = np.random.default_rng(6)
    xb = WB.normal_history(rng, 2, 200)
    x = bf16_bits_to_f64(xb)
    c0 = np.stack([x[p, :4] for p in range(2)]).astype(np.float32)
    c0[:, 3] = 500.0
    c, a, bcn = run(xb, c0, 0)
    np.testing.assert_array_equal(c, c0)
    assert np.all(a == -7)
    np.testing.assert_array_equal(bcn, KO.to_bf16_bits(c0))
    c, a, _ = run(xb, c0, 3)
    np.testing.assert_array_equal(c[:, 3], c0[:, 3])
    assert not np.any(a == 3)
