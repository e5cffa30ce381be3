"""GPU parity of beacon k-means (kvs_beacon_kmeans through the C ABI) against the
oracle.

The assignment is taken in fp32 on the GPU and in fp64 by the oracle, so where two
groups are nearly equidistant either choice is correct: a GPU choice passes when its
exact score is within the GPU's error bound of the exact minimum.  The bound: ||c||^2
is a sum of 128 fp32 squares (error <= 128 u ||c||^2, u = 2^-24); <x, c> is a sum of
256 exact bf16 products (the centroid in two bf16 parts, residual <= 2^-17 |c|)
accumulated in fp32, so its error is <= (2^-17 + 257 u) |x| |c| <= 2.3e-5 |x| |c|;
two scores are compared, so tol = 2 (128 u max||c||^2 + 2 2.3e-5 |x| max|c|), taken
here as 1e-4 (max||c||^2 + |x| max|c|).

Given the GPU's assignments, the update is compared with the oracle's plain member mean
(exact, rounded once to fp32).  The GPU sums the members exactly as integers on the
2^-32 grid, which holds every bf16 value with |x| >= 2^-25 exactly, and rounds the
quotient exactly: wherever no member coordinate lies in 0 < |x| < 2^-25 the centroid
must match bit for bit.  Elsewhere each such member is truncated toward zero by less
than 2^-32, so the mean moves by less than 2^-32 and the rounded centroids differ by at
most that plus one fp32 spacing of the result.
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


TINY = 2.0 ** -25


def check_update(x, a, c_prev, c_gpu, err_msg=""):
    """The GPU's centroids against the oracle's plain means of the GPU's assignments:
    bit for bit where no member coordinate is in (0, 2^-25); within 2^-32 plus one fp32
    spacing elsewhere.  Returns the number of (group, dim) pairs held to the bound."""
    want = KO.update(x, a, c_prev)
    tiny = (np.abs(x) > 0) & (np.abs(x) < TINY)
    loose = np.zeros(want.shape, bool)
    for k in range(want.shape[0]):
        m = a == k
        if m.any():
            loose[k] = tiny[m].any(axis=0)
    np.testing.assert_array_equal(c_gpu[~loose], want[~loose], err_msg=err_msg)
    if loose.any():
        w = want[loose].astype(np.float64)
        tol = 2.0 ** -32 + np.spacing(np.abs(want[loose])).astype(np.float64)
        assert np.all(np.abs(c_gpu[loose].astype(np.float64) - w) <= tol), err_msg
    return int(loose.sum())


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
            check_update(x[p], a[p], c[p], c_new[p], err_msg=f"iter {it} problem {p}")
        np.testing.assert_array_equal(bcn, KO.to_bf16_bits(c_new))
        c = c_new
    c6, a6, _ = run(xb, c0, 6)
    np.testing.assert_array_equal(c6, c)
    np.testing.assert_array_equal(a6, a)


@pytest.mark.parametrize("N", [16384, 16400])
def test_kmeans_long_histories(N):
    # up to 16 384 points, iterations after the first carry the integer sums and correct
    # them by the points that moved; beyond that every iteration sums afresh.  Both must
    # give the chain of single iterations, each checked against the oracle's update
    rng = np.random.default_rng(N)
    P, K = 1, 16
    xb = WB.normal_history(rng, P, N)
    x = bf16_bits_to_f64(xb)
    c0 = np.stack([x[p, WB.initial_rows(rng, N, K)] for p in range(P)]).astype(np.float32)
    print(f"kmeans long history N={N}", flush=True)
    c = c0
    for it in range(3):
        c_new, a, _ = run(xb, c, 1)
        check_assignment(x[0], c[0], a[0])
        check_update(x[0], a[0], c[0], c_new[0], err_msg=f"iter {it}")
        c = c_new
    c3, a3, _ = run(xb, c0, 3)
    np.testing.assert_array_equal(c3, c)
    np.testing.assert_array_equal(a3, a)


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


def _midpoint_count(xv, want):
    """How many exact member means sit exactly halfway between two fp32 values."""
    from fractions import Fraction
    n = 0
    for d in range(xv.shape[1]):
        exact = sum(Fraction(float(v)) for v in xv[:, d]) / xv.shape[0]
        w = want[d]
        for nb in (np.nextafter(w, np.float32(-np.inf)), np.nextafter(w, np.float32(np.inf))):
            n += int(exact == (Fraction(float(w)) + Fraction(float(nb))) / 2)
    return n


def test_kmeans_update_rounding_cases():
    # one group per problem (k = 1) with 2, 3 or 4 members of mixed magnitudes: the means
    # need the exact quotient, and many of them sit halfway between two fp32 values
    # (ties to even)
    rng = np.random.default_rng(8)
    P = 256
    for N in (2, 3, 4):
        mant = 1.0 + rng.integers(0, 128, (P, N, 128)) / 128.0
        expo = rng.integers(-24, 3, (P, N, 128)).astype(np.float64)
        x = rng.choice([-1.0, 1.0], (P, N, 128)) * mant * 2.0 ** expo
        x[: P // 2, N - 1] = x[: P // 2, 0]          # half the problems: a repeated member
        xb = WB.f64_to_bf16_bits(x)
        xv = bf16_bits_to_f64(xb)
        c0 = np.zeros((P, 1, 128), np.float32)
        print(f"kmeans update rounding cases N={N}", flush=True)
        c, a, _ = run(xb, c0, 1)
        assert np.all(a == 0)
        ties = 0
        for p in range(P):
            want = KO.update(xv[p], a[p], c0[p])
            np.testing.assert_array_equal(c[p], want, err_msg=f"N {N} problem {p}")
            if p < 16:
                ties += _midpoint_count(xv[p], want[0])
        assert N == 2 or ties > 0, N


def test_kmeans_tiny_coordinates_within_bound():
    # coordinates in (0, 2^-25) are truncated on the GPU's 2^-32 grid: held to the bound
    rng = np.random.default_rng(10)
    P, N, K = 2, 700, 4
    x = rng.standard_normal((P, N, 128))
    pick = rng.random((P, N, 128)) < 0.05
    x[pick] = rng.choice([-1.0, 1.0], pick.sum()) * 2.0 ** rng.uniform(-60, -25.5, pick.sum())
    xb = WB.f64_to_bf16_bits(x)
    xv = bf16_bits_to_f64(xb)
    c0 = np.stack([xv[p, :K] for p in range(P)]).astype(np.float32)
    print("kmeans tiny coordinates", flush=True)
    c, a, _ = run(xb, c0, 1)
    loose = 0
    for p in range(P):
        check_assignment(xv[p], c0[p], a[p])
        loose += check_update(xv[p], a[p], c0[p], c[p])
    assert loose > 0


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


def seed(xb, u):
    import torch
    K = _K()
    dev = torch.device("cuda", 0)
    P, N, _ = xb.shape
    pts = torch.from_numpy(xb.view(np.int16)).to(dev)
    uu = torch.from_numpy(np.ascontiguousarray(u, np.float32)).to(dev)
    cent = torch.full((P, u.shape[1], 128), float("nan"), dtype=torch.float32, device=dev)
    rows = torch.full((P, u.shape[1]), -1, dtype=torch.int32, device=dev)
    K.kvs_beacon_seed(pts, uu, cent, rows=rows)
    torch.cuda.synchronize()
    return cent.cpu().numpy(), rows.cpu().numpy()


# fp32 running sums of up to 16 384 squared distances: the target u * sum can move
# across a row boundary by the sums' rounding, at most about n u_32 of the total
SEED_RTOL = 3e-4


@pytest.mark.parametrize("N,K", [(16384, 5), (4096, 16), (1000, 7), (300, 16), (17, 4), (1, 3)])
def test_seed_draws_are_valid_kmeanspp_steps(N, K):
    # every draw, given the GPU's earlier rows, is a valid inverse-CDF draw of the
    # oracle's fp64 D2; the centroids are the drawn rows exactly; most draws equal the
    # oracle's own
    rng = np.random.default_rng(N * 7 + K)
    P = 3
    xb = WB.normal_history(rng, P, N)
    x = bf16_bits_to_f64(xb)
    u = rng.random((P, K)).astype(np.float32)
    print(f"kmeans++ seed N={N} K={K}", flush=True)
    cent, rows = seed(xb, u)
    same = 0
    for p in range(P):
        assert rows[p, 0] == KO.seed_index(u[p, 0], N)
        for c in range(1, K):
            assert KO.seed_step_valid(x[p], rows[p, :c], u[p, c], int(rows[p, c]), SEED_RTOL), (p, c)
        np.testing.assert_array_equal(cent[p], x[p, rows[p]].astype(np.float32))
        same += int(np.array_equal(rows[p], KO.kmeanspp(x[p], u[p])[1]))
    assert same >= P - 1


def test_seed_degenerate_rows():
    # every row equal: D2 is 0 after the first draw, so each draw is floor(u n); a
    # history with duplicated rows never draws a row already chosen while D2 > 0
    rng = np.random.default_rng(9)
    xb = np.repeat(WB.normal_history(rng, 1, 1), 64, axis=1)
    u = np.array([[0.05, 0.5, 0.99, 0.0]], np.float32)
    cent, rows = seed(xb, u)
    np.testing.assert_array_equal(rows[0], [3, 32, 63, 0])
    yb = np.concatenate([WB.normal_history(rng, 1, 8)] * 20, axis=1)       # 160 rows, 8 distinct
    u2 = rng.random((1, 8)).astype(np.float32)
    _, rows2 = seed(yb, u2)
    distinct = {tuple(yb[0, r]) for r in rows2[0]}
    assert len(distinct) == 8


def test_seed_then_lloyd_matches_oracle_on_separated_groups():
    # seeding and 10 Lloyd iterations on separated groups: the draws match the oracle's
    # and so does the whole run
    rng = np.random.default_rng(12)
    xs, _ = zip(*[WB.grouped_history(rng, 2000, 16, spread=6.0, noise=0.2) for _ in range(2)])
    xb = np.stack(xs)
    x = bf16_bits_to_f64(xb)
    u = rng.random((2, 16)).astype(np.float32)
    cent, rows = seed(xb, u)
    for p in range(2):
        c_ref, r_ref = KO.kmeanspp(x[p], u[p])
        np.testing.assert_array_equal(rows[p], r_ref)
        np.testing.assert_array_equal(cent[p], c_ref)
    c, a, _ = run(xb, cent, 10)
    for p in range(2):
        cw, aw = KO.lloyd(x[p], cent[p], 10)
        np.testing.assert_array_equal(a[p], aw)
        np.testing.assert_array_equal(c[p], cw)
