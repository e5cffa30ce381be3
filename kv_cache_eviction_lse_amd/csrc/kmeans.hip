// kvs_beacon_kmeans: Lloyd k-means over each (layer, query head)'s history queries,
// for beacon queries.
//
// BeaconKV Compresses KV Cache for Long-Reasoning Models with Beacon Queries, Key
// ideas: queries that revisit distant context fall into a few similarity groups, and
// one representative per group (a beacon) is kept beside the recent queries.  The
// groups are found here by Lloyd's k-means from given initial centroids:
//   assignment  a_i = argmin_k ||c_k||^2 - 2 <x_i, c_k>   (ties to the lower k);
//   update      c_kd = the mean of the members' coordinates, rounded once to fp32
//               (nearest, ties to even); an empty group keeps its centroid.
// The member sums are exact int64 sums of the coordinates on the 2^-32 grid
// (trunc(x 2^32), exact for every bf16 value with |x| >= 2^-25, and |x| < 2^15), so
// they do not depend on the members' order, and the quotient sum / n_k is rounded
// exactly from those integers.  A coordinate 0 < |x| < 2^-25 is truncated toward zero
// on the grid, which moves the mean by less than 2^-32.
//
// One 512-thread workgroup per problem keeps the centroids in LDS for all iterations;
// two workgroups share a CU (at most 128 VGPRs).
// Per 16-point tile a wave computes the 16 x 16 block of <c_k, x_i> on
// v_mfma_f32_16x16x32_bf16 with the centroids on M (each fp32 centroid split into two
// bf16 parts, 16 significant bits; the points are exact bf16) and the points on N (each lane
// loads 16 bytes of one point row per slice), takes the argmin, then adds the tile's
// points to their groups' integer sums with LDS 64-bit atomics (lane = two dimensions;
// the rows come back from the cache that just served the MFMA operands).  The next
// tile's rows are loaded while a tile is processed.  From the second iteration on, the
// integer sums are carried over and corrected by the points that changed group only.  Member counts
// stay in registers (lane k counts group k) until the end of the iteration.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kKmMaxK = 16;
constexpr int kKmThreads = 512;
constexpr int kKmWaves = kKmThreads / 64;
// Up to this many points per problem, iterations after the first update the integer
// sums by the points that changed group only (their previous groups are kept in LDS).
constexpr int kKmDeltaMaxN = 16384;
// Points per problem: the int64 grid sums stay below 2^63 for |x| < 2^15.
constexpr int kKmMaxN = 65536;

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float kfloatx4;

struct KmArgs {
  const uint16_t *x;       // bf16 [P][N][128]
  float *cent;             // fp32 [P][K][128]: initial in, final out
  int32_t *assign;         // int32 [P][N] or null
  uint16_t *beacons;       // bf16 [P][K][128] or null
  int32_t N, K, T;
};

__device__ __forceinline__ uint16_t bf16_rn(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// trunc(x 2^32) of a bf16 value x (bit pattern h) with |x| < 2^15, as an exact integer
// (|result| < 2^47): the 8-bit significand shifted to the 2^-32 grid, truncated toward
// zero below it (subnormal bf16 values are below 2^-126, so they give 0).
__device__ __forceinline__ long long bf16_grid32(uint32_t h) {
  const int32_t e = (int32_t)((h >> 7) & 0xFFu);
  const uint64_t sig = (uint64_t)(0x80u | (h & 0x7Fu));
  const int32_t sh = e - 102;                       // value = sig 2^(e - 134) = sig 2^sh 2^-32
  uint64_t v;
  if (e == 0) v = 0;
  else if (sh >= 0) v = sig << (sh < 40 ? sh : 40);
  else v = sh > -8 ? sig >> (-sh) : 0;
  return (h & 0x8000u) ? -(long long)v : (long long)v;
}

// Sign of T - m n 2^32 for a double m with at most 25 significant bits (the product is
// exact: at most 42 bits).
__device__ __forceinline__ int cmp_scaled(uint64_t T, uint32_t n, double m) {
  const double v = m * (double)n * 0x1p32;
  if (v >= 0x1p63) return -1;                       // T < 2^63
  const double fl = floor(v);
  const uint64_t vi = (uint64_t)fl;                 // exact
  if (T != vi) return T > vi ? 1 : -1;
  return v > fl ? -1 : 0;
}

// fp32(S 2^-32 / n), rounded to nearest with ties to even, exactly, for |S| < 2^63 and
// 1 <= n <= 2^16.  A double quotient lands within one fp32 step of the exact value; the
// midpoints to both neighbours are then compared with S exactly in integers.
__device__ __forceinline__ float grid_mean_rn(long long S, uint32_t n) {
  if (S == 0) return 0.f;
  const uint64_t T = S < 0 ? 0ull - (uint64_t)S : (uint64_t)S;
  float f = (float)((double)T / (double)n * 0x1p-32);   // >= 2^-48, a normal number
  const uint32_t fb = __float_as_uint(f);
  const float up = __uint_as_float(fb + 1u), dn = __uint_as_float(fb - 1u);
  const int hi = cmp_scaled(T, n, 0.5 * ((double)f + (double)up));
  if (hi > 0 || (hi == 0 && (fb & 1u))) {
    f = up;
  } else {
    const int lo = cmp_scaled(T, n, 0.5 * ((double)dn + (double)f));
    if (lo < 0 || (lo == 0 && (fb & 1u))) f = dn;
  }
  return S < 0 ? -f : f;
}

__device__ __forceinline__ float km_wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__global__ __launch_bounds__(kKmThreads, 4) void kmeans_kernel(KmArgs a) {
  __shared__ float c_lds[kKmMaxK][kHeadDim];
  __shared__ float cn_lds[kKmMaxK];
  __shared__ unsigned long long sum_lds[kKmMaxK][kHeadDim];
  __shared__ uint32_t cnt_lds[kKmMaxK];
  __shared__ uint8_t prev_lds[kKmDeltaMaxN];      // each point's group in the previous iteration

  const int64_t p = blockIdx.x;
  const int32_t N = a.N, K = a.K;
  const uint16_t *xp = a.x + p * (int64_t)N * kHeadDim;
  float *cp = a.cent + p * (int64_t)K * kHeadDim;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int blk = lane >> 4, n16 = lane & 15;
  for (int e = tid; e < kKmMaxK * kHeadDim; e += kKmThreads) {
    const int k = e / kHeadDim, d = e % kHeadDim;
    c_lds[k][d] = k < K ? cp[k * kHeadDim + d] : 0.f;
  }
  const int32_t ntiles = (N + 15) / 16;

  for (int32_t t = 0; t < a.T; ++t) {
    // The sums are exact integers, so they can be carried from one iteration to the next
    // and corrected by the points that moved (subtracted from the old group, added to the
    // new): the same integers as summing all members afresh.
    const bool delta = t > 0 && N <= kKmDeltaMaxN;
    if (!delta) {
      for (int e = tid; e < kKmMaxK * kHeadDim; e += kKmThreads) sum_lds[e / kHeadDim][e % kHeadDim] = 0ull;
      if (tid < kKmMaxK) cnt_lds[tid] = 0u;
    }
    __syncthreads();                                   // c_lds (initial or updated) visible
    // ||c_k||^2: wave w takes groups 2w, 2w + 1 (groups beyond K score +inf)
#pragma unroll
    for (int q = 0; q < kKmMaxK / kKmWaves; ++q) {
      const int k = (kKmMaxK / kKmWaves) * wave + q;
      const float v0 = c_lds[k][2 * lane], v1 = c_lds[k][2 * lane + 1];
      const float s = km_wave_sum(__builtin_fmaf(v1, v1, v0 * v0));
      if (lane == 0) cn_lds[k] = k < K ? s : __builtin_inff();
    }
    // MFMA A operands: lane (group n16, block blk) holds dims 32 sl + 8 blk .. + 7 of its
    // group's centroid as hi + lo bf16 parts (|c - hi - lo| <= 2^-17 |c|)
    bf16x8 ah[4], al[4];
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = c_lds[n16][32 * sl + 8 * blk + e];
        const uint16_t h = bf16_rn(c);
        const uint16_t lo = bf16_rn(c - bf16_f(h));
        ah[sl][e] = __builtin_bit_cast(__bf16, h);
        al[sl][e] = __builtin_bit_cast(__bf16, lo);
      }
    }
    __syncthreads();                                   // cn_lds visible
    float cn4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cn4[i] = cn_lds[4 * blk + i];

    uint32_t cnt_reg = 0;   // lane k < 16: change of group k's member count seen by this wave (mod 2^32)
    // B operands: lane (point n16, block blk) loads dims 32 sl + 8 blk .. + 7; then the
    // tile's rows again, lane = dims 2 lane, 2 lane + 1 (for the update).
    // A tile of 16 whole rows starting at base <= N - 16: one address, rows at offsets.
    auto load_full = [&](int32_t base, bf16x8 (&b)[4], uint32_t (&rw)[16]) {
      const uint16_t *xr = xp + (int64_t)(base + n16) * kHeadDim + 8 * blk;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) b[sl] = *(const bf16x8 *)(xr + 32 * sl);
      const uint32_t *rr = (const uint32_t *)(xp + (int64_t)base * kHeadDim) + lane;
#pragma unroll
      for (int q = 0; q < 16; ++q) rw[q] = rr[q * (kHeadDim / 2)];
    };
    // The last, partial tile: rows past the end are clamped to row N - 1 (and not added).
    auto load_tail = [&](int32_t base, bf16x8 (&b)[4], uint32_t (&rw)[16]) {
      const int32_t pc = min(base + n16, N - 1);
      const uint16_t *xr = xp + (int64_t)pc * kHeadDim + 8 * blk;
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) b[sl] = *(const bf16x8 *)(xr + 32 * sl);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int32_t pq = min(base + q, N - 1);
        rw[q] = ((const uint32_t *)(xp + (int64_t)pq * kHeadDim))[lane];
      }
    };
    auto process = [&](int32_t base, const bf16x8 (&b)[4], const uint32_t (&rw)[16]) {
      kfloatx4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[sl], b[sl], d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[sl], b[sl], d, 0, 0, 0);
      }
      // lane (point n16, blk) holds <c_k, x> for k = 4 blk + i: argmin, then across the
      // four blocks (lanes n16 + 16 j); ties to the lower group
      float best = cn4[0] - 2.f * d[0];
      int bi = 4 * blk;
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        const float sc = cn4[i] - 2.f * d[i];
        if (sc < best) {
          best = sc;
          bi = 4 * blk + i;
        }
      }
#pragma unroll
      for (int msk = 16; msk <= 32; msk <<= 1) {
        const float ob = __shfl_xor(best, msk);
        const int oi = __shfl_xor(bi, msk);
        if (ob < best || (ob == best && oi < bi)) {
          best = ob;
          bi = oi;
        }
      }
      if (t == a.T - 1 && a.assign && blk == 0 && base + n16 < N) a.assign[p * N + base + n16] = bi;
      // previous groups of the tile's points (read before this wave overwrites them)
      int prev = 0;
      if (N <= kKmDeltaMaxN) {
        const bool live = base + n16 < N;
        if (delta) prev = live ? prev_lds[base + n16] : 0;
        if (blk == 0 && live) prev_lds[base + n16] = (uint8_t)bi;
      }
      // exact integer sums of the members on the 2^-32 grid (|sum| < 2^47 N <= 2^63)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (base + q < N) {
          const int aq = __builtin_amdgcn_readlane(bi, q);
          const int pq = delta ? __builtin_amdgcn_readlane(prev, q) : -1;
          if (aq != pq) {
            const long long v0 = bf16_grid32(rw[q] & 0xFFFFu);
            const long long v1 = bf16_grid32(rw[q] >> 16);
            atomicAdd(&sum_lds[aq][2 * lane], (unsigned long long)v0);
            atomicAdd(&sum_lds[aq][2 * lane + 1], (unsigned long long)v1);
            cnt_reg += lane == aq ? 1u : 0u;
            if (pq >= 0) {
              atomicAdd(&sum_lds[pq][2 * lane], (unsigned long long)(-v0));
              atomicAdd(&sum_lds[pq][2 * lane + 1], (unsigned long long)(-v1));
              cnt_reg -= lane == pq ? 1u : 0u;
            }
          }
        }
      }
    };
    // Whole tiles, the next tile's loads issued before this one is processed (the last
    // whole tile of a wave loads itself again instead, from the cache); then the partial
    // tile, if any.
    const int32_t nfull = N / 16;
    int32_t tile = wave;
    bf16x8 b0[4];
    uint32_t rw0[16];
    if (tile < nfull) {
      load_full(tile * 16, b0, rw0);
      for (; tile < nfull; tile += kKmWaves) {
        bf16x8 b1[4];
        uint32_t rw1[16];
        const int32_t next = tile + kKmWaves < nfull ? tile + kKmWaves : tile;
        load_full(next * 16, b1, rw1);
        process(tile * 16, b0, rw0);
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) b0[sl] = b1[sl];
#pragma unroll
        for (int q = 0; q < 16; ++q) rw0[q] = rw1[q];
      }
    }
    for (; tile < ntiles; tile += kKmWaves) {
      load_tail(tile * 16, b0, rw0);
      process(tile * 16, b0, rw0);
    }
    if (lane < kKmMaxK && cnt_reg) atomicAdd(&cnt_lds[lane], cnt_reg);
    __syncthreads();                                   // every sum and count in
    for (int e = tid; e < K * kHeadDim; e += kKmThreads) {
      const int k = e / kHeadDim, d = e % kHeadDim;
      const uint32_t cnt = cnt_lds[k];
      if (cnt) c_lds[k][d] = grid_mean_rn((long long)sum_lds[k][d], cnt);
    }
    __syncthreads();                                   // sums read before the next iteration clears them
  }
  for (int e = tid; e < K * kHeadDim; e += kKmThreads) {
    const float c = c_lds[e / kHeadDim][e % kHeadDim];
    cp[e] = c;
    if (a.beacons) a.beacons[p * (int64_t)K * kHeadDim + e] = bf16_rn(c);
  }
}

// ---- k-means++ seeding ----
//
// The initial centroids: row floor(u_0 n); then, with D2_i the squared distance from row
// i to its nearest chosen centroid, the first row (in row order) whose running sum of D2
// exceeds u_c sum(D2) -- a draw with probability D2_i / sum(D2) by inverting the
// cumulative sum -- or floor(u_c n) when every D2 is 0.  The uniforms are inputs.  One
// 256-thread workgroup per problem: D2 lives in LDS; per round every thread takes whole
// rows (fp32 sums of squares) for the newest centroid, then per-thread runs of D2 in row
// order, a block scan and a block minimum find the drawn row.
constexpr int kSeedThreads = 256;
constexpr int kSeedMaxN = 16384;

struct SeedArgs {
  const uint16_t *x;       // bf16 [P][N][128]
  const float *u;          // [P][K] uniforms in [0, 1)
  float *cent;             // fp32 [P][K][128]
  int32_t *rows;           // int32 [P][K] or null
  int32_t N, K;
};

__device__ __forceinline__ int32_t seed_row(float u, int32_t n) {
  const double v = u >= 0.f ? (double)u * (double)n : 0.0;   // (a NaN outside the contract: row 0)
  return v < (double)(n - 1) ? (int32_t)floor(v) : n - 1;
}

__global__ __launch_bounds__(kSeedThreads) void kmeanspp_kernel(SeedArgs a) {
  __shared__ float d2[kSeedMaxN];
  __shared__ __attribute__((aligned(16))) float cen[kHeadDim];
  __shared__ float wtot[kSeedThreads / 64];
  __shared__ int32_t wred[2][kSeedThreads / 64];
  const int64_t p = blockIdx.x;
  const int32_t N = a.N, K = a.K;
  const uint16_t *xp = a.x + p * (int64_t)N * kHeadDim;
  const float *up = a.u + p * K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t per = (N + kSeedThreads - 1) / kSeedThreads;
  const int32_t j0 = min(tid * per, N), j1 = min(j0 + per, N);
  int32_t row = seed_row(up[0], N);
  for (int32_t c = 0; c < K; ++c) {
    __syncthreads();                                   // the previous round is done with cen
    if (tid < kHeadDim) {
      const float v = bf16_f(xp[(int64_t)row * kHeadDim + tid]);
      cen[tid] = v;
      a.cent[(p * K + c) * kHeadDim + tid] = v;
    }
    if (tid == 0 && a.rows) a.rows[p * K + c] = row;
    if (c == K - 1) break;
    __syncthreads();
    for (int32_t j = tid; j < N; j += kSeedThreads) {
      const uint4 *xr = (const uint4 *)(xp + (int64_t)j * kHeadDim);
      float acc = 0.f;
#pragma unroll 4
      for (int q = 0; q < kHeadDim / 8; ++q) {
        const uint4 w = xr[q];
        const float4 c0 = *(const float4 *)&cen[8 * q], c1 = *(const float4 *)&cen[8 * q + 4];
        const float t[8] = {__uint_as_float(w.x << 16) - c0.x, __uint_as_float(w.x & 0xFFFF0000u) - c0.y,
                            __uint_as_float(w.y << 16) - c0.z, __uint_as_float(w.y & 0xFFFF0000u) - c0.w,
                            __uint_as_float(w.z << 16) - c1.x, __uint_as_float(w.z & 0xFFFF0000u) - c1.y,
                            __uint_as_float(w.w << 16) - c1.z, __uint_as_float(w.w & 0xFFFF0000u) - c1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(t[e], t[e], acc);
      }
      d2[j] = c == 0 ? acc : fminf(d2[j], acc);
    }
    __syncthreads();
    // running sums in row order: thread t owns rows j0 .. j1 - 1
    float part = 0.f;
    for (int32_t j = j0; j < j1; ++j) part += d2[j];
    float incl = part;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    float before = 0.f, total = 0.f;
#pragma unroll
    for (int w = 0; w < kSeedThreads / 64; ++w) {
      before += w < wave ? wtot[w] : 0.f;
      total += wtot[w];
    }
    const float un = up[c + 1];
    int32_t next;
    if (!(total > 0.f)) {
      next = seed_row(un, N);
    } else {
      const float target = un * total;
      int32_t cand = INT32_MAX, last = -1;
      float run = before + (incl - part);
      for (int32_t j = j0; j < j1; ++j) {
        const float v = d2[j];
        run += v;
        if (v > 0.f) {
          last = j;
          if (cand == INT32_MAX && run > target) cand = j;
        }
      }
      // the first candidate row of the block (else the last row with D2 > 0)
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        cand = min(cand, __shfl_xor(cand, o));
        last = max(last, __shfl_xor(last, o));
      }
      if (lane == 0) {
        wred[0][wave] = cand;
        wred[1][wave] = last;
      }
      __syncthreads();
      cand = INT32_MAX;
      last = -1;
#pragma unroll
      for (int w = 0; w < kSeedThreads / 64; ++w) {
        cand = min(cand, wred[0][w]);
        last = max(last, wred[1][w]);
      }
      next = cand != INT32_MAX ? cand : last;
    }
    row = next;
  }
}

}  // namespace

hipError_t launch_kmeans(const uint16_t *points, int64_t P, int32_t N, int32_t K, int32_t T, float *centroids,
                         int32_t *assign, uint16_t *beacons, hipStream_t st) {
  if (P == 0) return hipSuccess;
  KmArgs a{};
  a.x = points;
  a.cent = centroids;
  a.assign = assign;
  a.beacons = beacons;
  a.N = N;
  a.K = K;
  a.T = T;
  kmeans_kernel<<<dim3((unsigned)P), kKmThreads, 0, st>>>(a);
  return hipGetLastError();
}

int32_t kmeans_max_k() { return kKmMaxK; }
int32_t kmeans_max_points() { return kKmMaxN; }
int32_t kmeans_seed_max_points() { return kSeedMaxN; }

hipError_t launch_kmeanspp(const uint16_t *points, int64_t P, int32_t N, int32_t K, const float *uniforms,
                           float *centroids, int32_t *rows, hipStream_t st) {
  if (P == 0) return hipSuccess;
  SeedArgs a{};
  a.x = points;
  a.u = uniforms;
  a.cent = centroids;
  a.rows = rows;
  a.N = N;
  a.K = K;
  kmeanspp_kernel<<<dim3((unsigned)P), kSeedThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
