// kvs_token_confidence kernels: per decode step, the mean negative log-probability
// of the step's k most probable tokens.
//
// ActKV Dissected, Component 2: hesitation is read from the output distribution of
// each step through its top-20 tokens.  With z the step's logits over the
// vocabulary, p = softmax(z) and T the k largest logits,
//     conf = (1/k) sum_{j in T} -ln p_j = LSE(z) - mean_{j in T} z_j
//          = ln S + (1/k) sum_{j in T} (M - z_j),   M = max z,  S = sum_j exp(z_j - M).
//
// Rows are cut into chunks of 64 KiB of logits (32 768 bf16 or 16 384 fp32) when
// k <= 32, else 32 KiB, one per 256-thread workgroup, held in 64 (32) VGPRs per
// thread; workgroups are small so that several share a CU and one's barriers overlap
// the others' loads.  Per chunk:
//   * the maximum M and S = sum exp(z - M): per-thread maxima and sums, the sums
//     rescaled to M and added over the block;
//   * the k-th largest of the 256 per-thread maxima, M_k: each wave sorts its 64
//     maxima (bitonic, in registers), and each of the first k of every sorted list is
//     ranked against the first k of the other lists; the one of rank k is M_k;
//   * at least k values are >= M_k (one per thread whose maximum is >= M_k), and
//     values > M_k only occur in the at most k-1 threads whose maximum is > M_k,
//     so at most (k-1) x (logits per thread) <= 4 032 of them exist: they are
//     appended to an LDS list;
//   * if there are k or more, each is ranked among them (value, then position);
//     otherwise the rest of the top k are copies of M_k.
// A second kernel merges the chunks of a row: M = max M_c, S = sum S_c exp(M_c - M),
// and the top k of the chunks' top-k lists.  Reading and reduction orders are fixed,
// so results are deterministic.
#include "kvs_device.h"

#include <mutex>
#include <vector>

namespace kvs {
namespace {

constexpr int kConfThreads = 256;
constexpr int kConfWaves = kConfThreads / 64;
// Words (u32) of logits per thread: 64 while k <= 32, else 32 (the candidate list of a
// chunk, at most (k-1) x logits per thread, then still fits its 4 032 entries).
constexpr int kConfWordsSmallK = 64, kConfWordsLargeK = 32, kConfSmallK = 32;
constexpr int kConfMaxK = 64;
constexpr int kCandCap = (kConfMaxK - 1) * 64;               // values above M_k, at most
constexpr int kCombineThreads = 256;
constexpr int kConfMaxChunks = 128;                          // vocabularies up to 2^20 (fp32 chunks)
constexpr int kConfWavesPerSimd = 6;                         // occupancy the kernel is compiled for
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <bool BF16, int W> constexpr int conf_per() { return BF16 ? 2 * W : W; }   // logits per thread
template <bool BF16, int W> constexpr int conf_chunk() { return kConfThreads * conf_per<BF16, W>(); }

struct ConfArgs {
  const void *logits;
  int64_t rows;
  int64_t vocab;
  int64_t stride;    // elements between rows
  int64_t total;     // rows * chunks
  int32_t k;
  int32_t chunks;    // per row
  float *conf;       // [rows], written directly when chunks == 1
  float *part;       // [rows][chunks][2 + k]: M, S, then the chunk's top k values
};

struct ConfShared {
  alignas(16) uint32_t sorted[kConfWaves][64];   // each wave's thread maxima (keys), descending
  alignas(16) uint32_t cand[kCandCap];           // read 4 at a time: capacity a multiple of 4
  float topv[kConfMaxK];
  float ws[kConfWaves];                          // each wave's sum of exp(z - M)
  uint32_t mk;
  uint32_t ncand;
};
static_assert(kCandCap % 4 == 0, "candidate list read 4 at a time");

// Wave sum of a float, result in lane 63 (DPP row shifts and broadcasts, no LDS).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xF, false));
}
__device__ __forceinline__ float wave_sum_dpp_f32(float x) {
  x = dpp_add<kRowShr1, 0xF>(x);
  x = dpp_add<kRowShr2, 0xF>(x);
  x = dpp_add<kRowShr4, 0xF>(x);
  x = dpp_add<kRowShr8, 0xF>(x);
  x = dpp_add<kRowBcast15, 0xA>(x);
  x = dpp_add<kRowBcast31, 0xC>(x);
  return x;
}

// Order-preserving map of fp32 bit patterns to unsigned keys (NaN excluded).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Value of lane (lane ^ MASK).  Masks below 32 use ds_swizzle in bit-mask mode (the
// pattern is an immediate: no address register); 32 uses ds_bpermute with the
// partner address recomputed from the lane id.
template <int MASK>
__device__ __forceinline__ uint32_t xshfl(uint32_t v) {
  if constexpr (MASK < 32) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (MASK << 10) | 0x1F);
  } else {
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    return (uint32_t)__builtin_amdgcn_ds_bpermute((lane ^ MASK) << 2, (int)v);
  }
}
template <int MASK>
__device__ __forceinline__ float xshfl_f(float v) { return __uint_as_float(xshfl<MASK>(__float_as_uint(v))); }

__device__ __forceinline__ float wave_sum_f32(float x) {
  x += xshfl_f<32>(x);
  x += xshfl_f<16>(x);
  x += xshfl_f<8>(x);
  x += xshfl_f<4>(x);
  x += xshfl_f<2>(x);
  x += xshfl_f<1>(x);
  return x;
}

// Workgroup barrier that waits for this wave's LDS operations only: vector loads of
// the next chunk stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A copy of the thread index the compiler cannot see through: index arithmetic is
// then recomputed where it is used instead of being hoisted out of the chunk loop
// and kept live (or spilled) across it.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

// Logit i of this thread from a buffer of 32 words (bf16 pairs or fp32).
template <bool BF16, int W>
__device__ __forceinline__ float logit(const uint32_t (&w)[W], int i) {
  const uint32_t x = w[BF16 ? (i >> 1) : i];
  if (BF16) return __uint_as_float((i & 1) ? (x & 0xFFFF0000u) : (x << 16));
  return __uint_as_float(x);
}

// The buffer's words pass through an empty asm (in place, no instructions), so that
// each pass over the buffer unpacks it again instead of keeping 64 unpacked values
// (and their keys) live from one pass to the next.
template <int W>
__device__ __forceinline__ void fence_words(uint32_t (&w)[W]) {
#pragma unroll
  for (int i = 0; i < W; ++i) asm volatile("" : "+v"(w[i]));
}

// Number of valid logits in chunk cidx (>= 1; < chunk size only in a row's last chunk).
template <bool BF16, int W>
__device__ __forceinline__ int32_t conf_nvalid(const ConfArgs &a, int64_t cidx) {
  constexpr int CH = conf_chunk<BF16, W>();
  const int64_t row = cidx / a.chunks;
  const int64_t rem = a.vocab - (cidx - row * a.chunks) * CH;
  return (int32_t)(rem < CH ? rem : CH);
}

// Issue the loads of chunk `cidx` (row-major over (row, chunk)) into w.  Every load is
// at an index clamped into the chunk's valid range, so no load depends on a branch and
// nothing here waits on the data; conf_mask replaces the out-of-range positions.
// VEC (rows 16-byte aligned and the vocabulary a multiple of the vector width):
// 16-byte vector u of thread t holds logits (u * T + t) * per-vector, T the workgroup
// size, and whole vectors are either valid or not.  Otherwise word i holds logits
// 2i * T + t and (2i+1) * T + t (bf16), or logit i * T + t (fp32).
template <bool BF16, bool VEC, int W>
__device__ __forceinline__ void conf_load(const ConfArgs &a, int64_t cidx, uint32_t (&w)[W]) {
  constexpr int CH = conf_chunk<BF16, W>();
  const int t = opaque_tid();
  const int64_t row = cidx / a.chunks;
  const int64_t c0 = (cidx - row * a.chunks) * CH;
  const int32_t nvalid = conf_nvalid<BF16, W>(a, cidx);
  if (VEC) {
    constexpr int EPV = BF16 ? 8 : 4;                           // logits per vector
    const uint4 *src = (const uint4 *)((const uint8_t *)a.logits + (row * a.stride + c0) * (BF16 ? 2 : 4));
    const int32_t last = nvalid / EPV - 1;                        // vocab % EPV == 0
#pragma unroll
    for (int u = 0; u < W / 4; ++u) {
      const int32_t vi = u * kConfThreads + t;
      const uint4 v = src[vi < last ? vi : last];
      w[4 * u] = v.x;
      w[4 * u + 1] = v.y;
      w[4 * u + 2] = v.z;
      w[4 * u + 3] = v.w;
    }
  } else if (BF16) {
    const uint16_t *src = (const uint16_t *)a.logits + row * a.stride + c0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const int32_t e0 = 2 * i * kConfThreads + t, e1 = e0 + kConfThreads;
      const uint32_t lo = src[e0 < nvalid ? e0 : nvalid - 1], hi = src[e1 < nvalid ? e1 : nvalid - 1];
      w[i] = lo | (hi << 16);
    }
  } else {
    const uint32_t *src = (const uint32_t *)a.logits + row * a.stride + c0;
#pragma unroll
    for (int i = 0; i < W; ++i) {
      const int32_t e = i * kConfThreads + t;
      w[i] = src[e < nvalid ? e : nvalid - 1];
    }
  }
}

// Set the positions of a partial chunk that lie past the row end to -inf.
template <bool BF16, bool VEC, int W>
__device__ __forceinline__ void conf_mask(int32_t nvalid, uint32_t (&w)[W]) {
  const int t = opaque_tid();
#pragma unroll
  for (int i = 0; i < W; ++i) {
    if (VEC) {
      constexpr int EPV = BF16 ? 8 : 4;
      const int32_t vi = (i / 4) * kConfThreads + t;
      if (vi >= nvalid / EPV) w[i] = BF16 ? 0xFF80FF80u : 0xFF800000u;
    } else if (BF16) {
      const int32_t e0 = 2 * i * kConfThreads + t, e1 = e0 + kConfThreads;
      if (e0 >= nvalid) w[i] = (w[i] & 0xFFFF0000u) | 0xFF80u;
      if (e1 >= nvalid) w[i] = (w[i] & 0x0000FFFFu) | 0xFF800000u;
    } else {
      if (i * kConfThreads + t >= nvalid) w[i] = 0xFF800000u;
    }
  }
}

// Reduce one chunk held in w and write its result.
template <bool BF16, bool VEC, int W>
__device__ __forceinline__ void conf_reduce(const ConfArgs &a, int64_t cidx, uint32_t (&w)[W],
                                            ConfShared &sh) {
  constexpr int PER = conf_per<BF16, W>();
  {
    const int32_t nvalid = conf_nvalid<BF16, W>(a, cidx);
    if (nvalid < conf_chunk<BF16, W>()) conf_mask<BF16, VEC, W>(nvalid, w);   // uniform branch
  }
  const float NEG = -__builtin_inff();
  const int t = opaque_tid(), lane = t & 63, wave = t >> 6;
  const int k = a.k;
  if (t == 0) sh.ncand = 0;

  // ---- per-thread maximum (three-input max over unpacked pairs) ----
  fence_words(w);
  float tmax = NEG;
#pragma unroll
  for (int i = 0; i < PER; i += 2) {
    tmax = __builtin_fmaxf(tmax, __builtin_fmaxf(logit<BF16, W>(w, i), logit<BF16, W>(w, i + 1)));
    if ((i & 7) == 6) __builtin_amdgcn_sched_barrier(0);
  }
  const uint32_t tkey = fkey(tmax);
  // ---- sort the wave's 64 thread maxima, descending (bitonic, in registers) ----
  uint32_t v = tkey;
  auto cx = [&](uint32_t o, int size, int j) {
    const bool desc_block = (lane & size) == 0;     // blocks alternate; the last is whole
    const bool lower = (lane & j) == 0;
    v = (desc_block == lower) ? max(v, o) : min(v, o);
  };
  cx(xshfl<1>(v), 2, 1);
  cx(xshfl<2>(v), 4, 2);
  cx(xshfl<1>(v), 4, 1);
  cx(xshfl<4>(v), 8, 4);
  cx(xshfl<2>(v), 8, 2);
  cx(xshfl<1>(v), 8, 1);
  cx(xshfl<8>(v), 16, 8);
  cx(xshfl<4>(v), 16, 4);
  cx(xshfl<2>(v), 16, 2);
  cx(xshfl<1>(v), 16, 1);
  cx(xshfl<16>(v), 32, 16);
  cx(xshfl<8>(v), 32, 8);
  cx(xshfl<4>(v), 32, 4);
  cx(xshfl<2>(v), 32, 2);
  cx(xshfl<1>(v), 32, 1);
  cx(xshfl<32>(v), 64, 32);
  cx(xshfl<16>(v), 64, 16);
  cx(xshfl<8>(v), 64, 8);
  cx(xshfl<4>(v), 64, 4);
  cx(xshfl<2>(v), 64, 2);
  cx(xshfl<1>(v), 64, 1);
  sh.sorted[wave][lane] = v;
  // ---- per-thread sum of exp(z - tmax) (one FMA per logit: c = tmax log2 e is rounded
  // once, which scales every term of this thread by the same factor, within
  // 2^-24 |tmax| log2 e of 1), overlapping the barrier wait ----
  fence_words(w);
  float tsum = 0.f;
  if (tmax != NEG) {
    const float c = tmax * kLog2e;
    auto term = [&](int i) { return __builtin_amdgcn_exp2f(__builtin_fmaf(logit<BF16, W>(w, i), kLog2e, -c)); };
    float t0 = term(0), t1 = term(1), t2 = term(2), t3 = term(3);
#pragma unroll
    for (int i = 4; i < PER; i += 4) {
      t0 += term(i);
      t1 += term(i + 1);
      t2 += term(i + 2);
      t3 += term(i + 3);
      if ((i & 7) == 4) __builtin_amdgcn_sched_barrier(0);
    }
    tsum = (t0 + t1) + (t2 + t3);
  }
  lds_barrier();

  // ---- M, each wave's sum rescaled to M; M_k = the key of rank k among the maxima ----
  uint32_t mkey = 0;
#pragma unroll
  for (int q = 0; q < kConfWaves; ++q) mkey = max(mkey, sh.sorted[q][0]);
  const float M = key_f(mkey);
  {
    const float r = tmax != NEG ? tsum * __builtin_amdgcn_exp2f((tmax - M) * kLog2e) : 0.f;
    const float ws = wave_sum_dpp_f32(r);
    if (lane == 63) sh.ws[wave] = ws;
  }
  if (t < kConfWaves * k) {
    // order: key descending, then list, then position in the list; only the first k
    // of a list can rank below k, so only those are compared
    const int lw = t / k, p = t - lw * k;
    const uint32_t key = sh.sorted[lw][p];
    int rank = p;
    for (int q = 0; q < kConfWaves; ++q) {
      if (q == lw) continue;
      const uint32_t *lq = sh.sorted[q];
      const bool ge = q < lw;
      for (int j = 0; j < k; j += 4) {
        const uint4 x4 = *(const uint4 *)(lq + j);
        const uint32_t xs[4] = {x4.x, x4.y, x4.z, x4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          rank += (j + e < k && (xs[e] > key || (ge && xs[e] == key))) ? 1 : 0;
      }
    }
    if (rank == k - 1) sh.mk = key;
  }
  lds_barrier();
  const uint32_t mk = sh.mk;

  // ---- values above M_k (at most (k-1) * PER of them) appended to the LDS list;
  // only the at most k-1 threads whose maximum is above M_k hold any ----
  fence_words(w);
  if (tkey > mk) {
    // Count this thread's values above M_k, reserve that many slots with one LDS
    // atomic, then write them (an atomic per value, each waiting for its slot index,
    // cost more than the rest of the chunk).  A thread with one such value holds only
    // its maximum, which it writes without a second pass.  The compare is on floats:
    // it differs from the key order only in placing +0 level with a -0 M_k, and both
    // add the same zero to the sum of the k largest.
    const float fmk = key_f(mk);
    uint32_t n = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      n += logit<BF16, W>(w, i) > fmk ? 1u : 0u;
      if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);
    }
    if (n == 1) {
      sh.cand[atomicAdd(&sh.ncand, 1u)] = tkey;
    } else {
      uint32_t at = atomicAdd(&sh.ncand, n);
      fence_words(w);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const float x = logit<BF16, W>(w, i);
        if (x > fmk) sh.cand[at++] = fkey(x);
        if ((i & 7) == 7) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  lds_barrier();
  // the list's order depends on atomic order; ranks break ties by position, so the
  // chosen values (and their sum) do not.  Reads take 4 entries at a time (the list
  // capacity is a multiple of 4; entries past nc are masked).
  // The chunk's k largest are written in descending order: every candidate is ranked
  // (ranks below k land in topv[rank]); with fewer than k candidates the rest are
  // copies of M_k, which is below all of them.
  const int nc = (int)sh.ncand;
  {
    for (int i = t; i < nc; i += kConfThreads) {
      const uint32_t ki = sh.cand[i];
      int rank = 0;
      for (int j = 0; j < nc; j += 4) {
        const uint4 c4 = *(const uint4 *)(sh.cand + j);
        const uint32_t cs[4] = {c4.x, c4.y, c4.z, c4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t kj = cs[e];
          rank += (j + e < nc && (kj > ki || (kj == ki && j + e < i))) ? 1 : 0;
        }
      }
      if (rank < k) sh.topv[rank] = key_f(ki);
    }
    if (t >= nc && t < k) sh.topv[t] = key_f(mk);
  }
  lds_barrier();

  // ---- result (wave 0) ----
  if (wave == 0) {
    float S = 0.f;
#pragma unroll
    for (int q = 0; q < kConfWaves; ++q) S += sh.ws[q];
    const float tv = lane < k ? sh.topv[lane] : 0.f;
    if (a.chunks == 1) {
      const float d = wave_sum_f32(lane < k ? M - tv : 0.f);
      if (lane == 0) a.conf[cidx] = __builtin_amdgcn_logf(S) * kLn2 + d / (float)k;
    } else {
      float *p = a.part + cidx * (int64_t)(2 + k);
      if (lane == 0) {
        p[0] = M;
        p[1] = S;
      }
      if (lane < k) p[2 + lane] = tv;
    }
  }
}

// One chunk per workgroup.
template <bool BF16, bool VEC, int W>
__global__ __launch_bounds__(kConfThreads, kConfWavesPerSimd) void conf_chunk_kernel(ConfArgs a) {
  __shared__ ConfShared sh;
  const int64_t c = blockIdx.x;
  if (c >= a.total) return;
  uint32_t w[W];
  conf_load<BF16, VEC, W>(a, c, w);
  conf_reduce<BF16, VEC, W>(a, c, w, sh);
}

// Block sum of a float in wave order (deterministic).  scratch: one float per wave.
__device__ __forceinline__ float block_sum_f32(float x, float *scratch) {
  x = wave_sum_f32(x);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[wave] = x;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += scratch[w];
  __syncthreads();
  return t;
}

// Wave maximum of a u32, uniform result (DPP row shifts and broadcasts).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr1, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr2, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr4, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr8, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast15, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast31, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

constexpr int kMergeChunks = 64;   // chunks per row the one-wave merge takes

// Merge the chunks of one row with one wave (rows of at most 64 chunks).  Each chunk's
// k values are stored in descending order, so the row's k largest are taken by k
// rounds of "largest current head": lane c holds the head of chunk c's list, the wave
// maximum picks the next value, and the lowest lane holding it advances.
__global__ __launch_bounds__(64) void conf_merge_kernel(ConfArgs a) {
  __shared__ float L[kMergeChunks * (2 + kConfMaxK)];
  const int64_t row = blockIdx.x;
  if (row >= a.rows) return;
  const int lane = threadIdx.x;
  const int k = a.k, C = a.chunks;
  const int w = 2 + k;
  const float *p = a.part + row * (int64_t)C * w;
  for (int i = lane; i < C * w; i += 64) L[i] = p[i];
  __builtin_amdgcn_s_waitcnt(0);     // the wave's own LDS writes, before its reads
  const bool live = lane < C;
  const float mc = live ? L[lane * w] : -__builtin_inff();
  const float M = key_f(wave_max_u32(fkey(mc)));
  const float sc = (live && mc != -__builtin_inff()) ? L[lane * w + 1] * __builtin_amdgcn_exp2f((mc - M) * kLog2e) : 0.f;
  const float S = wave_sum_f32(sc);
  int h = 0;
  uint32_t head = live ? fkey(L[lane * w + 2]) : 0u;
  float d = 0.f;
  for (int r = 0; r < k; ++r) {
    const uint32_t mx = wave_max_u32(head);
    const uint64_t hit = __ballot(head == mx);
    const int winner = __ffsll((long long)hit) - 1;
    d += M - key_f(mx);
    if (lane == winner) {
      ++h;
      head = h < k ? fkey(L[lane * w + 2 + h]) : 0u;
    }
  }
  if (lane == 0) a.conf[row] = __builtin_amdgcn_logf(S) * kLn2 + d / (float)k;
}

// Merge the chunks of one row (one workgroup per row; rows of more than 64 chunks).
__global__ __launch_bounds__(kCombineThreads) void conf_combine_kernel(ConfArgs a) {
  __shared__ float red[kCombineThreads / 64];
  __shared__ float topv[kConfMaxK];
  __shared__ uint32_t keys[kConfMaxChunks * kConfMaxK];
  const int64_t row = blockIdx.x;
  if (row >= a.rows) return;
  const int t = threadIdx.x;
  const int k = a.k;
  const int C = a.chunks;
  const int64_t w = 2 + k;
  const float *p = a.part + row * C * w;
  const float NEG = -__builtin_inff();
  // M over the chunks (every thread reads the C maxima)
  float M = NEG;
  for (int c = 0; c < C; ++c) M = fmaxf(M, p[c * w]);
  float s = 0.f;
  for (int c = t; c < C; c += kCombineThreads) {
    const float mc = p[c * w];
    s += mc != NEG ? p[c * w + 1] * __builtin_amdgcn_exp2f((mc - M) * kLog2e) : 0.f;
  }
  const float S = block_sum_f32(s, red);
  // the top k of the C*k chunk values, ranked by (value, position)
  const int n = C * k;
  for (int i = t; i < n; i += kCombineThreads) keys[i] = fkey(p[(i / k) * w + 2 + (i % k)]);
  __syncthreads();
  for (int i = t; i < n; i += kCombineThreads) {
    const uint32_t ki = keys[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const uint32_t kj = keys[j];
      rank += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
    }
    if (rank < k) topv[rank] = key_f(ki);
  }
  __syncthreads();
  if (t < 64) {
    const float d = wave_sum_f32(t < k ? M - topv[t] : 0.f);
    if (t == 0) a.conf[row] = __builtin_amdgcn_logf(S) * kLn2 + d / (float)k;
  }
}

}  // namespace

int64_t conf_max_vocab() { return (int64_t)1 << 20; }
int32_t conf_max_k() { return kConfMaxK; }

int32_t conf_chunks(int64_t vocab, bool bf16, int32_t k) {
  const bool small = k <= kConfSmallK;
  const int64_t ch = bf16 ? (small ? conf_chunk<true, kConfWordsSmallK>() : conf_chunk<true, kConfWordsLargeK>())
                          : (small ? conf_chunk<false, kConfWordsSmallK>() : conf_chunk<false, kConfWordsLargeK>());
  return (int32_t)((vocab + ch - 1) / ch);
}

// The workspace is sized for fp32 rows (the smaller chunk), which covers bf16 too.
size_t conf_workspace_bytes(int64_t rows, int64_t vocab, int32_t k) {
  const int32_t C = conf_chunks(vocab, false, k);
  if (C <= 1) return 0;
  return (size_t)rows * C * (2 + k) * sizeof(float);
}

// The library's own partial-result buffer, for callers that cannot allocate
// (kvs_token_confidence_static): one copy per GPU, held until the process ends.
static __device__ __align__(256) uint8_t scratch[kConfScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::vector<void *> g_scratch_ptr;     // per device: the address of that device's copy
}  // namespace

hipError_t conf_scratch(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    // the array's name is a host-side stand-in: its device address comes from the runtime,
    // once per device, with that device current
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_confidence(const void *logits, bool bf16, int64_t rows, int64_t vocab, int64_t stride,
                             int32_t k, float *conf, void *ws, hipStream_t st) {
  ConfArgs a{};
  a.logits = logits;
  a.rows = rows;
  a.vocab = vocab;
  a.stride = stride;
  a.k = k;
  a.chunks = conf_chunks(vocab, bf16, k);
  a.total = rows * a.chunks;
  a.conf = conf;
  a.part = (float *)ws;
  const size_t es = bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)logits % 16 == 0) && ((size_t)stride * es) % 16 == 0 &&
                   ((size_t)vocab * es) % 16 == 0;
  const unsigned grid = (unsigned)a.total;
  const bool small = k <= kConfSmallK;
  constexpr int WS = kConfWordsSmallK, WL = kConfWordsLargeK;
  if (bf16) {
    if (vec) {
      if (small) conf_chunk_kernel<true, true, WS><<<grid, kConfThreads, 0, st>>>(a);
      else conf_chunk_kernel<true, true, WL><<<grid, kConfThreads, 0, st>>>(a);
    } else {
      if (small) conf_chunk_kernel<true, false, WS><<<grid, kConfThreads, 0, st>>>(a);
      else conf_chunk_kernel<true, false, WL><<<grid, kConfThreads, 0, st>>>(a);
    }
  } else {
    if (vec) {
      if (small) conf_chunk_kernel<false, true, WS><<<grid, kConfThreads, 0, st>>>(a);
      else conf_chunk_kernel<false, true, WL><<<grid, kConfThreads, 0, st>>>(a);
    } else {
      if (small) conf_chunk_kernel<false, false, WS><<<grid, kConfThreads, 0, st>>>(a);
      else conf_chunk_kernel<false, false, WL><<<grid, kConfThreads, 0, st>>>(a);
    }
  }
  if (a.chunks > kMergeChunks) conf_combine_kernel<<<(unsigned)rows, kCombineThreads, 0, st>>>(a);
  else if (a.chunks > 1) conf_merge_kernel<<<(unsigned)rows, 64, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
