// Register-resident per-stream kernels: the attention-mass cut with the LRFU update,
// the top-B keep set, or both in one pass over the data.  One 1024-thread workgroup
// per stream; thread t holds the scores and CRF of slots u * 1024 + t (u < kRegU) in
// registers, so each input is read from memory once and every selection pass runs
// on registers.  Streams longer than kRegU * 1024 entries take the kernels of
// lrfu.hip and select.hip.
//
// ActKV Dissected, Component 1: hits are the shortest prefix of (s desc, slot asc)
// holding the mass fraction num/den of the stream's integer attention mass
// m = floor(s * 2^32); LRFU with lambda = 0.5 gives CRF <- fma(d, CRF, hit), the prior
// taken as 0 for entries appended since the previous round.  Summary / Results: a
// fixed entry budget per head keeps the first K = min(B, n) entries of
// (CRF desc, s desc, slot asc) -- or, for step-aware ranking, of (key desc, s desc,
// slot asc) with caller keys in place of the CRF.  Both orders compare fp32 bit patterns (values >= 0)
// and ties at a threshold go to the lowest slots, so the results are exact.
//
// Selection: radix search on the key bits below the candidates' common prefix (from
// the AND and OR of their keys), 12 bits per pass, with a 4096-bin LDS histogram of
// counts or of integer masses; the crossing bin is found with one block-wide scan.
#include "kvs_device.h"

namespace kvs {

constexpr int kRegU = 32;                                        // slots per thread
constexpr int32_t kRegMaxLen = kRegU * kStreamThreads;           // 32768 entries per stream
constexpr int kRegBtCap = (kRegMaxLen + 2 * kPage - 2) / kPage;  // pages of a stream (start < 16)
constexpr int kDigitBits = 12;
constexpr int kTieList = 512;   // CRF ties at the threshold ranked directly up to this many
#ifndef KVS_CRF_CHUNK
#define KVS_CRF_CHUNK 8
#endif
static_assert(kRegU % 8 == 0, "the 8-row load and CRF chunks tile the rows exactly");
constexpr int kBins = 1 << kDigitBits;

namespace {

struct StreamArgs {
  const float *scores;
  float *crf;
  uint8_t *hit;          // nullable
  const float *decay;
  const int32_t *n_prev;
  const int32_t *budget;
  uint8_t *keep;
  const float *keys;     // nullable: top-B keys per entry [L*Hkv][E] in place of the CRF
  Batch b;
  uint32_t num, den;
};

struct RegShared {
  uint64_t hist[kBins];
  uint64_t scratch[kStreamWaves];
  uint64_t found[3];
};

struct Sel {
  uint32_t key;     // v*
  uint64_t above;   // weight of candidates with key > v*
  uint64_t at;      // weight of candidates with key == v*
  uint64_t target;  // the target the search used
};

// Exclusive block-wide prefix sum of a u64 (thread order), and the block total.  One
// barrier pair.
__device__ __forceinline__ uint64_t block_excl_u64(uint64_t x, uint64_t *scratch, uint64_t &total) {
  const uint64_t incl = wave_scan_u64(x);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) scratch[wave] = incl;
  __syncthreads();
  // lane w < waves holds wave w's total; one wave scan gives every wave its offset
  const int lane = threadIdx.x & 63;
  const uint64_t wsc = wave_scan_u64(lane < kStreamWaves ? scratch[lane] : 0ull);
  __syncthreads();
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  auto lane_u64 = [&](int l) -> uint64_t {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)wsc, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(wsc >> 32), l);
    return ((uint64_t)hi << 32) | lo;
  };
  const uint64_t before = wv ? lane_u64(wv - 1) : 0ull;
  total = lane_u64(kStreamWaves - 1);
  return before + incl - x;
}

// A copy of x the compiler cannot see through: index arithmetic derived from it is
// recomputed where it is used instead of being kept live (and spilled) across the
// whole kernel (per-row masks and indices would otherwise be hoisted out of the
// pass loops).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Ranks of flagged slots in slot order (slot u * 1024 + t: row u, then thread t) with
// a handful of barriers: every wave counts its flags per row (ballots), one block scan
// over the (row, wave) counts in row-major order gives each (row, wave) its offset, and
// a lane adds the flags of the lower lanes of its wave.  take(u, rank) is called for
// every row u < rounds (rank is meaningful where bit u of fmask is set).  cnt must hold
// kRegU * kStreamWaves words of LDS that no other thread uses meanwhile.
template <typename F>
__device__ __forceinline__ void rank_flags(uint32_t fmask, int rounds, uint32_t *cnt, uint32_t *scratch, F take) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int u = 0; u < kRegU; ++u) {
    const uint64_t b = __ballot(u < rounds && ((fmask >> u) & 1u));
    if (lane == 0) cnt[u * kStreamWaves + wave] = (uint32_t)__popcll(b);
  }
  __syncthreads();
  static_assert(kRegU * kStreamWaves <= kStreamThreads, "one (row, wave) count per thread");
  const uint32_t v = threadIdx.x < kRegU * kStreamWaves ? cnt[threadIdx.x] : 0u;
  uint32_t tot;
  const uint32_t ex = block_exclusive_scan(v, tot, scratch);
  if (threadIdx.x < kRegU * kStreamWaves) cnt[threadIdx.x] = ex;
  __syncthreads();
  const uint32_t *mine = cnt + opaque(wave);
#pragma unroll
  for (int u = 0; u < kRegU; ++u) {
    if (u < rounds) {
      const uint64_t b = __ballot((fmask >> u) & 1u);
      take(u, mine[u * kStreamWaves] + (uint32_t)__popcll(b & lanemask_lt()));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();     // cnt is free again
}

// v* with weight(keys > v*) < target <= weight(keys >= v*) over the candidates
// (slot valid and cand(u)); key[u] holds the key of this thread's row u.  With CUT the
// target is ceil(num * W / den) for the candidates' total weight W, which the first
// pass yields (so W needs no pass of its own); otherwise it is `target`.  A target of
// 0 returns key ~0 and at = 0.
template <bool COUNT, bool CUT, typename CandF, typename WF>
__device__ __forceinline__ Sel reg_select(const uint32_t (&key)[kRegU], int cnt, CandF cand, WF weight_of,
                                          uint64_t target, uint32_t num, uint32_t den, uint32_t and_all,
                                          uint32_t or_all, RegShared &sh) {
  auto target_of = [&](uint64_t W) -> uint64_t {
    if constexpr (CUT) return (W / den) * num + ((W % den) * num + den - 1) / den;
    else return target;
  };
  Sel r;
  const uint32_t diff = and_all ^ or_all;
  if (diff == 0) {
    uint64_t w = 0;
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      if (u < cnt && cand(u)) w += COUNT ? 1ull : weight_of(key[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const uint64_t tot = block_sum_u64(w, sh.scratch);
    r.target = target_of(tot);
    r.key = r.target ? and_all : ~0u;
    r.above = 0;
    r.at = r.target ? tot : 0;
    return r;
  }
  int top = 31 - __clz(diff);
  uint32_t prefix = top == 31 ? 0u : (and_all & ~((2u << top) - 1u));
  uint64_t need = CUT ? 0 : target, above = 0, at = 0;
  r.target = need;
  bool first = CUT;
  while (top >= 0) {
    const int width = top + 1 < kDigitBits ? top + 1 : kDigitBits;
    const int lo = top - width + 1;
    const uint32_t nb = 1u << width;
    for (uint32_t b = threadIdx.x; b < nb; b += kStreamThreads) sh.hist[b] = 0;
    __syncthreads();
    const int hs = top + 1;
    const int cnt_p = opaque(cnt);
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      // (the weight of a key is pass-invariant; computing it from an opaque copy keeps
      // the compiler from hoisting all kRegU weights out of the pass loop)
      const uint32_t k = COUNT ? key[u] : (uint32_t)opaque((int)key[u]);
      const bool v = u < cnt_p && cand(u) && (hs >= 32 || (k >> hs) == (prefix >> hs));
      const uint32_t bin = (k >> lo) & (nb - 1u);
      if (COUNT) hist_add_count(sh.hist, v, bin);
      else hist_add_u64(sh.hist, v, bin, v ? weight_of(k) : 0ull);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // bins in descending order, 4 per thread; the exclusive scan is the weight of all
    // higher bins
    uint64_t h[4], ls = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = (int)nb - 1 - (4 * (int)threadIdx.x + q);
      h[q] = b >= 0 ? sh.hist[b] : 0ull;
      ls += h[q];
    }
    uint64_t tot;
    uint64_t acc = block_excl_u64(ls, sh.scratch, tot);
    if (first) {
      first = false;
      need = target_of(tot);
      r.target = need;
      if (need == 0) {
        r.key = ~0u;
        r.above = 0;
        r.at = 0;
        return r;
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int b = (int)nb - 1 - (4 * (int)threadIdx.x + q);
      if (b >= 0 && acc < need && need <= acc + h[q]) {
        sh.found[0] = (uint64_t)b;
        sh.found[1] = acc;
        sh.found[2] = h[q];
      }
      acc += h[q];
    }
    __syncthreads();
    const uint32_t b = (uint32_t)sh.found[0];
    const uint64_t a = sh.found[1];
    at = sh.found[2];
    __syncthreads();
    prefix |= b << lo;
    need -= a;
    above += a;
    top = lo - 1;
  }
  r.key = prefix;
  r.above = above;
  r.at = at;
  return r;
}

// Stores for slot rows: rows u < full exist in every thread (uniform branch); the
// partial row after them is predicated per lane.
#define KVS_FOR_VALID(u, ...)   \
  if ((u) < full) {             \
    __VA_ARGS__                 \
  } else if ((u) < cnt) {       \
    __VA_ARGS__                 \
  }

template <bool LRFU, bool SELECT>
__global__ __launch_bounds__(kStreamThreads) void stream_reg_kernel(StreamArgs a) {
  __shared__ int32_t bt_lds[kRegBtCap];
  __shared__ RegShared sh;
  __shared__ uint32_t flag_scratch[kStreamWaves];
  __shared__ __attribute__((aligned(16))) uint32_t tie_s[kTieList];
  __shared__ __attribute__((aligned(16))) int32_t tie_j[kTieList];
  __shared__ uint32_t tie_count;

  const int32_t i = blockIdx.y;
  const int32_t lg = blockIdx.x;
  const int32_t n = a.b.len[i];
  if (n <= 0) return;
  const int32_t l = lg / a.b.Hkv;
  const int32_t g = lg - l * a.b.Hkv;
  const int64_t e0 = a.b.entry_off[i];
  const int32_t start = a.b.start[i];
  const int32_t tid = threadIdx.x;
  const int cnt = tid < n ? (n - tid + kStreamThreads - 1) / kStreamThreads : 0;   // rows of this thread
  const int full = n / kStreamThreads;                                              // rows of every thread
  const int rounds = (n + kStreamThreads - 1) / kStreamThreads;
  const uint32_t *sp = (const uint32_t *)(a.scores + (int64_t)lg * a.b.E + e0);
  // CRF of (layer, head) at 32-bit offsets page * Hkv * 16 + slot-in-page (the host
  // checks that every offset fits)
  float *crf_base = a.crf + (((int64_t)l * a.b.num_pages) * a.b.Hkv + g) * kPage;
  const uint32_t page_stride = (uint32_t)a.b.Hkv * kPage;
  uint8_t *kp = a.keep + (int64_t)lg * a.b.E + e0;

  int32_t K = 0;
  if (SELECT) {
    const int32_t bud = a.budget[i];
    K = bud < n ? (bud > 0 ? bud : 0) : n;
    if (!LRFU && (K == 0 || K == n)) {
      for (int32_t j = tid; j < n; j += kStreamThreads) kp[j] = K == n ? 1 : 0;
      return;
    }
  }
  const int32_t npages = (start + n + kPage - 1) / kPage;
  const int32_t *bt_row = a.b.bt + (int64_t)i * a.b.max_pages;
  for (int32_t p = tid; p < npages; p += kStreamThreads) bt_lds[p] = bt_row[p];
  // slot of row u (t = this thread's index), clamped to the last live slot so that
  // loads can be unconditional
  auto slot = [&](int u, int t) -> int32_t { return min(u * kStreamThreads + t, n - 1); };
  auto crf_off = [&](int u, int t) -> uint32_t {
    const int32_t pos = start + slot(u, t);
    return (uint32_t)bt_lds[pos >> 4] * page_stride + (uint32_t)(pos & 15);
  };

  uint32_t s[kRegU];
  uint32_t c[kRegU];
  bool have_s = false;
  auto load_s = [&]() {
    // 8 loads in flight per thread and chunk; a chunk's offsets die at issue
#pragma unroll
    for (int u0 = 0; u0 < kRegU; u0 += 8) {
      const int t = opaque(tid);
#pragma unroll
      for (int u = u0; u < u0 + 8; ++u) s[u] = sp[slot(u, t)];
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = 0; u < kRegU; ++u) s[u] = u < cnt ? s[u] : 0u;
  };
  // every row's CRF in flight at once, issued in 8-row groups so that only a group's
  // offsets are live at a time (nothing waits between the groups)
  auto gather_crf = [&]() {
#pragma unroll
    for (int u0 = 0; u0 < kRegU; u0 += 8) {
      const int t = opaque(tid);
#pragma unroll
      for (int u = u0; u < u0 + 8; ++u) c[u] = __float_as_uint(crf_base[crf_off(u, t)]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto all = [](int) { return true; };
  auto one = [](uint32_t) -> uint64_t { return 1; };
  __syncthreads();   // block-table slice visible

  if (LRFU) {
    load_s();
    have_s = true;
    uint32_t band = ~0u, bor = 0u;
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      band &= u < cnt ? s[u] : ~0u;
      bor |= s[u];
    }
    block_and_or(band, bor, (uint32_t *)sh.scratch);
    // T = ceil(num * M / den), M = the stream's total integer mass (from the first pass)
    const Sel r = reg_select<false, true>(s, cnt, all, fixed_mass, 0, a.num, a.den, band, bor, sh);
    const uint64_t T = r.target;
    const bool none = T == 0;
    uint32_t vstar = 0xFFFFFFFFu;
    uint64_t k_needed = 0, ties = 0;
    if (!none) {
      vstar = r.key;
      const uint64_t mstar = fixed_mass(vstar);
      k_needed = (T - r.above + mstar - 1) / mstar;
      ties = r.at / mstar;
    }
    // hit bits (bit u)
    uint64_t hbits = 0;
    if (!none && k_needed < ties) {
      // ties at the threshold exceed the hits still needed: lowest slots first
      uint32_t tmask = 0;
#pragma unroll
      for (int u = 0; u < kRegU; ++u) tmask |= (uint32_t)(u < cnt && s[u] == vstar) << u;
      rank_flags(tmask, rounds, (uint32_t *)sh.hist, flag_scratch, [&](int u, uint32_t rk) {
        const bool valid = u < cnt;
        const bool tie = (tmask >> u) & 1u;
        const bool h = valid && (s[u] > vstar || (tie && rk < k_needed));
        hbits |= (uint64_t)h << u;
      });
    } else if (!none) {
#pragma unroll
      for (int u = 0; u < kRegU; ++u) hbits |= (uint64_t)(u < cnt && s[u] >= vstar) << u;
    }
    // LRFU update of the paged CRF, KVS_CRF_CHUNK rows per round trip
    const float d = a.decay[i];
    const int np_rel = a.n_prev[i] - tid;       // row u has a prior iff u * 1024 < np_rel
    constexpr int kChunk = KVS_CRF_CHUNK;
#pragma unroll
    for (int u0 = 0; u0 < kRegU; u0 += kChunk) {
      const int t = opaque(tid);
      uint32_t off[kChunk];
      float prior[kChunk];
#pragma unroll
      for (int v = 0; v < kChunk; ++v) {
        off[v] = crf_off(u0 + v, t);
        prior[v] = crf_base[off[v]];
      }
#pragma unroll
      for (int v = 0; v < kChunk; ++v) {
        const int u = u0 + v;
        const bool h = (hbits >> u) & 1;
        const float p = u * kStreamThreads < np_rel ? prior[v] : 0.f;
        const float nv = __builtin_fmaf(d, p, h ? 1.f : 0.f);
        c[u] = u < cnt ? __float_as_uint(nv) : 0u;
        KVS_FOR_VALID(u, crf_base[off[v]] = nv;)
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (a.hit) {
      uint8_t *hp = a.hit + (int64_t)lg * a.b.E + e0;
      const int t = opaque(tid);
#pragma unroll
      for (int u = 0; u < kRegU; ++u) {
        KVS_FOR_VALID(u, hp[u * kStreamThreads + t] = (uint8_t)((hbits >> u) & 1);)
      }
    }
    if (!SELECT) return;
    have_s = false;     // the selection reloads the scores only for ties at the threshold
    if (K == 0 || K == n) {
      const int t = opaque(tid);
#pragma unroll
      for (int u = 0; u < kRegU; ++u) {
        KVS_FOR_VALID(u, kp[u * kStreamThreads + t] = K == n ? 1 : 0;)
      }
      return;
    }
  } else {
    if (a.keys) {
      const uint32_t *kf = (const uint32_t *)(a.keys + (int64_t)lg * a.b.E + e0);
#pragma unroll
      for (int u0 = 0; u0 < kRegU; u0 += 8) {
        const int t = opaque(tid);
#pragma unroll
        for (int u = u0; u < u0 + 8; ++u) c[u] = kf[slot(u, t)];
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      gather_crf();
    }
#pragma unroll
    for (int u = 0; u < kRegU; ++u) c[u] = u < cnt ? c[u] : 0u;
  }

  // ---- top-K keep set ----
  // Common case first: when at least K entries share the largest CRF (every recent hit
  // has CRF exactly 1 once the decayed prior rounds away), that value is c* and no
  // radix pass over CRF is needed.
  // Otherwise CRF keys are split at 1.0 first (a hit's CRF is at least 1): c* lies among
  // the keys >= 1 when there are at least K of them, else among the keys below 1 (with
  // every key >= 1 kept).  The radix search then runs on one side only, whose keys
  // share a longer prefix, so it needs fewer passes.
  constexpr uint32_t kOne = 0x3F800000u;           // 1.0f; keys are fp32 bits of values >= 0
  uint32_t band_hi = ~0u, bor_hi = 0u, band_lo = ~0u, bor_lo = 0u, cmax = 0u, ge = 0u;
#pragma unroll
  for (int u = 0; u < kRegU; ++u) {
    const bool v = u < cnt, hi = c[u] >= kOne;
    band_hi &= v && hi ? c[u] : ~0u;
    bor_hi |= v && hi ? c[u] : 0u;
    band_lo &= v && !hi ? c[u] : ~0u;
    bor_lo |= v && !hi ? c[u] : 0u;
    ge += v && hi ? 1u : 0u;
    cmax = c[u] > cmax ? c[u] : cmax;
  }
  cmax = block_max_u32(cmax, (uint32_t *)sh.scratch);
  uint32_t at_max = 0;
#pragma unroll
  for (int u = 0; u < kRegU; ++u) at_max += (u < cnt && c[u] == cmax) ? 1u : 0u;
  const uint64_t n_max = block_sum_u64(at_max, sh.scratch);
  Sel r1;
  if (n_max >= (uint64_t)K) {
    r1.key = cmax;
    r1.above = 0;
    r1.at = n_max;
  } else if (!LRFU && a.keys) {
    // caller keys (step-aware ranking) have no reason to straddle 1.0: no split
    uint32_t band = band_hi & band_lo, bor = bor_hi | bor_lo;
    block_and_or(band, bor, (uint32_t *)sh.scratch);
    r1 = reg_select<true, false>(c, cnt, all, one, (uint64_t)K, 0, 1, band, bor, sh);
  } else {
    const uint64_t n_ge = block_sum_u64(ge, sh.scratch);
    const bool upper = n_ge >= (uint64_t)K;
    uint32_t band = upper ? band_hi : band_lo, bor = upper ? bor_hi : bor_lo;
    block_and_or(band, bor, (uint32_t *)sh.scratch);
    auto side = [&](int u) { return (c[u] >= kOne) == upper; };
    r1 = reg_select<true, false>(c, cnt, side, one, upper ? (uint64_t)K : (uint64_t)K - n_ge, 0, 1, band, bor, sh);
    if (!upper) r1.above += n_ge;
  }
  const uint32_t cstar = r1.key;
  const uint64_t need = K - r1.above;          // entries to keep among CRF == c*
  const bool lvl2 = need < r1.at;
  if (lvl2 && r1.at <= (uint64_t)kTieList) {
    // Few entries tie at c*: gather them (s, slot) into LDS and rank each one among
    // the ties by (s desc, slot asc) directly; the first `need` are kept.
    if (!have_s) load_s();
    if (tid == 0) tie_count = 0;
    __syncthreads();
    const int lane = tid & 63;
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      const bool t = u < cnt && c[u] == cstar;
      const uint64_t m = __ballot(t);
      if (m) {
        const int leader = __ffsll((long long)m) - 1;
        uint32_t base = 0;
        if (lane == leader) base = atomicAdd(&tie_count, (uint32_t)__popcll(m));
        base = (uint32_t)__builtin_amdgcn_readlane((int)base, leader);
        const uint32_t idx = base + (uint32_t)__popcll(m & lanemask_lt());
        if (t && idx < (uint32_t)kTieList) {
          tie_s[idx] = s[u];
          tie_j[idx] = u * kStreamThreads + tid;
        }
      }
    }
    __syncthreads();
    const int nt = (int)r1.at;     // == tie_count (the entries equal to c*)
    for (int x = tid; x < nt; x += kStreamThreads) {
      const uint32_t sx = tie_s[x];
      const int32_t jx = tie_j[x];
      // ties ahead of x in (s desc, slot asc), four at a time (16-byte LDS reads, the
      // same address in every lane); the slots past nt are never compared
      uint32_t rank = 0;
      int y = 0;
#pragma unroll 4
      for (; y + 4 <= nt; y += 4) {
        const uint4 sy = *(const uint4 *)&tie_s[y];
        const int4 jy = *(const int4 *)&tie_j[y];
        rank += (sy.x > sx || (sy.x == sx && jy.x < jx)) ? 1u : 0u;
        rank += (sy.y > sx || (sy.y == sx && jy.y < jx)) ? 1u : 0u;
        rank += (sy.z > sx || (sy.z == sx && jy.z < jx)) ? 1u : 0u;
        rank += (sy.w > sx || (sy.w == sx && jy.w < jx)) ? 1u : 0u;
      }
      for (; y < nt; ++y) {
        const uint32_t sy = tie_s[y];
        rank += (sy > sx || (sy == sx && tie_j[y] < jx)) ? 1u : 0u;
      }
      kp[jx] = rank < need ? 1 : 0;
    }
    const int t = opaque(tid);
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      if (c[u] != cstar) {
        KVS_FOR_VALID(u, kp[u * kStreamThreads + t] = c[u] > cstar ? 1 : 0;)
      }
    }
    return;
  }
  uint32_t sstar = 0;
  uint64_t need2 = 0, at2 = 0;
  if (lvl2) {
    if (!have_s) load_s();
    uint32_t sa = ~0u, so = 0u;
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      const bool t = u < cnt && c[u] == cstar;
      sa &= t ? s[u] : ~0u;
      so |= t ? s[u] : 0u;
    }
    block_and_or(sa, so, (uint32_t *)sh.scratch);
    auto in_tie = [&](int u) { return c[u] == cstar; };
    const Sel r2 = reg_select<true, false>(s, cnt, in_tie, one, need, 0, 1, sa, so, sh);
    sstar = r2.key;
    need2 = need - r2.above;
    at2 = r2.at;
  }
  if (!(lvl2 && need2 < at2)) {
    const int t = opaque(tid);
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      const bool k = lvl2 ? (c[u] > cstar || (c[u] == cstar && s[u] >= sstar)) : c[u] >= cstar;
      KVS_FOR_VALID(u, kp[u * kStreamThreads + t] = k ? 1 : 0;)
    }
  } else {
    uint32_t tmask = 0;
#pragma unroll
    for (int u = 0; u < kRegU; ++u) tmask |= (uint32_t)(u < cnt && c[u] == cstar && s[u] == sstar) << u;
    rank_flags(tmask, rounds, (uint32_t *)sh.hist, flag_scratch, [&](int u, uint32_t rk) {
      const bool tie = (tmask >> u) & 1u;
      const bool k = c[u] > cstar || (c[u] == cstar && (s[u] > sstar || (tie && rk < need2)));
      if (u < cnt) kp[u * kStreamThreads + tid] = k ? 1 : 0;
    });
  }
}

#undef KVS_FOR_VALID

}  // namespace

bool stream_reg_fits(int32_t max_len, int64_t num_pages, int32_t Hkv) {
  return max_len <= kRegMaxLen && num_pages * Hkv * kPage < (int64_t(1) << 31);
}

hipError_t launch_stream_reg(const kvs_cache &c, const Batch &b, const float *scores, bool lrfu, bool select,
                             uint32_t num, uint32_t den, const float *decay, const int32_t *n_prev,
                             uint8_t *hit, const int32_t *budget, uint8_t *keep, hipStream_t st,
                             const float *keys) {
  StreamArgs a{};
  a.keys = keys;
  a.scores = scores;
  a.crf = c.crf;
  a.hit = hit;
  a.decay = decay;
  a.n_prev = n_prev;
  a.budget = budget;
  a.keep = keep;
  a.b = b;
  a.num = num;
  a.den = den;
  dim3 grid((unsigned)(b.L * b.Hkv), (unsigned)b.S);
  if (lrfu && select) stream_reg_kernel<true, true><<<grid, kStreamThreads, 0, st>>>(a);
  else if (lrfu) stream_reg_kernel<true, false><<<grid, kStreamThreads, 0, st>>>(a);
  else stream_reg_kernel<false, true><<<grid, kStreamThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
