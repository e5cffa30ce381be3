// Register-resident per-stream kernels: the attention-mass cut with the LRFU update,
// the top-B keep set, or both in one pass over the data.  One 1024-thread workgroup
// per stream; thread t owns slots u * 1024 + t (u < kRegU): their scores sit in LDS
// (slot-major, each thread touching only its own) and their CRF, or caller keys, in
// registers, so each input is read from memory once and every selection pass runs on
// LDS and registers.  Streams longer than kRegU * 1024 entries take the kernels of
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
// the AND and OR of their keys), kDigitBits = 11 bits per pass, with a 2048-bin LDS
// histogram of counts or of integer masses; the crossing bin is found with one
// block-wide scan.

#include "kvs_device.h"

namespace kvs {

constexpr int kRegU = 32;                                        // slots per thread
constexpr int32_t kRegMaxLen = kRegU * kStreamThreads;           // 32768 entries per stream
constexpr int kRegBtCap = (kRegMaxLen + 2 * kPage - 2) / kPage;  // pages of a stream (start < 16)
constexpr int kDigitBits = 11;
constexpr int kBins = 1 << kDigitBits;
constexpr int kTieMax = 2 * kBins - 512;   // keys searched in an LDS list (plus 256 u64 bins) up to this many
constexpr int kSmallTies = 256;            // tie classes at c* ranked pairwise up to this many
static_assert(kRegU % 8 == 0, "the 8-row load groups tile the rows exactly");
// LDS: the stream's scores (u32, slot-major) in dynamic shared memory, the rest static
constexpr size_t kScoreLds = (size_t)kRegMaxLen * sizeof(uint32_t);

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
  // PLAN: the slot plan of kvs_plan, in the same workgroup
  int32_t *pairs;        // [L*Hkv][S][P][2]
  int32_t *pair_count;   // [L*Hkv][S]
  int64_t P;
};

struct RegShared {
  uint64_t hist[kBins];
  uint64_t scratch[kStreamWaves];
  uint64_t found[3];
  uint32_t list_n;
  // entry counts of the mass cut's first pass, two 16-bit bins per word (a bin holds at
  // most kRegMaxLen = 2^15 entries, so a count never carries into its neighbour)
  uint32_t cnt16[kBins / 2];
};
static_assert(kTieMax + 512 <= 2 * kBins && kTieMax % 2 == 0, "a key list and its bins fit in the histogram's space");
static_assert(kBins <= 4 * kStreamThreads, "the crossing-bin scan takes 4 bins per thread");

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
  lds_barrier();
  // lane w < waves holds wave w's total; one wave scan gives every wave its offset
  const int lane = threadIdx.x & 63;
  const uint64_t wsc = wave_scan_u64(lane < kStreamWaves ? scratch[lane] : 0ull);
  lds_barrier();
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
  lds_barrier();
  static_assert(kRegU * kStreamWaves <= kStreamThreads, "one (row, wave) count per thread");
  const uint32_t v = threadIdx.x < kRegU * kStreamWaves ? cnt[threadIdx.x] : 0u;
  uint32_t tot;
  const uint32_t ex = block_exclusive_scan(v, tot, scratch);
  if (threadIdx.x < kRegU * kStreamWaves) cnt[threadIdx.x] = ex;
  lds_barrier();
  const uint32_t *mine = cnt + opaque(wave);
#pragma unroll
  for (int u = 0; u < kRegU; ++u) {
    if (u < rounds) {
      const uint64_t b = __ballot((fmask >> u) & 1u);
      take(u, mine[u * kStreamWaves] + (uint32_t)__popcll(b & lanemask_lt()));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  lds_barrier();     // cnt is free again
}

// v* with weight(keys > v*) < need <= weight(keys >= v*) over the nt keys of an LDS
// list (1 <= need <= the list's total weight), the weight of a key being 1 (COUNT)
// or its integer mass: a radix search from the first bit where the keys differ, 8
// bits per pass, with a 256-bin u64 histogram (LDS atomics) scanned by one wave.
// bins: 256 u64 of LDS; found: 3 u64.  Every thread of the block must call it.
template <bool COUNT>
__device__ __forceinline__ Sel list_select(const uint32_t *key, int nt, uint64_t need, uint64_t *bins,
                                           uint32_t *scratch, uint64_t *found) {
  uint32_t a = ~0u, o = 0u;
  for (int x = threadIdx.x; x < nt; x += kStreamThreads) {
    a &= key[x];
    o |= key[x];
  }
  block_and_or(a, o, scratch);
  Sel r;
  r.target = need;
  const uint32_t diff = a ^ o;
  if (diff == 0) {
    r.key = a;
    r.above = 0;
    r.at = COUNT ? (uint64_t)nt : (uint64_t)nt * fixed_mass(a);
    return r;
  }
  int top = 31 - __clz(diff);
  uint32_t prefix = a & ~((2u << top) - 1u);      // (top = 31: the shift wraps to 0, mask all bits)
  uint64_t rem = need, above = 0, at = 0;
  while (top >= 0) {
    const int width = top + 1 < 8 ? top + 1 : 8;
    const int lo = top - width + 1;
    const uint32_t nb = 1u << width;
    if (threadIdx.x < 256) bins[threadIdx.x] = 0ull;
    lds_barrier();
    const int hs = top + 1;
    for (int x = threadIdx.x; x < nt; x += kStreamThreads) {
      const uint32_t k = key[x];
      if (hs >= 32 || (k >> hs) == (prefix >> hs))
        atomicAdd((unsigned long long *)&bins[(k >> lo) & (nb - 1u)],
                  COUNT ? 1ull : (unsigned long long)fixed_mass(k));
    }
    lds_barrier();
    if (threadIdx.x < 64) {
      // lane L takes bins nb-1-4L .. nb-4-4L (descending); the exclusive scan is the
      // weight of all higher bins
      const int lane = threadIdx.x;
      uint64_t h[4], ls = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = (int)nb - 1 - (4 * lane + q);
        h[q] = b >= 0 ? bins[b] : 0ull;
        ls += h[q];
      }
      uint64_t acc = wave_scan_u64(ls) - ls;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = (int)nb - 1 - (4 * lane + q);
        if (b >= 0 && acc < rem && rem <= acc + h[q]) {
          found[0] = (uint64_t)b;
          found[1] = acc;
          found[2] = h[q];
        }
        acc += h[q];
      }
    }
    lds_barrier();
    const uint32_t b = (uint32_t)found[0];
    const uint64_t ab = found[1];
    at = found[2];
    prefix |= b << lo;
    rem -= ab;
    above += ab;
    top = lo - 1;
  }
  r.key = prefix;
  r.above = above;
  r.at = at;
  return r;
}

// Appends key(u) of this thread's valid rows (u < cnt) where take(u, key(u)) holds to
// an LDS list of at most cap keys, in no particular order: per row, each wave
// reserves its range with one LDS atomic (lane 0, the wave's count of the row) and
// its lanes write at the ballot offsets.  Returns the number of keys that hold; all of
// them are in the list when it is at most cap (else some are missing).  Keys are read
// 8 rows at a time and take is evaluated without branches, so the reads and the
// atomics of a group overlap; groups of rows that every thread holds (u < full) skip
// the row test.  slots (optional) receives each key's slot u * 1024 + t at the same
// position.  Every thread of the block must call it.
template <typename KeyF, typename P>
__device__ __forceinline__ uint32_t gather_keys(KeyF key, P take, int cnt, int full, uint32_t *list, uint32_t cap,
                                                uint32_t *count, uint32_t *slots = nullptr) {
  if (threadIdx.x == 0) *count = 0;
  lds_barrier();
  const int lane = threadIdx.x & 63;
  // (an address the compiler takes as per-lane: it then adds no wave-reduction code of
  // its own around lane 0's atomics, code that would wait for each one in turn)
  uint32_t *cnt_lane = count + opaque(0);
#pragma unroll
  for (int u0 = 0; u0 < kRegU; u0 += 8) {
    uint32_t k[8], base[8];
    uint64_t m[8];
    const bool rows_full = u0 + 8 <= full;     // uniform
    const int cnt_p = opaque(cnt);
#pragma unroll
    for (int v = 0; v < 8; ++v) k[v] = key(u0 + v);
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      m[v] = ballot((rows_full || u0 + v < cnt_p) && take(u0 + v, k[v]));
      base[v] = 0;
      if (lane == 0) base[v] = atomicAdd(cnt_lane, (uint32_t)__popcll(m[v]));
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane((int)base[v]) +
                           (uint32_t)__popcll(m[v] & lanemask_lt());
      if (((m[v] >> lane) & 1ull) && pos < cap) {
        list[pos] = k[v];
        if (slots) slots[pos] = (uint32_t)((u0 + v) * kStreamThreads) + threadIdx.x;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  lds_barrier();
  return *count;
}

// Adds w (1 with COUNT) to bin in the lanes where ok holds.  Lanes that share the
// first adding lane's bin are summed first and added once when they are many (8 for
// counts, whose sum is a popcount; every adding lane for masses, whose sum takes a wave
// reduction: the case of equal scores); otherwise every lane adds its own and the LDS
// serialises lanes that share an address.  Zero masses add nothing.  Must be called
// by all lanes of the wave.
template <bool COUNT>
__device__ __forceinline__ void hist_add(uint64_t *hist, bool ok, uint32_t bin, uint64_t w) {
  if (!COUNT) ok = ok && w != 0;
  const uint64_t mask = ballot(ok);
  if (mask == 0) return;
  const int leader = (int)__builtin_ctzll(mask);
  const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
  const bool same = ok && bin == lb;
  const uint64_t smask = ballot(same);
  if (COUNT ? __popcll(smask) >= 8 : smask == mask) {
    const uint64_t agg = COUNT ? (uint64_t)__popcll(smask) : wave_sum_u64(same ? w : 0ull);
    // (the leader's own bin: an address the compiler takes as per-lane)
    if ((int)(threadIdx.x & 63) == leader) atomicAdd((unsigned long long *)&hist[bin], (unsigned long long)agg);
    if (ok && !same) atomicAdd((unsigned long long *)&hist[bin], (unsigned long long)(COUNT ? 1ull : w));
  } else if (ok) {
    atomicAdd((unsigned long long *)&hist[bin], (unsigned long long)(COUNT ? 1ull : w));
  }
}

// One histogram pass: every candidate whose key matches prefix above bit hs (hs = 32:
// no test, every candidate matches) adds its weight to bin (key >> lo) & (nb - 1).
// Keys are read 8 rows at a time; groups of rows that every thread holds (u < full)
// skip the per-lane row test.
template <bool COUNT, bool FIRST, typename KeyF, typename CandF, typename WF>
__device__ __forceinline__ void hist_pass(KeyF key, int cnt, int full, CandF cand, WF weight_of, int hs,
                                          uint32_t prefix, int lo, uint32_t nb, uint64_t *hist, uint32_t *cnt16) {
  const uint32_t ph = hs >= 32 ? 0u : prefix >> hs;
  const int hsc = hs & 31;
  // FIRST: every candidate matches the prefix (no test), and a mass pass also counts
  // its entries per bin into cnt16
  auto add = [&](bool ok, uint32_t k) {
    const uint32_t bin = (k >> lo) & (nb - 1u);
    hist_add<COUNT>(hist, ok, bin, COUNT ? 1ull : weight_of(k));
    if (FIRST && !COUNT && ok) atomicAdd(&cnt16[bin >> 1], 1u << ((bin & 1u) << 4));
  };
#pragma unroll
  for (int u0 = 0; u0 < kRegU; u0 += 8) {
    uint32_t k[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) k[v] = key(u0 + v);
    if (u0 + 8 <= full) {
#pragma unroll
      for (int v = 0; v < 8; ++v) add(cand(u0 + v) && (FIRST || (k[v] >> hsc) == ph), k[v]);
    } else {
      const int cnt_p = opaque(cnt);
#pragma unroll
      for (int v = 0; v < 8; ++v) add(u0 + v < cnt_p && cand(u0 + v) && (FIRST || (k[v] >> hsc) == ph), k[v]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// v* with weight(keys > v*) < target <= weight(keys >= v*) over the candidates
// (slot valid and cand(u)); key(u) is the key of this thread's row u (a register, or
// the thread's own slot of an LDS array).  With CUT the target is ceil(num * W / den)
// for the candidates' total weight W, which the first pass yields (so W needs no pass
// of its own); otherwise it is `target`.  A target of 0 returns key ~0 and at = 0.
// After each pass the candidates in the crossing bin are gathered into an LDS list
// when they are few enough (at most kTieMax: known from the count, or bounded by the
// bin's mass over the mass of its smallest key), and the search finishes there
// instead of with further passes over every row.
template <bool COUNT, bool CUT, typename KeyF, typename CandF, typename WF>
__device__ __forceinline__ Sel reg_select(KeyF key, int cnt, int full, CandF cand, WF weight_of, uint64_t target,
                                          uint32_t num, uint32_t den, uint32_t and_all, uint32_t or_all,
                                          RegShared &sh) {
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
      const uint32_t k = key(u);
      if ((u < opaque(cnt)) & cand(u)) w += COUNT ? 1ull : weight_of(k);
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
  uint32_t *list = (uint32_t *)sh.hist;
  uint64_t *list_bins = sh.hist + kTieMax / 2;
  int pass = 0;
  while (top >= 0) {
    const int width = top + 1 < kDigitBits ? top + 1 : kDigitBits;
    const int lo = top - width + 1;
    const uint32_t nb = 1u << width;
    for (uint32_t b = threadIdx.x; b < nb; b += kStreamThreads) sh.hist[b] = 0;
    if (!COUNT && pass == 0)
      for (uint32_t b = threadIdx.x; b < kBins / 2; b += kStreamThreads) sh.cnt16[b] = 0;
    lds_barrier();
    // (the first pass needs no prefix test: and_all and or_all cover every candidate)
    if (pass == 0)
      hist_pass<COUNT, true>(key, cnt, full, cand, weight_of, 32, prefix, lo, nb, sh.hist, sh.cnt16);
    else
      hist_pass<COUNT, false>(key, cnt, full, cand, weight_of, top + 1, prefix, lo, nb, sh.hist, sh.cnt16);
    ++pass;
    lds_barrier();
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
    lds_barrier();
    const uint32_t b = (uint32_t)sh.found[0];
    const uint64_t a = sh.found[1];
    at = sh.found[2];
    lds_barrier();
    prefix |= b << lo;
    need -= a;
    above += a;
    top = lo - 1;
    if (top < 0) break;
    bool try_list;
    if (COUNT) {
      try_list = at <= (uint64_t)kTieMax;
    } else if (pass == 1) {
      // the first pass counted the bin's entries
      try_list = ((sh.cnt16[b >> 1] >> ((b & 1u) << 4)) & 0xFFFFu) <= (uint32_t)kTieMax;
    } else {
      const uint64_t m_low = weight_of(prefix);      // the bin's smallest key
      try_list = m_low == 0 || at / m_low <= (uint64_t)kTieMax;
    }
    if (try_list) {
      const uint32_t pl = prefix >> lo;
      const uint32_t nl = gather_keys(
          key, [&](int u, uint32_t k) { return cand(u) && (k >> lo) == pl; }, cnt, full, list, (uint32_t)kTieMax,
          &sh.list_n);
      if (nl <= (uint32_t)kTieMax) {
        const Sel r2 = list_select<COUNT>(list, (int)nl, need, list_bins, (uint32_t *)sh.scratch, sh.found);
        r.key = r2.key;
        r.above = above + r2.above;
        r.at = r2.at;
        return r;
      }
    }
  }
  r.key = prefix;
  r.above = above;
  r.at = at;
  return r;
}

// The slot plan of one stream once its keep set is written (kvs_plan, in the
// selection's workgroup): plan_slots over the keep bytes, re-read after a full barrier
// so that this workgroup's stores are visible to all of it.  The moves are a kernel of
// their own, which spreads each stream's pairs over many small workgroups.
__device__ __forceinline__ void plan_pairs(const StreamArgs &a, int32_t K, RegShared &sh, uint32_t *flag_scratch,
                                           int32_t i, int32_t lg, int32_t n) {
  const int64_t pc = (int64_t)lg * a.b.S + i;
  const int32_t D = n - K;
  uint32_t c = 0;
  if ((D < K ? D : K) > 0) {
    __syncthreads();
    c = plan_slots(a.keep + (int64_t)lg * a.b.E + a.b.entry_off[i], n, K, a.pairs + pc * a.P * 2, flag_scratch,
                   (uint32_t *)sh.scratch);
  }
  if (threadIdx.x == 0) a.pair_count[pc] = (int32_t)c;
}

// Stores for slot rows: rows u < full exist in every thread (uniform branch); the
// partial row after them is predicated per lane.
#define KVS_FOR_VALID(u, ...)   \
  if ((u) < full) {             \
    __VA_ARGS__                 \
  } else if ((u) < cnt) {       \
    __VA_ARGS__                 \
  }

template <bool LRFU, bool SELECT, bool PLAN>
__global__ __launch_bounds__(kStreamThreads) void stream_reg_kernel(StreamArgs a) {
  static_assert(!PLAN || (LRFU && SELECT), "the plan follows the fused cut, update and keep set");
  __shared__ int32_t bt_lds[kRegBtCap];
  __shared__ RegShared sh;
  __shared__ uint32_t flag_scratch[kStreamWaves];
  extern __shared__ uint32_t s_lds[];     // kScoreLds bytes: score bits of slot u * 1024 + t

  const int32_t i = blockIdx.y;
  const int32_t lg = blockIdx.x;
  const int32_t n = a.b.len[i];
  if (n <= 0) {
    if (PLAN && threadIdx.x == 0) a.pair_count[(int64_t)lg * a.b.S + i] = 0;
    return;
  }
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

  // The scores live in LDS (each thread reads and writes only its own slots, so they
  // need no barrier); the CRF or caller keys live in registers c.
  uint32_t c[kRegU];
  // (two opaque base addresses, with the row in the instruction's offset, and an opaque
  // copy of cnt at each use: otherwise the compiler keeps 32 slot addresses and 32 row
  // masks live through the whole kernel, and spills them)
  const uint32_t *sb0 = s_lds + opaque(tid);                        // rows 0..15
  const uint32_t *sb1 = s_lds + 16 * kStreamThreads + opaque(tid);   // rows 16..31
  auto sv = [&](int u) -> uint32_t { return u < 16 ? sb0[u * kStreamThreads] : sb1[(u - 16) * kStreamThreads]; };
  auto valid = [&](int u) -> bool { return u < opaque(cnt); };
  bool have_s = false;
  // AND and OR of the valid scores (block-wide once reduced): the common prefix of
  // every score, so of every subset of them
  uint32_t s_and = ~0u, s_or = 0u;
  // scores of every row in flight at once through the registers tmp (8 or kRegU of
  // them), then into LDS (0 for slots past the end); this thread's AND and OR of them
  auto load_s = [&](uint32_t *tmp, int group) {
    for (int u0 = 0; u0 < kRegU; u0 += group) {
#pragma unroll
      for (int g0 = 0; g0 < group; g0 += 8) {
        const int t = opaque(tid);
#pragma unroll
        for (int v = 0; v < 8; ++v) tmp[g0 + v] = sp[slot(u0 + g0 + v, t)];
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int v = 0; v < group; ++v) {
        const int u = u0 + v;
        const bool ok = valid(u);
        s_lds[u * kStreamThreads + tid] = ok ? tmp[v] : 0u;
        s_and &= ok ? tmp[v] : ~0u;
        s_or |= ok ? tmp[v] : 0u;
      }
    }
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
  lds_barrier();   // block-table slice visible

  uint32_t cmx = 0, ncm = 0;   // this thread's largest CRF (or key) and its count
  // (the cut, the LRFU update and the keep set; each exit of the selection returns from
  // this lambda, after which PLAN writes the stream's slot plan)
  auto select_body = [&]() __attribute__((always_inline)) {
  if (LRFU) {
    // (c carries the scores on their way to LDS)
    load_s(c, kRegU);
    have_s = true;
    // The prior CRF is gathered now into c and waited for only where the update reads
    // it: the barriers of the cut order LDS only, so these loads stay in flight
    // through the whole mass cut.
    gather_crf();
    block_and_or(s_and, s_or, (uint32_t *)sh.scratch);
    // T = ceil(num * M / den), M = the stream's total integer mass (from the first pass)
    const Sel r = reg_select<false, true>(sv, cnt, full, all, fixed_mass, 0, a.num, a.den, s_and, s_or, sh);
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
      for (int u = 0; u < kRegU; ++u) tmask |= (uint32_t)(valid(u) & (sv(u) == vstar)) << u;
      rank_flags(tmask, rounds, (uint32_t *)sh.hist, flag_scratch, [&](int u, uint32_t rk) {
        const bool tie = (tmask >> u) & 1u;
        const bool h = valid(u) & ((sv(u) > vstar) | (tie & (rk < k_needed)));
        hbits |= (uint64_t)h << u;
      });
    } else if (!none) {
#pragma unroll
      for (int u = 0; u < kRegU; ++u) hbits |= (uint64_t)(valid(u) & (sv(u) >= vstar)) << u;
    }
    // LRFU update of the paged CRF in place (the priors are in c), the hit bytes, and
    // this thread's largest new CRF with its count, in one pass
    const float d = a.decay[i];
    const int np_rel = a.n_prev[i] - tid;       // row u has a prior iff u * 1024 < np_rel
    uint8_t *hp = a.hit ? a.hit + (int64_t)lg * a.b.E + e0 : nullptr;
    {
      const int t = opaque(tid);
#pragma unroll
      for (int u = 0; u < kRegU; ++u) {
        const bool h = (hbits >> u) & 1;
        const float p = u * kStreamThreads < np_rel ? __uint_as_float(c[u]) : 0.f;
        const float nv = __builtin_fmaf(d, p, h ? 1.f : 0.f);
        const uint32_t cb = __float_as_uint(nv);
        const bool ok = valid(u);
        c[u] = ok ? cb : 0u;
        const bool gt = ok && cb > cmx, eq = ok && cb == cmx;
        cmx = gt ? cb : cmx;
        ncm = gt ? 1u : ncm + (eq ? 1u : 0u);
        KVS_FOR_VALID(u, crf_base[crf_off(u, t)] = nv; if (hp) hp[u * kStreamThreads + t] = (uint8_t)h;)
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (!SELECT) return;
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
    for (int u = 0; u < kRegU; ++u) c[u] = valid(u) ? c[u] : 0u;
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
  auto cv = [&](int u) -> uint32_t { return c[u]; };
  if (!LRFU) {
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      const bool ok = valid(u);
      const bool gt = ok && c[u] > cmx, eq = ok && c[u] == cmx;
      cmx = gt ? c[u] : cmx;
      ncm = gt ? 1u : ncm + (eq ? 1u : 0u);
    }
  }
  const uint32_t cmax = block_max_u32(cmx, (uint32_t *)sh.scratch);
  const uint64_t n_max = block_sum_u64(cmx == cmax ? ncm : 0u, sh.scratch);
  Sel r1;
  if (n_max >= (uint64_t)K) {
    r1.key = cmax;
    r1.above = 0;
    r1.at = n_max;
  } else {
    uint32_t band_hi = ~0u, bor_hi = 0u, band_lo = ~0u, bor_lo = 0u, ge = 0u;
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      const bool v = valid(u), hi = c[u] >= kOne;
      band_hi &= v && hi ? c[u] : ~0u;
      bor_hi |= v && hi ? c[u] : 0u;
      band_lo &= v && !hi ? c[u] : ~0u;
      bor_lo |= v && !hi ? c[u] : 0u;
      ge += v && hi ? 1u : 0u;
    }
    if (!LRFU && a.keys) {
      // caller keys (step-aware ranking) have no reason to straddle 1.0: no split
      uint32_t band = band_hi & band_lo, bor = bor_hi | bor_lo;
      block_and_or(band, bor, (uint32_t *)sh.scratch);
      r1 = reg_select<true, false>(cv, cnt, full, all, one, (uint64_t)K, 0, 1, band, bor, sh);
    } else {
      const uint64_t n_ge = block_sum_u64(ge, sh.scratch);
      const bool upper = n_ge >= (uint64_t)K;
      uint32_t band = upper ? band_hi : band_lo, bor = upper ? bor_hi : bor_lo;
      block_and_or(band, bor, (uint32_t *)sh.scratch);
      auto side = [&](int u) { return (c[u] >= kOne) == upper; };
      r1 = reg_select<true, false>(cv, cnt, full, side, one, upper ? (uint64_t)K : (uint64_t)K - n_ge, 0, 1, band,
                                   bor, sh);
      if (!upper) r1.above += n_ge;
    }
  }
  const uint32_t cstar = r1.key;
  const uint64_t need = K - r1.above;          // entries to keep among CRF == c*
  const bool lvl2 = need < r1.at;
  if (lvl2 && r1.at <= (uint64_t)kSmallTies) {
    // A small tie class at c*: its entries' scores and slots are gathered, and each one's
    // rank in (s desc, slot asc) among them is counted directly, which settles the tied
    // entries' keep bits without a radix search or a block-wide slot ranking.
    uint32_t *ls = (uint32_t *)sh.hist;
    uint32_t *lslot = ls + kSmallTies;
    const int nt = (int)gather_keys(cv, [&](int u, uint32_t) { return c[u] == cstar; }, cnt, full, ls,
                                    (uint32_t)kSmallTies, &sh.list_n, lslot);
    // their scores: from LDS when the cut loaded them, else straight from memory (only
    // these few, not the whole stream)
    for (int x = tid; x < nt; x += kStreamThreads) ls[x] = have_s ? s_lds[lslot[x]] : sp[lslot[x]];
    lds_barrier();
    {
      // four threads per tied entry x, each counting a quarter of the list; lanes 4x..4x+3
      // of a wave add their counts with two shuffles
      static_assert(kSmallTies * 4 <= kStreamThreads, "four threads per tied entry");
      const int x = tid >> 2, part = tid & 3;
      const bool mine = x < nt;
      const uint32_t sx = mine ? ls[x] : 0u, qx = mine ? lslot[x] : 0u;
      const int y0 = part * (kSmallTies / 4), y1 = min(y0 + kSmallTies / 4, nt);
      uint32_t rank = 0;
      if (mine) {
#pragma unroll 8
        for (int y = y0; y < y1; ++y) {
          const uint32_t sy = ls[y];
          rank += (sy > sx || (sy == sx && lslot[y] < qx)) ? 1u : 0u;
        }
      }
      rank += (uint32_t)__shfl_xor((int)rank, 1);
      rank += (uint32_t)__shfl_xor((int)rank, 2);
      if (mine && part == 0) kp[qx] = rank < need ? 1 : 0;
    }
    const int t = opaque(tid);
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      KVS_FOR_VALID(u, if (c[u] != cstar) kp[u * kStreamThreads + t] = c[u] > cstar ? 1 : 0;)
    }
    return;
  }
  uint32_t sstar = 0;
  uint64_t need2 = 0, at2 = 0;
  if (lvl2) {
    // The entries tied at c* are ranked by this round's s: v* of s over them.
    if (!have_s) {
      uint32_t tmp[kRegU];      // every row's score in flight at once
      load_s(tmp, kRegU);
      block_and_or(s_and, s_or, (uint32_t *)sh.scratch);
    }
    Sel r2;
    if (r1.at <= (uint64_t)kTieMax) {
      // Few enough ties: their scores are gathered into an LDS list (sh.hist is free
      // here) and searched there, which touches at most kTieMax keys per pass instead
      // of every row of the stream.
      uint32_t *tl = (uint32_t *)sh.hist;
      const uint32_t nl = gather_keys(sv, [&](int u, uint32_t) { return c[u] == cstar; }, cnt, full, tl,
                                      (uint32_t)kTieMax, &sh.list_n);
      r2 = list_select<true>(tl, (int)nl, need, sh.hist + kTieMax / 2, (uint32_t *)sh.scratch, sh.found);
    } else {
      bool done = false;
      if (LRFU && s_and != s_or) {
        // The mass cut's first pass counted every entry per bin of the first score digit
        // (the same digit as here: both come from the AND and OR of every score).  Take
        // the lowest bin b0 whose entries, with those of the bins above, number at most
        // kTieMax: the tied entries scored from b0's lower edge up then fit the list,
        // and when there are at least `need` of them they hold the answer.
        const int top0 = 31 - __clz(s_and ^ s_or);
        const int width0 = top0 + 1 < kDigitBits ? top0 + 1 : kDigitBits;
        const int lo0 = top0 - width0 + 1;
        const int nb0 = 1 << width0;
        const uint32_t prefix0 = top0 == 31 ? 0u : (s_and & ~((2u << top0) - 1u));
        uint32_t best = 0xFFFFFFFFu;      // lowest qualifying bin of this lane's bins
        if (tid < 64) {
          constexpr int kPer = kBins / 64;  // bins per lane, in descending order
          uint32_t cb[kPer], ls = 0;
#pragma unroll
          for (int q = 0; q < kPer; ++q) {
            const int b = nb0 - 1 - (kPer * tid + q);
            cb[q] = b >= 0 ? (sh.cnt16[b >> 1] >> ((b & 1) << 4)) & 0xFFFFu : 0u;
            ls += cb[q];
          }
          uint32_t acc = wave_scan_u32(ls) - ls;   // entries in the bins above this lane's
#pragma unroll
          for (int q = 0; q < kPer; ++q) {
            const int b = nb0 - 1 - (kPer * tid + q);
            acc += cb[q];
            if (b >= 0 && acc <= (uint32_t)kTieMax) best = (uint32_t)b;
          }
        }
        const uint32_t b0 = ~block_max_u32(~best, flag_scratch);    // the lowest over lanes
        if (b0 != 0xFFFFFFFFu) {
          const uint32_t t0 = prefix0 | (b0 << lo0);
          uint32_t *tl = (uint32_t *)sh.hist;
          const uint32_t nl = gather_keys(sv, [&](int u, uint32_t k) { return c[u] == cstar && k >= t0; }, cnt,
                                          full, tl, (uint32_t)kTieMax, &sh.list_n);
          if ((uint64_t)nl >= need && nl <= (uint32_t)kTieMax) {
            r2 = list_select<true>(tl, (int)nl, need, sh.hist + kTieMax / 2, (uint32_t *)sh.scratch, sh.found);
            done = true;
          }
        }
      }
      if (!done) {
        // the prefix common to every score is common to the tied ones
        auto in_tie = [&](int u) { return c[u] == cstar; };
        r2 = reg_select<true, false>(sv, cnt, full, in_tie, one, need, 0, 1, s_and, s_or, sh);
      }
    }
    sstar = r2.key;
    need2 = need - r2.above;
    at2 = r2.at;
  }
  if (!(lvl2 && need2 < at2)) {
    const int t = opaque(tid);
#pragma unroll
    for (int u = 0; u < kRegU; ++u) {
      const uint32_t x = sv(u);
      const bool k = lvl2 ? ((c[u] > cstar) | ((c[u] == cstar) & (x >= sstar))) : c[u] >= cstar;
      KVS_FOR_VALID(u, kp[u * kStreamThreads + t] = k ? 1 : 0;)
    }
  } else {
    uint32_t tmask = 0;
#pragma unroll
    for (int u = 0; u < kRegU; ++u) tmask |= (uint32_t)(valid(u) & (c[u] == cstar) & (sv(u) == sstar)) << u;
    rank_flags(tmask, rounds, (uint32_t *)sh.hist, flag_scratch, [&](int u, uint32_t rk) {
      const bool tie = (tmask >> u) & 1u;
      const bool k = (c[u] > cstar) | ((c[u] == cstar) & ((sv(u) > sstar) | (tie & (rk < need2))));
      if (valid(u)) kp[u * kStreamThreads + tid] = k ? 1 : 0;
    });
  }
  };
  select_body();
  if constexpr (PLAN) plan_pairs(a, K, sh, flag_scratch, i, lg, n);
}

#undef KVS_FOR_VALID

}  // namespace

bool stream_reg_fits(int32_t max_len, int64_t num_pages, int32_t Hkv) {
  return max_len <= kRegMaxLen && num_pages * Hkv * kPage < (int64_t(1) << 31);
}

namespace {

// the scores' LDS exceeds the default dynamic limit: raise it once per device
hipError_t stream_reg_attrs() {
  static bool done[64] = {};
  const void *fns[4] = {(const void *)stream_reg_kernel<true, true, false>,
                        (const void *)stream_reg_kernel<true, false, false>,
                        (const void *)stream_reg_kernel<false, true, false>,
                        (const void *)stream_reg_kernel<true, true, true>};
  return raise_lds_limit(fns, 4, (int)kScoreLds, done);
}

}  // namespace

hipError_t launch_stream_reg_plan(const kvs_cache &c, const Batch &b, const float *scores, uint32_t num,
                                  uint32_t den, const float *decay, const int32_t *n_prev, uint8_t *hit,
                                  const int32_t *budget, uint8_t *keep, int32_t *pairs, int32_t *pair_count,
                                  int64_t pair_cap, hipStream_t st) {
  StreamArgs a{};
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
  a.pairs = pairs;
  a.pair_count = pair_count;
  a.P = pair_cap;
  hipError_t e = stream_reg_attrs();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(b.L * b.Hkv), (unsigned)b.S);
  stream_reg_kernel<true, true, true><<<grid, kStreamThreads, kScoreLds, st>>>(a);
  return hipGetLastError();
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
  hipError_t e = stream_reg_attrs();
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)(b.L * b.Hkv), (unsigned)b.S);
  if (lrfu && select) stream_reg_kernel<true, true, false><<<grid, kStreamThreads, kScoreLds, st>>>(a);
  else if (lrfu) stream_reg_kernel<true, false, false><<<grid, kStreamThreads, kScoreLds, st>>>(a);
  else stream_reg_kernel<false, true, false><<<grid, kStreamThreads, kScoreLds, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
