// kvs_select: per-(layer, KV head) top-B keep set, one workgroup per stream.
//
// ActKV Dissected, Summary / Results: eviction keeps an entry budget.  Exactly
// K = min(B, n) entries are kept per stream: the first K of the order
// (CRF desc, s desc, slot asc) on fp32 bit patterns (step-aware ranking passes keys per
// entry in place of the CRF).  Selection runs in up to three
// levels, each only over the entries still tied:
//   1. radix-select the K-th largest CRF value c* (CRF cached in LDS when it fits);
//   2. among CRF == c*, radix-select s* so that the remaining count is met;
//   3. among (c*, s*) ties, take the lowest slots (ballot scan in slot order).
// A level is skipped when every tied entry is kept.  Streams too long for the CRF cache
// (up to kMaskCap entries) keep two LDS bitmasks from level 1 (CRF above c*, CRF equal
// to c*), so the later passes read only the scores; level 1 skips the bits a large
// crossing bin shares (select_crf_jump), and level 2 finishes in an LDS list
// (select_count_list).
#include "select_common.h"

namespace kvs {
namespace {

struct SelectArgs {
  const float *scores;
  const float *crf;
  const int32_t *budget;
  uint8_t *keep;
  const float *keys;      // nullable: keys per entry [L*Hkv][E] in place of the CRF
  Batch b;
  int32_t cache_cap;     // entries per stream of the CRF cache (0: none)
  int32_t mask_cap;      // entries per stream of the level-1 masks (0: none)
  int32_t front_words;   // LDS words before the block table
  int32_t bt_cap;        // block-table entries per stream kept in LDS
};

constexpr int kU = 16;
constexpr int kBtCap = 16384;          // block-table entries per stream kept in LDS
constexpr int kCacheCap = 35 * 1024;   // CRF values (or keys) per stream kept in LDS
constexpr int kMaskCap = 1 << 18;      // entries per stream with the level-1 masks in LDS
constexpr uint64_t kJumpMin = 4096;    // crossing-bin size from which its AND/OR is taken

__device__ __forceinline__ bool mask_bit(const uint32_t *m, int32_t j) { return (m[j >> 5] >> (j & 31)) & 1u; }

// Writes one word of the bitmask m: the bits of the 32 consecutive entries of this
// thread's half wave, starting at entry j0 (a multiple of 32; every lane of the half wave
// passes the same j0).  Lanes 0 and 32 store the two halves of the ballot, so no atomics
// are needed.  Callers pass bit = 0 for entries past n.
__device__ __forceinline__ void store_mask_bits(uint32_t *m, int32_t j0, bool bit) {
  const uint64_t b = ballot(bit);
  const int lane = threadIdx.x & 63;
  if (lane == 0) m[j0 >> 5] = (uint32_t)b;
  if (lane == 32) m[j0 >> 5] = (uint32_t)(b >> 32);
}

// Level 1 for a stream whose CRF values are not in LDS: radix_select32's search with a
// jump.  After a pass, when the crossing bin holds more than kJumpMin entries, one more
// pass takes their AND and OR and writes the masks gt (key above the bin) and in (key in
// the bin).  Equal AND and OR: the bin is one key, the search ends, and the masks are
// those of the result (*masks_ok).  Otherwise the next pass starts at the highest bit in
// which the bin's keys differ.  At the 70B shape after a first update every CRF is 0 or
// 1, and this ends the search after one histogram pass instead of four.
template <typename KeyF>
__device__ __forceinline__ SelResult select_crf_jump(int32_t n, KeyF key_of, uint64_t target, uint32_t and_all, uint32_t or_all,
                                     SelShared &sh, uint32_t *m_gt, uint32_t *m_in, bool *masks_ok) {
  SelResult r;
  *masks_ok = false;
  const uint32_t diff = and_all ^ or_all;
  if (diff == 0) {
    r.key = and_all;
    r.above = 0;
    r.at = (uint64_t)n;
    return r;
  }
  int top = 31 - __clz(diff);
  uint32_t prefix = top == 31 ? 0u : (and_all & ~((2u << top) - 1u));
  uint64_t need = target, above = 0, at = 0;
  const int lane = threadIdx.x & 63;
  while (top >= 0) {
    const int width = top + 1 < 8 ? top + 1 : 8;
    const int lo = top - width + 1;
    const uint32_t nb = 1u << width;
    for (int b = threadIdx.x; b < 256; b += blockDim.x) sh.hist[b] = 0;
    __syncthreads();
    const int hs = top + 1;
    constexpr int U = 8;
    for (int32_t base = 0; base < n; base += U * (int32_t)blockDim.x) {
      uint32_t keys[U];
      bool ok_[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        ok_[u] = j < n;
        keys[u] = ok_[u] ? key_of(j) : 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t key = keys[u];
        const bool v = ok_[u] && (hs >= 32 ? true : ((key >> hs) == (prefix >> hs)));
        hist_add_count(sh.hist, v, (key >> lo) & (nb - 1u));
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      uint64_t h[4], ls = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = (int)nb - 1 - (4 * lane + q);
        h[q] = b >= 0 ? sh.hist[b] : 0ull;
        ls += h[q];
      }
      uint64_t acc = wave_scan_u64(ls) - ls;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = (int)nb - 1 - (4 * lane + q);
        if (b >= 0 && acc < need && need <= acc + h[q]) {
          sh.found[0] = (uint64_t)b;
          sh.found[1] = acc;
          sh.found[2] = h[q];
        }
        acc += h[q];
      }
    }
    __syncthreads();
    const uint32_t b = (uint32_t)sh.found[0];
    const uint64_t ab = sh.found[1];
    at = sh.found[2];
    __syncthreads();
    prefix |= b << lo;
    need -= ab;
    above += ab;
    top = lo - 1;
    if (top < 0 || at <= kJumpMin) continue;
    // the crossing bin's AND and OR, and the masks relative to the bin
    const uint32_t pb = prefix >> lo;
    uint32_t ba = ~0u, bo = 0u;
    for (int32_t base = 0; base < n; base += kU * (int32_t)blockDim.x) {
      uint32_t keys[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        keys[u] = j < n ? key_of(j) : 0u;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        const bool inb = j < n && (keys[u] >> lo) == pb;
        const bool gt = j < n && (keys[u] >> lo) > pb;
        if (inb) {
          ba &= keys[u];
          bo |= keys[u];
        }
        const int32_t j0 = base + u * (int32_t)blockDim.x + (int32_t)(threadIdx.x & ~63u) + (lane & 32);
        if (j0 < n) {
          store_mask_bits(m_gt, j0, gt);
          store_mask_bits(m_in, j0, inb);
        }
      }
    }
    block_and_or(ba, bo, (uint32_t *)sh.scratch);
    if (ba == bo) {
      *masks_ok = true;
      r.key = ba;
      r.above = above;
      r.at = at;
      return r;
    }
    top = 31 - __clz(ba ^ bo);
    prefix = ba & ~((2u << top) - 1u);
  }
  r.key = prefix;
  r.above = above;
  r.at = at;
  return r;
}

// Level 2 for a stream with the level-1 masks: radix_select32's count search over the
// scores of the candidates (ok), finished in LDS.  After a pass whose crossing bin holds
// at most cap candidates, their scores are gathered into `list` (each wave reserves its
// range with one LDS atomic per group of kU rows) and the search continues over the
// list, so the remaining 8-bit passes read at most cap keys from LDS instead of every
// score from HBM.
template <typename SF, typename OkF>
__device__ __forceinline__ SelResult select_count_list(int32_t n, SF s_of, OkF ok, uint64_t target, uint32_t and_all,
                                       uint32_t or_all, SelShared &sh, uint32_t *list, int32_t cap) {
  auto one = [](uint32_t) -> uint64_t { return 1; };
  const uint32_t diff = and_all ^ or_all;
  if (diff == 0 || cap <= 0) return radix_select32<true>(n, s_of, ok, one, target, and_all, or_all, sh);
  int top = 31 - __clz(diff);
  uint32_t prefix = top == 31 ? 0u : (and_all & ~((2u << top) - 1u));
  uint64_t need = target, above = 0, at = 0;
  const int lane = threadIdx.x & 63;
  while (top >= 0) {
    const int width = top + 1 < 8 ? top + 1 : 8;
    const int lo = top - width + 1;
    const uint32_t nb = 1u << width;
    for (int b = threadIdx.x; b < 256; b += blockDim.x) sh.hist[b] = 0;
    __syncthreads();
    const int hs = top + 1;
    constexpr int U = 8;
    for (int32_t base = 0; base < n; base += U * (int32_t)blockDim.x) {
      uint32_t keys[U];
      bool ok_[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        ok_[u] = j < n && ok(j);
        keys[u] = ok_[u] ? s_of(j) : 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t key = keys[u];
        const bool v = ok_[u] && (hs >= 32 ? true : ((key >> hs) == (prefix >> hs)));
        hist_add_count(sh.hist, v, (key >> lo) & (nb - 1u));
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      uint64_t h[4], ls = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = (int)nb - 1 - (4 * lane + q);
        h[q] = b >= 0 ? sh.hist[b] : 0ull;
        ls += h[q];
      }
      uint64_t acc = wave_scan_u64(ls) - ls;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = (int)nb - 1 - (4 * lane + q);
        if (b >= 0 && acc < need && need <= acc + h[q]) {
          sh.found[0] = (uint64_t)b;
          sh.found[1] = acc;
          sh.found[2] = h[q];
        }
        acc += h[q];
      }
    }
    __syncthreads();
    const uint32_t b = (uint32_t)sh.found[0];
    const uint64_t ab = sh.found[1];
    at = sh.found[2];
    __syncthreads();
    prefix |= b << lo;
    need -= ab;
    above += ab;
    top = lo - 1;
    if (top < 0 || at > (uint64_t)cap) continue;
    // gather the crossing bin's keys into the list
    uint32_t *cnt = (uint32_t *)&sh.found[3];
    if (threadIdx.x == 0) *cnt = 0u;
    __syncthreads();
    const uint32_t pb = prefix >> lo;
    for (int32_t base = 0; base < n; base += kU * (int32_t)blockDim.x) {
      uint32_t keys[kU];
      bool take[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        take[u] = j < n && ok(j);
        keys[u] = take[u] ? s_of(j) : 0u;
      }
      uint64_t m[kU];
      uint32_t tot = 0;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        take[u] = take[u] && (keys[u] >> lo) == pb;
        m[u] = ballot(take[u]);
        tot += (uint32_t)__popcll(m[u]);
      }
      uint32_t wb = 0;
      if (lane == 0 && tot) wb = atomicAdd(cnt, tot);
      wb = (uint32_t)__shfl((int)wb, 0);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const uint32_t x = wb + (uint32_t)__popcll(m[u] & lanemask_lt());
        if (take[u] && x < (uint32_t)cap) list[x] = keys[u];
        wb += (uint32_t)__popcll(m[u]);
      }
    }
    __syncthreads();
    const int32_t nl = (int32_t)min(*cnt, (uint32_t)cap);    // (= at)
    uint32_t la = ~0u, lor = 0u;
    for (int32_t x = threadIdx.x; x < nl; x += blockDim.x) {
      la &= list[x];
      lor |= list[x];
    }
    block_and_or(la, lor, (uint32_t *)sh.scratch);
    auto l_of = [&](int32_t x) -> uint32_t { return list[x]; };
    auto all = [](int32_t) { return true; };
    const SelResult r2 = radix_select32<true>(nl, l_of, all, one, need, la, lor, sh);
    SelResult r;
    r.key = r2.key;
    r.above = above + r2.above;
    r.at = r2.at;
    return r;
  }
  SelResult r;
  r.key = prefix;
  r.above = above;
  r.at = at;
  return r;
}

__global__ __launch_bounds__(kStreamThreads) void select_kernel(SelectArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  __shared__ SelShared sh;
  __shared__ uint32_t flag_scratch[kStreamWaves];

  const int32_t i = blockIdx.y;
  const int32_t lg = blockIdx.x;
  const int32_t n = a.b.len[i];
  if (n <= 0) return;
  const int32_t l = lg / a.b.Hkv;
  const int32_t g = lg - l * a.b.Hkv;
  const int64_t e0 = a.b.entry_off[i];
  const int32_t start = a.b.start[i];
  const int32_t *bt_row = a.b.bt + (int64_t)i * a.b.max_pages;
  const uint32_t *sp = (const uint32_t *)(a.scores + (int64_t)lg * a.b.E + e0);
  uint8_t *kp = a.keep + (int64_t)lg * a.b.E + e0;
  const int32_t bud = a.budget[i];
  const int32_t K = bud < n ? (bud > 0 ? bud : 0) : n;
  if (K == 0 || K == n) {
    const uint8_t v = K == n ? 1 : 0;
    for (int32_t j = threadIdx.x; j < n; j += blockDim.x) kp[j] = v;
    return;
  }
  // dynamic LDS: [front words: the CRF cache, or the two level-1 masks][block table]
  const bool cached = n <= a.cache_cap;
  const bool masked = !cached && n <= a.mask_cap;
  uint32_t *c_cache = dyn;
  const int32_t mwords = (a.mask_cap + 31) >> 5;
  uint32_t *m_gt = dyn;              // CRF > c*
  uint32_t *m_eq = dyn + mwords;     // CRF == c*
  int32_t *bt_lds = (int32_t *)(dyn + a.front_words);
  const int32_t npages = (start + n + kPage - 1) / kPage;
  const bool bt_cached = npages <= a.bt_cap;
  if (bt_cached) {
    for (int32_t p = threadIdx.x; p < npages; p += blockDim.x) bt_lds[p] = bt_row[p];
    __syncthreads();
  }
  const int32_t *bt_use = bt_cached ? bt_lds : bt_row;
  const uint32_t *crf_base = (const uint32_t *)a.crf + (((int64_t)l * a.b.num_pages) * a.b.Hkv + g) * kPage;
  const int64_t page_stride = (int64_t)a.b.Hkv * kPage;
  const uint32_t *kflat = a.keys ? (const uint32_t *)(a.keys + (int64_t)lg * a.b.E + e0) : nullptr;
  auto crf_addr = [&](int32_t j) -> const uint32_t * {
    if (kflat) return kflat + j;
    const int32_t pos = start + j;
    return crf_base + (int64_t)bt_use[pos >> 4] * page_stride + (pos & 15);
  };

  uint32_t band = ~0u, bor = 0u;
  for (int32_t base = 0; base < n; base += kU * (int32_t)blockDim.x) {
    uint32_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
      v[u] = j < n ? *crf_addr(j) : 0u;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
      if (j < n) {
        if (cached) c_cache[j] = v[u];
        band &= v[u];
        bor |= v[u];
      }
    }
  }
  block_and_or(band, bor, (uint32_t *)sh.scratch);
  auto crf_of = [&](int32_t j) -> uint32_t { return cached ? c_cache[j] : *crf_addr(j); };
  auto one = [](uint32_t) -> uint64_t { return 1; };
  auto all = [](int32_t) { return true; };

  // level 1: CRF
  SelResult r1;
  bool masks_ok = false;
  if (masked) {
    r1 = select_crf_jump(n, crf_of, (uint64_t)K, band, bor, sh, m_gt, m_eq, &masks_ok);
  } else {
    r1 = radix_select32<true>(n, crf_of, all, one, (uint64_t)K, band, bor, sh);
  }
  const uint32_t cstar = r1.key;
  const uint64_t need = K - r1.above;                 // entries to keep among CRF == c*
  const bool lvl2 = need < r1.at;
  if (masked && !masks_ok) {
    // the masks of c* (one pass over the CRF values)
    __syncthreads();
    const int lane = threadIdx.x & 63;
    for (int32_t base = 0; base < n; base += kU * (int32_t)blockDim.x) {
      uint32_t v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        v[u] = j < n ? crf_of(j) : 0u;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        const int32_t j0 = base + u * (int32_t)blockDim.x + (int32_t)(threadIdx.x & ~63u) + (lane & 32);
        if (j0 < n) {
          store_mask_bits(m_gt, j0, j < n && v[u] > cstar);
          store_mask_bits(m_eq, j0, j < n && v[u] == cstar);
        }
      }
    }
  }
  if (masked) __syncthreads();     // the masks are complete
  // CRF above c* / equal to c*: from the masks, else from the values
  auto above_c = [&](int32_t j, uint32_t c) -> bool { return masked ? mask_bit(m_gt, j) : c > cstar; };
  auto at_c = [&](int32_t j, uint32_t c) -> bool { return masked ? mask_bit(m_eq, j) : c == cstar; };
  auto crf_if = [&](int32_t j) -> uint32_t { return masked ? 0u : crf_of(j); };
  uint32_t sstar = 0;
  uint64_t need2 = 0, at2 = 0;
  if (lvl2) {
    // level 2: s among the CRF ties
    uint32_t sa = ~0u, so = 0u;
    for (int32_t base = 0; base < n; base += kU * (int32_t)blockDim.x) {
      bool t[kU];
      uint32_t v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        t[u] = j < n && at_c(j, crf_if(j));
        v[u] = t[u] ? sp[j] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (t[u]) { sa &= v[u]; so |= v[u]; }
    }
    block_and_or(sa, so, (uint32_t *)sh.scratch);
    auto s_of = [&](int32_t j) -> uint32_t { return sp[j]; };
    auto in_tie = [&](int32_t j) { return at_c(j, crf_if(j)); };
    // (with the masks, the block-table row is no longer read: its LDS holds the list)
    const SelResult r2 = masked ? select_count_list(n, s_of, in_tie, need, sa, so, sh, (uint32_t *)bt_lds, a.bt_cap)
                                : radix_select32<true>(n, s_of, in_tie, one, need, sa, so, sh);
    sstar = r2.key;
    need2 = need - r2.above;
    at2 = r2.at;
  }
  const bool lvl3 = lvl2 && need2 < at2;

  if (!lvl3) {
    for (int32_t base = 0; base < n; base += kU * (int32_t)blockDim.x) {
      uint32_t c[kU], v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        c[u] = j < n ? crf_if(j) : 0u;
        v[u] = (lvl2 && j < n && at_c(j, c[u])) ? sp[j] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        if (j < n) {
          const bool gt = above_c(j, c[u]), eq = at_c(j, c[u]);
          const bool k = lvl2 ? (gt || (eq && v[u] >= sstar)) : (gt || eq);
          kp[j] = k ? 1 : 0;
        }
      }
    }
  } else {
    uint64_t carry = 0;
    for (int32_t base = 0; base < n; base += blockDim.x) {
      const int32_t j = base + threadIdx.x;
      const bool valid = j < n;
      const uint32_t c = valid ? crf_if(j) : 0u;
      const bool gt = valid && above_c(j, c), eq = valid && at_c(j, c);
      const uint32_t s = eq ? sp[j] : 0u;
      const bool tie = eq && s == sstar;
      uint32_t tot;
      const uint32_t rk = block_flag_rank(tie, tot, flag_scratch);
      const bool k = gt || (eq && (s > sstar || (tie && carry + rk < need2)));
      carry += tot;
      if (valid) kp[j] = k ? 1 : 0;
    }
  }
}

}  // namespace

hipError_t launch_select(const kvs_cache &c, const Batch &b, const float *scores,
                         const int32_t *budget, uint8_t *keep, int32_t max_len, hipStream_t st,
                         const float *keys) {
  // LDS: the CRF cache (streams up to kCacheCap entries) or the level-1 masks (up to
  // kMaskCap), then the block-table row when it fits in what is left of 160 KiB
  constexpr int32_t kLdsWords = 156 * 1024 / 4;
  const int32_t cache = max_len <= kCacheCap ? max_len : 0;
  const int32_t mask = cache == 0 && max_len <= kMaskCap ? max_len : 0;
  const int32_t front = cache > 0 ? cache : 2 * ((mask + 31) >> 5);
  int32_t bt = max_len / kPage + 2;       // pages of a stream of max_len entries at any start
  if (bt > kBtCap) bt = kBtCap;
  if (front + bt > kLdsWords) bt = kLdsWords - front;
  const size_t dyn = ((size_t)front + (size_t)bt) * sizeof(uint32_t);
  static bool done[64] = {};
  const void *fn = (const void *)select_kernel;
  const hipError_t e = raise_lds_limit(&fn, 1, kLdsWords * 4, done);
  if (e != hipSuccess) return e;
  SelectArgs a{};
  a.scores = scores;
  a.crf = c.crf;
  a.budget = budget;
  a.keep = keep;
  a.keys = keys;
  a.b = b;
  a.cache_cap = cache;
  a.mask_cap = mask;
  a.front_words = front;
  a.bt_cap = bt;
  dim3 grid((unsigned)(b.L * b.Hkv), (unsigned)b.S);
  select_kernel<<<grid, kStreamThreads, dyn, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
