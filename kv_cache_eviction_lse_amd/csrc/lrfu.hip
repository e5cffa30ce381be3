// kvs_lrfu_update: the attention-mass cut and the LRFU update, one workgroup per stream.
//
// ActKV Dissected, Component 1: the attention each entry receives from all action
// tokens is tallied; entries in the top 90 % are "action-critical" (here: the
// shortest prefix of the (s desc, slot asc) order holding >= 90 % of the integer
// attention mass); that hit signal drives LRFU with lambda = 0.5:
//     CRF <- hit + 2^(-lambda dt) * CRF       (one fp32 fma, decay given per sequence)
// Entries appended since the previous round (slot >= n_prev) start from CRF 0.
//
// The threshold v* is found by radix selection on the fp32 bit patterns of s with
// the integer mass m = floor(s * 2^32) as weight, so the result does not depend on
// summation order.  Ties at v* take the lowest slots first (a ballot scan in slot
// order, only when not every tie is a hit).  Streams with n <= 35 K entries keep
// s in LDS for all passes; longer streams re-read it from global memory (L2).  The
// block-table row is staged in LDS and the streaming loops keep 8 loads in flight
// per thread.
#include "select_common.h"

namespace kvs {
namespace {

struct LrfuArgs {
  const float *scores;
  float *crf;
  uint8_t *hit;
  const float *decay;
  const int32_t *n_prev;
  Batch b;
  uint32_t num, den;
  int32_t cache_cap;   // scores cached in LDS when n <= cache_cap
  int32_t bt_cap;      // block-table row cached in LDS when npages <= bt_cap
};

constexpr int kU = 16;             // loads in flight per thread in the streaming passes
constexpr int kBtCap = 16384;      // block-table entries per stream kept in LDS
constexpr int kCacheCap = 35 * 1024;

__global__ __launch_bounds__(kStreamThreads) void lrfu_kernel(LrfuArgs a) {
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
  const bool cached = n <= a.cache_cap;
  uint32_t *s_cache = dyn;
  int32_t *bt_lds = (int32_t *)(dyn + a.cache_cap);
  const int32_t npages = (start + n + kPage - 1) / kPage;
  const bool bt_cached = npages <= a.bt_cap;
  if (bt_cached)
    for (int32_t p = threadIdx.x; p < npages; p += blockDim.x) bt_lds[p] = bt_row[p];
  const int32_t *bt_use = bt_cached ? bt_lds : bt_row;

  uint64_t msum = 0;
  uint32_t band = ~0u, bor = 0u;
  for (int32_t base = 0; base < n; base += kU * (int32_t)blockDim.x) {
    uint32_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
      v[u] = j < n ? sp[j] : 0u;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
      if (j < n) {
        if (cached) s_cache[j] = v[u];
        msum += fixed_mass(v[u]);
        band &= v[u];
        bor |= v[u];
      }
    }
  }
  const uint64_t M = block_sum_u64(msum, sh.scratch);
  block_and_or(band, bor, (uint32_t *)sh.scratch);
  const uint64_t T = (M / a.den) * a.num + ((M % a.den) * a.num + a.den - 1) / a.den;

  auto key_of = [&](int32_t j) -> uint32_t { return cached ? s_cache[j] : sp[j]; };
  auto all = [](int32_t) { return true; };

  const bool none = T == 0;
  uint32_t vstar = 0xFFFFFFFFu;
  uint64_t k_needed = 0, ties = 0;
  if (!none) {
    const SelResult r = radix_select32<false>(n, key_of, all, fixed_mass, T, band, bor, sh);
    vstar = r.key;
    const uint64_t mstar = fixed_mass(vstar);
    k_needed = (T - r.above + mstar - 1) / mstar;
    ties = r.at / mstar;
  }
  const bool rank_ties = !none && k_needed < ties;
  const float d = a.decay[i];
  const int32_t np = a.n_prev[i];
  float *crf_base = a.crf + (((int64_t)l * a.b.num_pages) * a.b.Hkv + g) * kPage;
  const int64_t page_stride = (int64_t)a.b.Hkv * kPage;
  uint8_t *hp = a.hit ? a.hit + (int64_t)lg * a.b.E + e0 : nullptr;

  if (!rank_ties) {
    // every entry at the threshold is a hit (or there are no hits)
    for (int32_t base = 0; base < n; base += kU * (int32_t)blockDim.x) {
      float *cp[kU];
      float prior[kU];
      uint32_t bits[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        const int32_t jj = j < n ? j : 0;
        const int32_t pos = start + jj;
        cp[u] = crf_base + (int64_t)bt_use[pos >> 4] * page_stride + (pos & 15);
        bits[u] = key_of(jj);
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        prior[u] = (j < n && j < np) ? *cp[u] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        if (j < n) {
          const bool h = !none && bits[u] >= vstar;
          *cp[u] = __builtin_fmaf(d, prior[u], h ? 1.f : 0.f);
          if (hp) hp[j] = h ? 1 : 0;
        }
      }
    }
  } else {
    // ties at the threshold exceed the hits still needed: lowest slots first
    uint64_t carry = 0;
    for (int32_t base = 0; base < n; base += blockDim.x) {
      const int32_t j = base + threadIdx.x;
      const bool valid = j < n;
      const uint32_t bits = valid ? key_of(j) : 0u;
      const bool tie = valid && bits == vstar;
      uint32_t tot;
      const uint32_t rk = block_flag_rank(tie, tot, flag_scratch);
      const bool h = bits > vstar || (tie && carry + rk < k_needed);
      carry += tot;
      if (valid) {
        const int32_t pos = start + j;
        float *cp = crf_base + (int64_t)bt_use[pos >> 4] * page_stride + (pos & 15);
        const float prior = j < np ? *cp : 0.f;
        *cp = __builtin_fmaf(d, prior, h ? 1.f : 0.f);
        if (hp) hp[j] = h ? 1 : 0;
      }
    }
  }
}

}  // namespace

hipError_t launch_lrfu(const kvs_cache &c, const Batch &b, const float *scores, uint32_t num,
                       uint32_t den, const float *decay, const int32_t *n_prev, uint8_t *hit,
                       int32_t max_len, hipStream_t st) {
  // LDS: the scores (streams up to kCacheCap entries), then the block-table row when it
  // fits in what is left of 156 KiB
  constexpr int32_t kLdsWords = 156 * 1024 / 4;
  const int32_t cache = max_len <= kCacheCap ? max_len : 0;
  int32_t bt = max_len / kPage + 2;       // pages of a stream of max_len entries at any start
  if (bt > kBtCap) bt = kBtCap;
  if (cache + bt > kLdsWords) bt = kLdsWords - cache;
  const size_t dyn = ((size_t)cache + (size_t)bt) * sizeof(uint32_t);
  static bool done[64] = {};
  const void *fn = (const void *)lrfu_kernel;
  const hipError_t e = raise_lds_limit(&fn, 1, kLdsWords * 4, done);
  if (e != hipSuccess) return e;
  LrfuArgs a{};
  a.scores = scores;
  a.crf = c.crf;
  a.hit = hit;
  a.decay = decay;
  a.n_prev = n_prev;
  a.b = b;
  a.num = num;
  a.den = den;
  a.cache_cap = cache;
  a.bt_cap = bt;
  dim3 grid((unsigned)(b.L * b.Hkv), (unsigned)b.S);
  lrfu_kernel<<<grid, kStreamThreads, dyn, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
