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
// A level is skipped when every tied entry is kept.
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
  int32_t cache_cap;
  int32_t bt_cap;
};

constexpr int kU = 16;
constexpr int kBtCap = 4096;
constexpr int kCacheCap = 35 * 1024;

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
  const bool cached = n <= a.cache_cap;
  uint32_t *c_cache = dyn;
  int32_t *bt_lds = (int32_t *)(dyn + a.cache_cap);
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
  const SelResult r1 = radix_select32<true>(n, crf_of, all, one, (uint64_t)K, band, bor, sh);
  const uint32_t cstar = r1.key;
  const uint64_t need = K - r1.above;                 // entries to keep among CRF == c*
  const bool lvl2 = need < r1.at;
  uint32_t sstar = 0;
  uint64_t need2 = 0, at2 = 0;
  if (lvl2) {
    // level 2: s among the CRF ties
    uint32_t sa = ~0u, so = 0u;
    for (int32_t base = 0; base < n; base += kU * (int32_t)blockDim.x) {
      uint32_t c[kU], v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        c[u] = j < n ? crf_of(j) : ~cstar;
        v[u] = j < n ? sp[j] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (c[u] == cstar) { sa &= v[u]; so |= v[u]; }
    }
    block_and_or(sa, so, (uint32_t *)sh.scratch);
    auto s_of = [&](int32_t j) -> uint32_t { return sp[j]; };
    auto in_tie = [&](int32_t j) { return crf_of(j) == cstar; };
    const SelResult r2 = radix_select32<true>(n, s_of, in_tie, one, need, sa, so, sh);
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
        c[u] = j < n ? crf_of(j) : 0u;
        v[u] = (lvl2 && j < n) ? sp[j] : 0u;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        if (j < n) {
          const bool k = lvl2 ? (c[u] > cstar || (c[u] == cstar && v[u] >= sstar)) : c[u] >= cstar;
          kp[j] = k ? 1 : 0;
        }
      }
    }
  } else {
    uint64_t carry = 0;
    for (int32_t base = 0; base < n; base += blockDim.x) {
      const int32_t j = base + threadIdx.x;
      const bool valid = j < n;
      const uint32_t c = valid ? crf_of(j) : 0u;
      const uint32_t s = valid && c == cstar ? sp[j] : 0u;
      const bool tie = valid && c == cstar && s == sstar;
      uint32_t tot;
      const uint32_t rk = block_flag_rank(tie, tot, flag_scratch);
      const bool k = valid && (c > cstar || (c == cstar && (s > sstar || (tie && carry + rk < need2))));
      carry += tot;
      if (valid) kp[j] = k ? 1 : 0;
    }
  }
}

}  // namespace

hipError_t launch_select(const kvs_cache &c, const Batch &b, const float *scores,
                         const int32_t *budget, uint8_t *keep, int32_t max_len, hipStream_t st,
                         const float *keys) {
  static bool attr_set = false;
  const int32_t cache = max_len <= kCacheCap ? max_len : 0;
  const size_t dyn = ((size_t)cache + kBtCap) * sizeof(uint32_t);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (kCacheCap + kBtCap) * 4);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  SelectArgs a{};
  a.scores = scores;
  a.crf = c.crf;
  a.budget = budget;
  a.keep = keep;
  a.keys = keys;
  a.b = b;
  a.cache_cap = cache;
  a.bt_cap = kBtCap;
  dim3 grid((unsigned)(b.L * b.Hkv), (unsigned)b.S);
  select_kernel<<<grid, kStreamThreads, dyn, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
