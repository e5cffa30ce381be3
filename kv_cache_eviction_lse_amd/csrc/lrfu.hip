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
// order, only when not every tie is a hit).  Streams with n <= ~39 K entries keep
// s in LDS for all passes; longer streams re-read it from global memory (L2).
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
  int32_t cache_cap;
};

__global__ __launch_bounds__(kStreamThreads) void lrfu_kernel(LrfuArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t s_cache[];
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

  uint64_t msum = 0;
  uint32_t band = ~0u, bor = 0u;
  for (int32_t j = threadIdx.x; j < n; j += blockDim.x) {
    const uint32_t bits = sp[j];
    if (cached) s_cache[j] = bits;
    msum += fixed_mass(bits);
    band &= bits;
    bor |= bits;
  }
  const uint64_t M = block_sum_u64(msum, sh.scratch);
  block_and_or(band, bor, (uint32_t *)sh.scratch);
  const uint64_t T = (M / a.den) * a.num + ((M % a.den) * a.num + a.den - 1) / a.den;

  auto key_of = [&](int32_t j) -> uint32_t { return cached ? s_cache[j] : sp[j]; };
  auto all = [](int32_t) { return true; };

  bool none = T == 0;
  uint32_t vstar = 0xFFFFFFFFu;
  uint64_t k_needed = 0, ties = 0;
  if (!none) {
    const SelResult r = radix_select32(n, key_of, all, fixed_mass, T, band, bor, sh);
    vstar = r.key;
    const uint64_t mstar = fixed_mass(vstar);
    k_needed = (T - r.above + mstar - 1) / mstar;
    ties = r.at / mstar;
  }
  const bool rank_ties = !none && k_needed < ties;

  const float d = a.decay[i];
  const int32_t np = a.n_prev[i];
  uint64_t carry = 0;
  for (int32_t base = 0; base < n; base += blockDim.x) {
    const int32_t j = base + threadIdx.x;
    const bool valid = j < n;
    const uint32_t bits = valid ? key_of(j) : 0u;
    bool h;
    if (rank_ties) {
      const bool tie = valid && bits == vstar;
      uint32_t tot;
      const uint32_t rk = block_flag_rank(tie, tot, flag_scratch);
      h = bits > vstar || (tie && carry + rk < k_needed);
      carry += tot;
    } else {
      h = !none && bits >= vstar;
    }
    if (valid) {
      float *cp = crf_slot(a.crf, bt_row, start, j, l, g, a.b.num_pages, a.b.Hkv);
      const float prior = j < np ? *cp : 0.f;
      *cp = __builtin_fmaf(d, prior, h ? 1.f : 0.f);
      if (a.hit) a.hit[(int64_t)lg * a.b.E + e0 + j] = h ? 1 : 0;
    }
  }
}

}  // namespace

hipError_t launch_lrfu(const kvs_cache &c, const Batch &b, const float *scores, uint32_t num,
                       uint32_t den, const float *decay, const int32_t *n_prev, uint8_t *hit,
                       int32_t max_len, hipStream_t st) {
  static bool attr_set = false;
  const int32_t cap = 39 * 1024;
  const size_t dyn = (size_t)(max_len <= cap ? max_len : 0) * sizeof(uint32_t);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)lrfu_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, cap * 4);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  LrfuArgs a{};
  a.scores = scores;
  a.crf = c.crf;
  a.hit = hit;
  a.decay = decay;
  a.n_prev = n_prev;
  a.b = b;
  a.num = num;
  a.den = den;
  a.cache_cap = max_len <= cap ? max_len : 0;
  dim3 grid((unsigned)(b.L * b.Hkv), (unsigned)b.S);
  lrfu_kernel<<<grid, kStreamThreads, dyn, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
