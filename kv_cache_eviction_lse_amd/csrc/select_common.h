// Radix selection over 32-bit keys inside one 1024-thread workgroup.
//
// Keys are bit patterns of non-negative fp32 values, so unsigned order is value
// order.  Each entry carries a weight (attention mass for the cut, 1 for top-B).
// Given a target W > 0, the search finds the key v* such that
//     weight(keys > v*) < W <= weight(keys >= v*)
// among the entries that pass a predicate.  Bits that all candidates share (found
// from the AND and OR of their keys) are skipped; the rest is resolved 8 bits per
// pass with an LDS histogram.
#pragma once

#include "kvs_device.h"

namespace kvs {

struct SelResult {
  uint32_t key;        // v*
  uint64_t above;      // weight of candidates with key > v*
  uint64_t at;         // weight of candidates with key == v*
};

struct SelShared {
  uint64_t hist[256];
  uint64_t scratch[kStreamWaves];
  uint64_t found[4];
};

// key_of(j) -> uint32 key; ok(j) -> candidate?; weight_of(key) -> uint64.
// COUNT: every weight is 1 (weight_of is not called in the histogram passes).
template <bool COUNT, typename KeyF, typename OkF, typename WF>
__device__ __forceinline__ SelResult radix_select32(int32_t n, KeyF key_of, OkF ok, WF weight_of, uint64_t target,
                                    uint32_t and_all, uint32_t or_all, SelShared &sh) {
  SelResult r;
  const uint32_t diff = and_all ^ or_all;
  if (diff == 0) {
    // every candidate has the same key
    uint64_t w = 0;
    for (int32_t j = threadIdx.x; j < n; j += blockDim.x)
      if (ok(j)) w += weight_of(key_of(j));
    w = block_sum_u64(w, sh.scratch);
    r.key = and_all;
    r.above = 0;
    r.at = w;
    return r;
  }
  int top = 31 - __clz(diff);
  uint32_t prefix = top == 31 ? 0u : (and_all & ~((2u << top) - 1u));
  uint64_t need = target;
  uint64_t above = 0, at = 0;
  const int lane = threadIdx.x & 63;
  while (top >= 0) {
    const int width = top + 1 < 8 ? top + 1 : 8;
    const int lo = top - width + 1;
    const uint32_t nb = 1u << width;
    for (int b = threadIdx.x; b < 256; b += blockDim.x) sh.hist[b] = 0;
    __syncthreads();
    const int hs = top + 1;
    // 8 keys per thread per round, loaded before any is used (latency overlap)
    constexpr int U = 8;
    for (int32_t base = 0; base < n; base += U * (int32_t)blockDim.x) {
      uint32_t keys[U];
      bool ok_[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int32_t j = base + u * (int32_t)blockDim.x + (int32_t)threadIdx.x;
        ok_[u] = j < n && ok(j);
        keys[u] = ok_[u] ? key_of(j) : 0u;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t key = keys[u];
        const bool v = ok_[u] && (hs >= 32 ? true : ((key >> hs) == (prefix >> hs)));
        const uint32_t bin = (key >> lo) & (nb - 1u);
        if (COUNT) hist_add_count(sh.hist, v, bin);
        else hist_add_u64(sh.hist, v, bin, v ? weight_of(key) : 0ull);
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane L owns bins nb-1-4L .. nb-4-4L (descending), so an exclusive prefix sum
      // over lanes is the weight of all higher bins
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

}  // namespace kvs
