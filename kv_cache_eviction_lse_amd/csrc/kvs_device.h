// Device helpers for the per-stream kernels (one 1024-thread workgroup per stream).
#pragma once

#include "kvs_internal.h"

namespace kvs {

constexpr int kStreamThreads = 1024;
constexpr int kStreamWaves = kStreamThreads / 64;

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, d);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), d);
    v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v &= __shfl_xor(v, d);
  return v;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v |= __shfl_xor(v, d);
  return v;
}

// Block-wide reductions through a small LDS scratch (kStreamWaves slots).  Every
// thread of the block must call them; all threads receive the result.
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t *scratch) {
  v = wave_sum_u64(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[wave] = v;
  __syncthreads();
  uint64_t t = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += scratch[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ void block_and_or(uint32_t &a, uint32_t &o, uint32_t *scratch) {
  a = wave_and(a);
  o = wave_or(o);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { scratch[2 * wave] = a; scratch[2 * wave + 1] = o; }
  __syncthreads();
  uint32_t ra = ~0u, ro = 0u;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) { ra &= scratch[2 * w]; ro |= scratch[2 * w + 1]; }
  __syncthreads();
  a = ra;
  o = ro;
}

// Exclusive rank of this thread's flag among all flags of the block in thread order,
// plus the block total.  One barrier pair.
__device__ __forceinline__ uint32_t block_flag_rank(bool flag, uint32_t &total, uint32_t *scratch) {
  const uint64_t m = __ballot(flag);
  const int wave = threadIdx.x >> 6;
  const uint32_t in_wave = __popcll(m & lanemask_lt());
  if ((threadIdx.x & 63) == 0) scratch[wave] = __popcll(m);
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    const uint32_t c = scratch[w];
    before += (w < wave) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return before + in_wave;
}

// floor(s * 2^32) for a finite fp32 s >= 0, from its bit pattern.  Negative values,
// infinities and NaNs (outside the kernel contract) count as zero mass.
__device__ __forceinline__ uint64_t fixed_mass(uint32_t bits) {
  if (bits & 0x80000000u) return 0;
  const uint32_t e = bits >> 23;
  if (e == 255) return 0;
  const uint64_t mant = (bits & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  const int sh = (int)(e ? e : 1u) - 118;     // s * 2^32 = mant * 2^(E - 118)
  if (sh >= 0) return sh < 40 ? (mant << sh) : 0;
  return sh > -64 ? (mant >> (-sh)) : 0;
}

// Address of the CRF of live slot j of a stream.
__device__ __forceinline__ float *crf_slot(float *crf, const int32_t *bt_row, int32_t start, int32_t j,
                                           int32_t l, int32_t g, int64_t num_pages, int32_t Hkv) {
  const int32_t pos = start + j;
  const int64_t phys = bt_row[pos >> 4];
  return crf + (((int64_t)l * num_pages + phys) * Hkv + g) * kPage + (pos & 15);
}

// Add v into an LDS histogram bin.  Lanes whose bin equals the first valid lane's
// bin are summed in registers first (one atomic for them), which removes the
// contention of value distributions concentrated in one bin; the other lanes add
// directly.
__device__ __forceinline__ void hist_add_u64(uint64_t *hist, bool valid, uint32_t bin, uint64_t v) {
  const uint64_t mask = __ballot(valid);
  if (mask == 0) return;
  const int leader = __ffsll((long long)mask) - 1;
  const uint32_t lb = __shfl(bin, leader);
  const bool same = valid && bin == lb;
  const uint64_t agg = wave_sum_u64(same ? v : 0ull);
  if ((int)(threadIdx.x & 63) == leader) atomicAdd((unsigned long long *)&hist[lb], (unsigned long long)agg);
  if (valid && !same) atomicAdd((unsigned long long *)&hist[bin], (unsigned long long)v);
}

__device__ __forceinline__ void hist_add_u32(uint32_t *hist, bool valid, uint32_t bin) {
  const uint64_t mask = __ballot(valid);
  if (mask == 0) return;
  const int leader = __ffsll((long long)mask) - 1;
  const uint32_t lb = __shfl(bin, leader);
  const bool same = valid && bin == lb;
  const uint64_t sm = __ballot(same);
  if ((int)(threadIdx.x & 63) == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(sm));
  if (valid && !same) atomicAdd(&hist[bin], 1u);
}

}  // namespace kvs
