// Device helpers for the per-stream kernels (one 1024-thread workgroup per stream).
//
// Wave-level sums and scans use DPP row shifts and row broadcasts (VALU only, no
// LDS crossbar round trips): four row_shr steps scan each 16-lane row, then
// row_bcast:15 and row_bcast:31 carry the row totals across the wave.
#pragma once

#include "kvs_internal.h"

namespace kvs {

constexpr int kStreamThreads = 1024;
constexpr int kStreamWaves = kStreamThreads / 64;

// DPP controls (gfx9 encoding)
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Workgroup barrier that orders LDS only.  The fences are scoped to the local address
// space, so a wave waits for its own LDS operations (lgkmcnt) but not for its global
// loads and stores: those stay in flight across the barrier.  Every block helper below
// exchanges data through LDS only; a kernel that passes data between its threads
// through global memory needs __syncthreads() for that.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Mask of the lanes where b holds.  (The bool goes to the builtin as the compare
// result it is; through an int it would be materialised in a VGPR and compared again.)
__device__ __forceinline__ uint64_t ballot(bool b) { return __builtin_amdgcn_ballot_w64(b); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// Inclusive prefix sum over the wave (lane i gets lanes 0..i).
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr1, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr2, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr4, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr8, 0xF, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast15, 0xA, 0xF, false);
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast31, 0xC, 0xF, false);
  return x;
}

// Wave total of a u32 (exact while the total fits in 32 bits), uniform result.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_u32(x), 63);
}

// Wave total of a u64 (mod 2^64), uniform result: DPP moves of both halves, then a
// 64-bit add with carry.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROW_MASK, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROW_MASK, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

// Inclusive prefix sum of a u64 over the wave (lane i gets lanes 0..i), mod 2^64.
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v) {
  v += dpp_u64<kRowShr1, 0xF>(v);
  v += dpp_u64<kRowShr2, 0xF>(v);
  v += dpp_u64<kRowShr4, 0xF>(v);
  v += dpp_u64<kRowShr8, 0xF>(v);
  v += dpp_u64<kRowBcast15, 0xA>(v);
  v += dpp_u64<kRowBcast31, 0xC>(v);
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  v += dpp_u64<kRowShr1, 0xF>(v);
  v += dpp_u64<kRowShr2, 0xF>(v);
  v += dpp_u64<kRowShr4, 0xF>(v);
  v += dpp_u64<kRowShr8, 0xF>(v);
  v += dpp_u64<kRowBcast15, 0xA>(v);
  v += dpp_u64<kRowBcast31, 0xC>(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_and(uint32_t x) {
  x &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, kRowShr1, 0xF, 0xF, false);
  x &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, kRowShr2, 0xF, 0xF, false);
  x &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, kRowShr4, 0xF, 0xF, false);
  x &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, kRowShr8, 0xF, 0xF, false);
  x &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, kRowBcast15, 0xA, 0xF, false);
  x &= (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)x, kRowBcast31, 0xC, 0xF, false);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr1, 0xF, 0xF, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr2, 0xF, 0xF, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr4, 0xF, 0xF, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr8, 0xF, 0xF, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast15, 0xA, 0xF, false);
  x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast31, 0xC, 0xF, false);
  return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// Block-wide reductions through a small LDS scratch (kStreamWaves slots).  Every
// thread of the block must call them; all threads receive the result.
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t *scratch) {
  v = wave_sum_u64(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[wave] = v;
  lds_barrier();
  uint64_t t = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += scratch[w];
  lds_barrier();
  return t;
}

__device__ __forceinline__ void block_and_or(uint32_t &a, uint32_t &o, uint32_t *scratch) {
  a = wave_and(a);
  o = wave_or(o);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { scratch[2 * wave] = a; scratch[2 * wave + 1] = o; }
  lds_barrier();
  uint32_t ra = ~0u, ro = 0u;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) { ra &= scratch[2 * w]; ro |= scratch[2 * w + 1]; }
  lds_barrier();
  a = ra;
  o = ro;
}

// Block-wide maximum of a u32.  scratch: kStreamWaves u32.  Every thread must call it.
__device__ __forceinline__ uint32_t block_max_u32(uint32_t x, uint32_t *scratch) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr1, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr2, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr4, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowShr8, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast15, 0xA, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kRowBcast31, 0xC, 0xF, false));
  x = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[wave] = x;
  lds_barrier();
  uint32_t r = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) r = max(r, scratch[w]);
  lds_barrier();
  return r;
}

// Exclusive block-wide prefix sum of one u32 per thread (thread order), plus the
// total.  scratch: kStreamWaves u32.  One barrier pair.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t x, uint32_t &total, uint32_t *scratch) {
  const uint32_t incl = wave_scan_u32(x);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) scratch[wave] = incl;
  lds_barrier();
  uint32_t before = 0, tot = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    const uint32_t c = scratch[w];
    before += (w < wave) ? c : 0u;
    tot += c;
  }
  lds_barrier();
  total = tot;
  return before + incl - x;
}

// The slot plan of one stream from its keep bytes kp[0..n) with K kept (ActKV
// Dissected, Component 3: survivors skew toward the tail, so the tail is the target
// region).  With D = n - K the sources are the kept slots below D and the destinations
// the evicted slots from D on, both ascending; pair t = (source t, destination t) goes
// to pp[2t], pp[2t + 1] for t < min(D, K), so a keep mask with the wrong count cannot
// overrun.  Returns the pair count, min(#sources, #destinations, D, K), in every
// thread.  Slots go in rounds of blockDim x 32: thread t owns 32 consecutive slots of a
// round, read as two 16-byte loads when aligned, and one block scan per list and round
// gives its starting ranks.  sc1, sc2: kStreamWaves words of LDS each.  Every thread of
// the block must call it.
__device__ __forceinline__ uint32_t plan_slots(const uint8_t *kp, int32_t n, int32_t K, int32_t *pp, uint32_t *sc1,
                                               uint32_t *sc2) {
  const int32_t D = n - K;
  const int32_t cap = D < K ? D : K;
  if (cap <= 0) return 0u;
  constexpr int U = 32;
  uint32_t base_s = 0, base_d = 0;
  for (int32_t r0 = 0; r0 < n; r0 += U * (int32_t)blockDim.x) {
    const int32_t j0 = r0 + (int32_t)threadIdx.x * U;
    uint8_t kv[U];
    const uint8_t *kpj = kp + j0;
    if (j0 + U <= n && ((uintptr_t)kpj & 15u) == 0) {
      const uint4 w0 = *(const uint4 *)kpj, w1 = *(const uint4 *)(kpj + 16);
      const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int u = 0; u < U; ++u) kv[u] = (uint8_t)(w[u >> 2] >> ((u & 3) * 8));
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) kv[u] = (j0 + u < n) ? kpj[u] : (uint8_t)0;
    }
    uint32_t cs = 0, cd = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t j = j0 + u;
      cs += (j < n && j < D && kv[u]) ? 1u : 0u;
      cd += (j < n && j >= D && !kv[u]) ? 1u : 0u;
    }
    uint32_t rts, rtd;
    uint32_t rs = base_s + block_exclusive_scan(cs, rts, sc1);
    uint32_t rd = base_d + block_exclusive_scan(cd, rtd, sc2);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int32_t j = j0 + u;
      if (j >= n) continue;
      if (j < D && kv[u]) {
        if (rs < (uint32_t)cap) pp[(int64_t)rs * 2] = j;
        ++rs;
      } else if (j >= D && !kv[u]) {
        if (rd < (uint32_t)cap) pp[(int64_t)rd * 2 + 1] = j;
        ++rd;
      }
    }
    base_s += rts;
    base_d += rtd;
  }
  uint32_t c = base_s < base_d ? base_s : base_d;
  return c < (uint32_t)cap ? c : (uint32_t)cap;
}

// Exclusive rank of this thread's flag among all flags of the block in thread order,
// plus the block total.  One barrier pair.
__device__ __forceinline__ uint32_t block_flag_rank(bool flag, uint32_t &total, uint32_t *scratch) {
  const uint64_t m = __ballot(flag);
  const int wave = threadIdx.x >> 6;
  const uint32_t in_wave = __popcll(m & lanemask_lt());
  if ((threadIdx.x & 63) == 0) scratch[wave] = __popcll(m);
  lds_barrier();
  uint32_t before = 0, tot = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    const uint32_t c = scratch[w];
    before += (w < wave) ? c : 0u;
    tot += c;
  }
  lds_barrier();
  total = tot;
  return before + in_wave;
}

// floor(s * 2^32) for a finite fp32 s >= 0, from its bit pattern, without branches:
// the integer part of s and the fraction times 2^32, each by a truncating conversion.
// Both steps are exact (the fraction of an fp32 value and its product with a power of
// two are representable, and truncation is floor for s >= 0).  Negative values,
// infinities and NaNs (outside the kernel contract) count as zero mass; values of 2^32
// and more (also outside it) saturate.
__device__ __forceinline__ uint64_t fixed_mass(uint32_t bits) {
  const float s = __uint_as_float(bits);
  const uint32_t hi = __float2uint_rz(s);
  const uint32_t lo = __float2uint_rz((s - (float)hi) * 4294967296.0f);
  const uint64_t m = ((uint64_t)hi << 32) | lo;
  return bits < 0x7F800000u ? m : 0ull;
}

// Nearest fp32 (ties to even) to an unsigned 64-bit integer, by integer steps.
__device__ __forceinline__ float u64_to_f32_rn(uint64_t x) {
  if (x < (1ull << 24)) return (float)(uint32_t)x;             // exact
  const int e = 63 - __clzll((long long)x);                     // 2^e <= x < 2^(e+1), e >= 24
  const int sh = e - 23;
  uint64_t m = x >> sh;                                         // the 24 leading bits
  const uint64_t rem = x & ((1ull << sh) - 1ull);
  const uint64_t half = 1ull << (sh - 1);
  m += (rem > half || (rem == half && (m & 1ull))) ? 1ull : 0ull;   // 2^24 at most: exact below
  return __builtin_ldexpf((float)(uint32_t)m, sh);
}

// Address of the CRF of live slot j of a stream.
__device__ __forceinline__ float *crf_slot(float *crf, const int32_t *bt_row, int32_t start, int32_t j,
                                           int32_t l, int32_t g, int64_t num_pages, int32_t Hkv) {
  const int32_t pos = start + j;
  const int64_t phys = bt_row[pos >> 4];
  return crf + (((int64_t)l * num_pages + phys) * Hkv + g) * kPage + (pos & 15);
}

// Add v into an LDS histogram bin.  When many lanes of the wave share the first
// valid lane's bin (value distributions concentrated in one bin), those lanes are
// summed in registers first and added with one atomic; every other lane adds
// directly.  Must be called by all lanes of the wave.
__device__ __forceinline__ void hist_add_u64(uint64_t *hist, bool valid, uint32_t bin, uint64_t v) {
  const uint64_t mask = ballot(valid);
  if (mask == 0) return;
  const int leader = __ffsll((long long)mask) - 1;
  const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
  const bool same = valid && bin == lb;
  const uint64_t smask = ballot(same);
  if (__popcll(smask) >= 8) {
    const uint64_t agg = wave_sum_u64(same ? v : 0ull);
    // (the leader's own bin, lb: an address the compiler takes as per-lane, so it adds
    // no wave-reduction code of its own around this single-lane atomic)
    if ((int)(threadIdx.x & 63) == leader) atomicAdd((unsigned long long *)&hist[bin], (unsigned long long)agg);
    if (valid && !same) atomicAdd((unsigned long long *)&hist[bin], (unsigned long long)v);
  } else if (valid) {
    atomicAdd((unsigned long long *)&hist[bin], (unsigned long long)v);
  }
}

// Count version: add 1 per valid lane; the lanes sharing the first valid lane's bin
// are counted with a popcount and added once.
__device__ __forceinline__ void hist_add_count(uint64_t *hist, bool valid, uint32_t bin) {
  const uint64_t mask = ballot(valid);
  if (mask == 0) return;
  const int leader = __ffsll((long long)mask) - 1;
  const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
  const bool same = valid && bin == lb;
  const uint64_t smask = ballot(same);
  if ((int)(threadIdx.x & 63) == leader) atomicAdd((unsigned long long *)&hist[bin], (unsigned long long)__popcll(smask));
  if (valid && !same) atomicAdd((unsigned long long *)&hist[bin], 1ull);
}

}  // namespace kvs
