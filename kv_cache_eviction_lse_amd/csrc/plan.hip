// kvs_plan (device part): conflict-free slot plan, one workgroup per stream.
//
// ActKV Dissected, Component 3: survivors skew toward the tail, so the tail is the
// target region; survivors outside it are paired one-to-one with holes inside it.
// With K kept and D = n - K, sources are the kept slots below D and destinations
// the evicted slots at or above D, both ascending; pair t = (source t, dest t).
// Slots are processed in rounds in which each thread takes 16 consecutive slots;
// one block-wide scan per list and round gives every thread its starting ranks.  Writes are bounded by the stream's
// capacity min(D, K) so that a keep mask with the wrong count cannot overrun.
#include "kvs_device.h"

namespace kvs {
namespace {

struct PlanArgs {
  const uint8_t *keep;
  const int32_t *budget;
  int32_t *pairs;
  int32_t *pair_count;
  Batch b;
  int64_t P;   // pair capacity per stream
};

__device__ __forceinline__ int32_t kept_of(int32_t len, int32_t bud) {
  return bud < len ? (bud > 0 ? bud : 0) : len;
}

__global__ __launch_bounds__(kStreamThreads) void plan_kernel(PlanArgs a) {
  __shared__ uint32_t sc1[kStreamWaves], sc2[kStreamWaves];

  const int32_t i = blockIdx.y;
  const int32_t lg = blockIdx.x;
  const int32_t n = a.b.len[i];
  const int32_t K = kept_of(n, a.budget[i]);
  const int32_t D = n - K;
  const int32_t cap = min(D, K);
  int32_t *pp = a.pairs + (((int64_t)lg * a.b.S + i) * a.P) * 2;
  const uint8_t *kp = a.keep + (int64_t)lg * a.b.E + a.b.entry_off[i];
  uint32_t ts = 0, td = 0;
  if (cap > 0 && cap <= a.P) {
    // rounds of 1024 x 16 slots: thread t owns 16 consecutive slots of the round; one
    // block scan per list and round gives every thread its starting ranks
    constexpr int U = 16;
    uint32_t base_s = 0, base_d = 0;
    for (int32_t r0 = 0; r0 < n; r0 += U * (int32_t)blockDim.x) {
      const int32_t j0 = r0 + (int32_t)threadIdx.x * U;
      uint8_t kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) kv[u] = (j0 + u < n) ? kp[j0 + u] : (uint8_t)0;
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
    ts = base_s;
    td = base_d;
  }
  if (threadIdx.x == 0) {
    uint32_t c = ts < td ? ts : td;
    if (c > (uint32_t)(cap > 0 ? cap : 0)) c = (uint32_t)(cap > 0 ? cap : 0);
    a.pair_count[(int64_t)lg * a.b.S + i] = (int32_t)c;
  }
}

}  // namespace

hipError_t launch_plan(const Batch &b, const uint8_t *keep, const int32_t *budget, int32_t *pairs,
                       int32_t *pair_count, int64_t pair_cap, hipStream_t st) {
  PlanArgs a{};
  a.keep = keep;
  a.budget = budget;
  a.pairs = pairs;
  a.pair_count = pair_count;
  a.b = b;
  a.P = pair_cap;
  dim3 grid((unsigned)(b.L * b.Hkv), (unsigned)b.S);
  plan_kernel<<<grid, kStreamThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
