// kvs_plan (device part): conflict-free slot plan, one workgroup per stream.
//
// ActKV Dissected, Component 3: survivors skew toward the tail, so the tail is the
// target region; survivors outside it are paired one-to-one with holes inside it.
// With K kept and D = n - K, sources are the kept slots below D and destinations
// the evicted slots at or above D, both ascending; pair t = (source t, dest t).
// The plan itself is plan_slots (shared with the fused selection kernel).
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
  const uint32_t c = cap > 0 && cap <= a.P ? plan_slots(kp, n, K, pp, sc1, sc2) : 0u;
  if (threadIdx.x == 0) a.pair_count[(int64_t)lg * a.b.S + i] = (int32_t)c;
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
