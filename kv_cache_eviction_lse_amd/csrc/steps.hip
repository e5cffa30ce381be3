// kvs_step_select: step-aware ranking keys.
//
// StepKV: Step-Aware KV Cache Compression for LLM Agents, Abstract: every cache entry
// belongs to the reasoning step that generated it; a step's utility, estimated from
// the trajectory, is combined with token-level saliency, and the combined scores rank
// the prunable entries globally under a budget.  Here a step is a contiguous run of a
// sequence's live slots, its utility U is the mean attention score of its entries on
// the mass cut's fixed-point grid (a_j = floor(s_j 2^32), an exact integer sum, the
// mean floored and rounded once to fp32), and an entry's key is
//     c_j = fma(beta, U, fp32((1 - beta) s_j)).
// The keep set is the top-B of (c desc, s desc, slot asc), chosen by the kvs_select
// kernels with these keys in the CRF's place.
//
// One wave per (step, layer x KV head): it sums the step's masses, forms U, then writes
// the keys of the step's entries (their scores are re-read from cache).  No atomics,
// nothing to clear, no entry-to-step table.
#include "kvs_device.h"

namespace kvs {
namespace {

struct StepArgs {
  const float *scores;        // [L*Hkv][E]
  const int64_t *step_off;    // [S+1]: steps of sequence i are step_off[i] .. step_off[i+1]-1
  const int32_t *first;       // [M]: first live slot of each step
  float *keys;                // [L*Hkv][E]
  float *utility;             // [L*Hkv][M] or null
  Batch b;
  int64_t M;
  float beta;
  float w;                    // fp32(1 - beta)
};

constexpr int kStepWaves = 4;

__global__ __launch_bounds__(64 * kStepWaves) void step_key_kernel(StepArgs a) {
  // the wave index is uniform within the wave: saying so makes every per-step value
  // below scalar (scalar loads through the constant cache, not vector loads)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t gk = (int64_t)blockIdx.x * kStepWaves + wave;
  if (gk >= a.M) return;
  const int32_t lg = blockIdx.y;
  // the sequence holding step gk: step_off[i] <= gk < step_off[i + 1] (empty sequences
  // share their offset with the next one and are skipped by taking the largest such i)
  int32_t lo = 0, hi = a.b.S;
  while (hi - lo > 1) {
    const int32_t mid = (lo + hi) >> 1;
    if (a.step_off[mid] <= gk) lo = mid;
    else hi = mid;
  }
  const int32_t i = lo;
  const int32_t n = a.b.len[i];
  const int32_t first = a.first[gk];
  const int32_t next_first = a.first[gk + 1 < a.M ? gk + 1 : gk];           // read with the others
  const int32_t last = gk + 1 < a.step_off[i + 1] ? next_first : n;          // one past the step
  const int64_t e0 = a.b.entry_off[i];
  const uint32_t *sp = (const uint32_t *)(a.scores + (int64_t)lg * a.b.E + e0);
  // four loads in flight per lane, then the tail
  uint64_t sum = 0;
  int32_t j = first + lane;
  for (; j + 192 < last; j += 256) {
    const uint32_t x0 = sp[j], x1 = sp[j + 64], x2 = sp[j + 128], x3 = sp[j + 192];
    sum += (fixed_mass(x0) + fixed_mass(x1)) + (fixed_mass(x2) + fixed_mass(x3));
  }
  for (; j < last; j += 64) sum += fixed_mass(sp[j]);
  sum = wave_sum_u64(sum);
  const int32_t len = last - first;
  const float U = len > 0 ? u64_to_f32_rn(sum / (uint64_t)len) * 0x1p-32f : 0.f;   // scaling is exact
  if (a.utility && lane == 0) a.utility[(int64_t)lg * a.M + gk] = U;
  float *kp = a.keys + (int64_t)lg * a.b.E + e0;
  auto key = [&](uint32_t x) { return __builtin_fmaf(a.beta, U, a.w * __uint_as_float(x)); };
  j = first + lane;
  for (; j + 192 < last; j += 256) {
    const uint32_t x0 = sp[j], x1 = sp[j + 64], x2 = sp[j + 128], x3 = sp[j + 192];
    kp[j] = key(x0);
    kp[j + 64] = key(x1);
    kp[j + 128] = key(x2);
    kp[j + 192] = key(x3);
  }
  for (; j < last; j += 64) kp[j] = key(sp[j]);
}

}  // namespace

hipError_t launch_step_keys(const Batch &b, const float *scores, const int64_t *step_off, const int32_t *first,
                            int64_t num_steps, float beta, float *keys, float *utility, hipStream_t st) {
  if (num_steps == 0) return hipSuccess;
  StepArgs a{};
  a.scores = scores;
  a.step_off = step_off;
  a.first = first;
  a.keys = keys;
  a.utility = utility;
  a.b = b;
  a.M = num_steps;
  a.beta = beta;
  a.w = 1.0f - beta;
  const dim3 grid((unsigned)((num_steps + kStepWaves - 1) / kStepWaves), (unsigned)(b.L * b.Hkv));
  step_key_kernel<<<grid, 64 * kStepWaves, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
