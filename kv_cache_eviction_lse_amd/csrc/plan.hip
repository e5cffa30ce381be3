// kvs_plan (device part): conflict-free slot plan, one workgroup per stream.
//
// ActKV Dissected, Component 3: survivors skew toward the tail, so the tail is the
// target region; survivors outside it are paired one-to-one with holes inside it.
// With K kept and D = n - K, sources are the kept slots below D and destinations
// the evicted slots at or above D, both ascending; pair t = (source t, dest t).
// Slots are processed in rounds in which each thread takes 16 consecutive slots; one
// block-wide scan per list and round gives every thread its starting ranks.  Writes
// are bounded by the stream's capacity min(D, K), so a keep mask with the wrong count
// cannot overrun.  kvs_plan_compact runs the same plan and then moves the pairs from
// the same workgroup (the pairs are disjoint: sources below D, destinations at or
// above it).
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

constexpr int kFusedPairs = 8192;   // pairs per stream the fused mover keeps in LDS
constexpr int kFusedPages = 8192;   // block-table entries per stream it keeps in LDS

struct MoveArgs {
  uint16_t *k;
  uint16_t *v;
  float *crf;
};

// MOVE = false: the plan only.  MOVE = true: the plan, then the same workgroup moves
// its stream's pairs (K row, V row, CRF) from the pair lists and block-table row it
// holds in LDS, so the move does not wait on reloading them.
template <bool MOVE>
__global__ __launch_bounds__(kStreamThreads) void plan_kernel(PlanArgs a, MoveArgs m) {
  __shared__ uint32_t sc1[kStreamWaves], sc2[kStreamWaves];
  extern __shared__ int32_t mv[];    // MOVE: src[kFusedPairs], dst[kFusedPairs], bt[npages]

  const int32_t i = blockIdx.y;
  const int32_t lg = blockIdx.x;
  const int32_t n = a.b.len[i];
  const int32_t K = kept_of(n, a.budget[i]);
  const int32_t D = n - K;
  const int32_t cap = min(D, K);
  const int32_t start = a.b.start[i];
  int32_t *pp = a.pairs + (((int64_t)lg * a.b.S + i) * a.P) * 2;
  const uint8_t *kp = a.keep + (int64_t)lg * a.b.E + a.b.entry_off[i];
  int32_t *ls_src = mv;
  int32_t *ls_dst = mv + kFusedPairs;
  int32_t *ls_bt = mv + 2 * kFusedPairs;
  const int32_t npages = (start + n + kPage - 1) / kPage;
  if (MOVE && cap > 0) {
    const int32_t *bt_row = a.b.bt + (int64_t)i * a.b.max_pages;
    for (int32_t p = threadIdx.x; p < npages; p += kStreamThreads) ls_bt[p] = bt_row[p];
  }
  uint32_t ts = 0, td = 0;
  if (cap > 0 && cap <= a.P) {
    // rounds of 1024 x 32 slots (one round up to 32 768 entries): thread t owns 32
    // consecutive slots of the round, read as two 16-byte loads when they are aligned;
    // one block scan per list and round gives every thread its starting ranks
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
          if (rs < (uint32_t)cap) {
            pp[(int64_t)rs * 2] = j;
            if (MOVE) ls_src[rs] = j;
          }
          ++rs;
        } else if (j >= D && !kv[u]) {
          if (rd < (uint32_t)cap) {
            pp[(int64_t)rd * 2 + 1] = j;
            if (MOVE) ls_dst[rd] = j;
          }
          ++rd;
        }
      }
      base_s += rts;
      base_d += rtd;
    }
    ts = base_s;
    td = base_d;
  }
  uint32_t c = ts < td ? ts : td;
  if (c > (uint32_t)(cap > 0 ? cap : 0)) c = (uint32_t)(cap > 0 ? cap : 0);
  if (threadIdx.x == 0) a.pair_count[(int64_t)lg * a.b.S + i] = (int32_t)c;
  if (!MOVE || c == 0) return;
  lds_barrier();   // pair lists and block-table row complete (in LDS)

  const int32_t l = lg / a.b.Hkv;
  const int32_t g = lg - l * a.b.Hkv;
  const int64_t head_base = ((int64_t)l * a.b.num_pages) * a.b.Hkv + g;   // in 16-slot blocks
  auto slot_elem = [&](int32_t j) -> int64_t {
    const int32_t pos = start + j;
    return (head_base + (int64_t)ls_bt[pos >> 4] * a.b.Hkv) * kPage + (pos & 15);
  };
  // 16-byte chunks: chunk x = pair x / 32, K or V row (x / 16) % 2, piece x % 16; a
  // thread keeps the same row half for every x it takes
  const int kvsel = (threadIdx.x >> 4) & 1;
  uint16_t *pool = kvsel ? m.v : m.k;
  const int ch = threadIdx.x & 15;
  const int32_t chunks = (int32_t)c * 32;
  // 16 chunks per thread in flight (every chunk of up to 512 pairs in one round trip);
  // destinations are recomputed from the LDS lists at the stores, so only the data is
  // held in registers meanwhile
  constexpr int kInFlight = 16;
  for (int32_t x0 = 0; x0 < chunks; x0 += kInFlight * kStreamThreads) {
    uint4 buf[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int32_t x = x0 + u * kStreamThreads + (int32_t)threadIdx.x;
      if (x < chunks) buf[u] = *(const uint4 *)(pool + slot_elem(ls_src[x >> 5]) * kHeadDim + ch * 8);
    }
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) {
      const int32_t x = x0 + u * kStreamThreads + (int32_t)threadIdx.x;
      if (x < chunks) *(uint4 *)(pool + slot_elem(ls_dst[x >> 5]) * kHeadDim + ch * 8) = buf[u];
    }
  }
  for (int32_t t = threadIdx.x; t < (int32_t)c; t += kStreamThreads)
    m.crf[slot_elem(ls_dst[t])] = m.crf[slot_elem(ls_src[t])];
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
  plan_kernel<false><<<grid, kStreamThreads, 0, st>>>(a, MoveArgs{});
  return hipGetLastError();
}

bool plan_move_fits(int64_t pair_cap, int32_t max_npages) {
  return pair_cap <= kFusedPairs && max_npages <= kFusedPages;
}

hipError_t launch_plan_move(const kvs_cache &c, const Batch &b, const uint8_t *keep, const int32_t *budget,
                            int32_t *pairs, int32_t *pair_count, int64_t pair_cap, int32_t max_npages,
                            hipStream_t st) {
  static bool attr_set = false;
  const size_t dyn = (2 * (size_t)kFusedPairs + (size_t)max_npages) * sizeof(int32_t);
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void *)plan_kernel<true>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)((2 * kFusedPairs + kFusedPages) * sizeof(int32_t)));
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  PlanArgs a{};
  a.keep = keep;
  a.budget = budget;
  a.pairs = pairs;
  a.pair_count = pair_count;
  a.b = b;
  a.P = pair_cap;
  MoveArgs m{(uint16_t *)c.k, (uint16_t *)c.v, c.crf};
  dim3 grid((unsigned)(b.L * b.Hkv), (unsigned)b.S);
  plan_kernel<true><<<grid, kStreamThreads, dyn, st>>>(a, m);
  return hipGetLastError();
}

}  // namespace kvs
