// kvs_compact: the in-place mover.
//
// ActKV Dissected, Component 3: all planned pairs are copied in one parallel pass,
// with no extra KV buffer.  Sources and destinations are disjoint, so there is no
// ordering between pairs.  A workgroup moves 8 pairs of one stream: 8 pairs x (K row +
// V row) = 256 chunks of 16 bytes, one per thread; the thread at the start of each
// pair's 32 also moves the pair's CRF value.  One chunk per thread over many small
// workgroups keeps reads and writes interleaved across the chip: the same rows moved
// with 8 or 16 chunks per thread (all loads before the stores) take 1.4-1.6x longer.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kPairsPerBlock = 8;
constexpr int kMoveThreads = 256;

struct CompactArgs {
  uint16_t *k;
  uint16_t *v;
  float *crf;
  const int32_t *pairs;
  const int32_t *pair_count;
  Batch b;
  int64_t P;
};

__device__ __forceinline__ int64_t row_elem(const CompactArgs &a, const int32_t *bt_row, int32_t start,
                                            int32_t j, int32_t l, int32_t g) {
  const int32_t pos = start + j;
  const int64_t phys = bt_row[pos >> 4];
  return ((((int64_t)l * a.b.num_pages + phys) * a.b.Hkv + g) * kPage + (pos & 15));
}

__global__ __launch_bounds__(kMoveThreads) void compact_kernel(CompactArgs a) {
  static_assert(kPairsPerBlock * 32 == kMoveThreads, "one 16-byte chunk per thread");
  const int32_t i = blockIdx.z;
  const int32_t lg = blockIdx.y;
  const int32_t t = (int32_t)blockIdx.x * kPairsPerBlock + (int32_t)(threadIdx.x >> 5);
  if (t >= a.P) return;   // (the grid rounds P up to whole workgroups)
  const int64_t pc = (int64_t)lg * a.b.S + i;
  // the pair is read together with the count (slot t < P is in the buffer whatever the
  // count), so the row addresses wait on one round trip instead of two
  const int2 pr = *(const int2 *)(a.pairs + (pc * a.P + t) * 2);
  const int32_t cnt = a.pair_count[pc];
  if (t >= cnt || cnt > a.P) return;
  const int32_t l = lg / a.b.Hkv;
  const int32_t g = lg - l * a.b.Hkv;
  const int32_t start = a.b.start[i];
  const int32_t n = a.b.len[i];
  const int32_t *bt_row = a.b.bt + (int64_t)i * a.b.max_pages;
  const int32_t src = pr.x;
  const int32_t dst = pr.y;
  if (src < 0 || src >= n || dst < 0 || dst >= n) return;
  const int64_t se = row_elem(a, bt_row, start, src, l, g);
  const int64_t de = row_elem(a, bt_row, start, dst, l, g);
  // chunk = pair (threadIdx / 32), row half (K or V) (threadIdx / 16) % 2, 16-byte piece
  // threadIdx % 16
  uint16_t *pool = ((threadIdx.x >> 4) & 1) ? a.v : a.k;
  const int ch = threadIdx.x & 15;
  const uint4 x = *(const uint4 *)(pool + se * kHeadDim + ch * 8);
  const bool lead = (threadIdx.x & 31) == 0;
  float cval = 0.f;
  if (lead) cval = a.crf[se];
  *(uint4 *)(pool + de * kHeadDim + ch * 8) = x;
  if (lead) a.crf[de] = cval;
}

}  // namespace

hipError_t launch_compact(const kvs_cache &c, const Batch &b, const int32_t *pairs,
                          const int32_t *pair_count, int64_t pair_cap, hipStream_t st) {
  if (pair_cap <= 0 || b.S == 0 || b.L == 0 || b.Hkv == 0) return hipSuccess;
  CompactArgs a{};
  a.k = (uint16_t *)c.k;
  a.v = (uint16_t *)c.v;
  a.crf = c.crf;
  a.pairs = pairs;
  a.pair_count = pair_count;
  a.b = b;
  a.P = pair_cap;
  dim3 grid((unsigned)((pair_cap + kPairsPerBlock - 1) / kPairsPerBlock), (unsigned)(b.L * b.Hkv),
            (unsigned)b.S);
  compact_kernel<<<grid, kMoveThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
