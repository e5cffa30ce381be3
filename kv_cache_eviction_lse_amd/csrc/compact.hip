// kvs_compact: the in-place mover.
//
// ActKV Dissected, Component 3: all planned pairs are copied in one parallel pass,
// with no extra KV buffer.  Sources and destinations are disjoint, so there is no
// ordering between pairs.  A workgroup moves 64 pairs of one stream: 64 pairs x
// (K row + V row) = 2048 chunks of 16 bytes, 8 per thread, all loads issued before
// the stores; the first 64 threads also move the pairs' CRF values.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kPairsPerBlock = 64;
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
  const int32_t i = blockIdx.z;
  const int32_t lg = blockIdx.y;
  const int32_t cnt = a.pair_count[(int64_t)lg * a.b.S + i];
  const int32_t p0 = blockIdx.x * kPairsPerBlock;
  if (p0 >= cnt || cnt > a.P) return;
  const int32_t l = lg / a.b.Hkv;
  const int32_t g = lg - l * a.b.Hkv;
  const int32_t start = a.b.start[i];
  const int32_t n = a.b.len[i];
  const int32_t *bt_row = a.b.bt + (int64_t)i * a.b.max_pages;
  const int32_t *pp = a.pairs + (((int64_t)lg * a.b.S + i) * a.P) * 2;

  // chunk c = threadIdx.x + 256u: pair c / 32, row half (K or V) (c / 16) % 2, 16-byte
  // piece c % 16; the K/V choice is the same for every u of a thread
  const int kv = (threadIdx.x >> 4) & 1;
  uint16_t *pool = kv ? a.v : a.k;
  const int ch = threadIdx.x & 15;
  uint4 buf[8];
  int64_t dst_off[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int32_t t = p0 + ((threadIdx.x + u * kMoveThreads) >> 5);
    dst_off[u] = -1;
    if (t < cnt) {
      const int32_t src = pp[2 * t];
      const int32_t dst = pp[2 * t + 1];
      if (src < 0 || src >= n || dst < 0 || dst >= n) continue;
      buf[u] = *(const uint4 *)(pool + row_elem(a, bt_row, start, src, l, g) * kHeadDim + ch * 8);
      dst_off[u] = row_elem(a, bt_row, start, dst, l, g) * kHeadDim + ch * 8;
    }
  }
  float cval = 0.f;
  int64_t cdst = -1;
  if (threadIdx.x < kPairsPerBlock) {
    const int32_t t = p0 + threadIdx.x;
    if (t < cnt) {
      const int32_t src = pp[2 * t];
      const int32_t dst = pp[2 * t + 1];
      if (src >= 0 && src < n && dst >= 0 && dst < n) {
        cval = a.crf[row_elem(a, bt_row, start, src, l, g)];
        cdst = row_elem(a, bt_row, start, dst, l, g);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < 8; ++u)
    if (dst_off[u] >= 0) *(uint4 *)(pool + dst_off[u]) = buf[u];
  if (cdst >= 0) a.crf[cdst] = cval;
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
