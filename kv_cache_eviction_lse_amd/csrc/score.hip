// kvs_score kernels: attention recovered from the log-sum-exp, summed per cached entry.
//
// ActKV Dissected, Component 3: the LSE of each query row is a byproduct of paged
// attention, so the probability a row puts on an entry is exp(logit - LSE): no
// softmax pass, no attention matrix.  Component 1: the signal of an entry is the
// attention it receives from all observer (action) tokens, here also summed over
// the query heads of the entry's GQA group.
//
// Two kernels share one work decomposition (a work item is a chunk of consecutive
// 8-page steps of one stream and one group of up to 256 observer rows):
//   score_mfma_kernel : observers >= 16.  QK^T on v_mfma_f32_32x32x16_bf16 with the
//       observer rows on M and the keys on N, so each lane ends up holding one key
//       and 16 rows: the exp and the row sum stay in-lane.  K pages stream from HBM
//       straight into LDS (global_load_lds_dwordx4, 1 KiB per instruction, XOR-
//       swizzled 16-byte chunks), double-buffered, shared by the 4 waves.
//   score_valu_kernel : observers < 16.  One key per lane, 64 keys per wave; the
//       key row is pulled from LDS into registers and every observer row (uniform
//       across the wave, so it lives in SGPRs) is dotted with v_dot2c_f32_bf16.
// Both evaluate p = exp2(fma(dot, scale*log2 e, -LSE*log2 e)) and accumulate in fp32.
#include "kvs_internal.h"

namespace kvs {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStepPages = 8;                       // one pipeline step: 8 pages, 128 keys
constexpr int kStepKeys = kStepPages * kPage;
constexpr int kStepBytes = kStepPages * kPageElems * 2;   // 32 KiB
constexpr int kTileKeys = 32;                       // one MFMA N tile (2 pages)
constexpr int kStepTiles = kStepKeys / kTileKeys;   // 4
constexpr int kRowsPerWave = 64;                    // 2 MFMA M tiles
constexpr int kRowsPerGroup = kRowsPerWave * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

struct ScoreArgs {
  const uint16_t *k;          // bf16 K pool
  const uint16_t *q;          // bf16 observers
  const float *lse;
  const int64_t *obs_off;
  const int32_t *item_off;    // [S+1] work items per (layer, head) of this path
  float *out;                 // scores, or per-row-group partials
  Batch b;
  int64_t obs_total;
  int64_t total_items;        // items_per_lg * L * Hkv
  int64_t padded_items;       // total rounded up to a multiple of 8
  int32_t items_per_lg;
  int32_t Hq;
  int32_t G;
  int32_t chunk_steps;
  int32_t partials;           // 1: write [rg][L][Hkv][E] partial sums
  float alpha;                // scale * log2(e)
};

struct Item {
  int32_t i, l, g, rg, chunk;
  int32_t start, n, O, npages, nsteps;
  int64_t e0, o0;
};

// Work item for this workgroup, or false if it has none.  Consecutive hardware
// workgroup ids go round-robin over the 8 XCDs; item = (id % 8) * (padded / 8) + id / 8
// gives each XCD a contiguous run of items, i.e. consecutive chunks of the same
// stream, which share the stream's observer rows in that XCD's L2.
__device__ __forceinline__ bool decode_item(const ScoreArgs &a, Item &it) {
  const int64_t per_xcd = a.padded_items >> 3;
  const int64_t id = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (id >= a.total_items) return false;
  const int32_t lg = (int32_t)(id / a.items_per_lg);
  const int32_t rem = (int32_t)(id - (int64_t)lg * a.items_per_lg);
  int lo = 0, hi = a.b.S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.item_off[mid] <= rem) lo = mid; else hi = mid;
  }
  it.i = lo;
  it.l = lg / a.b.Hkv;
  it.g = lg - it.l * a.b.Hkv;
  it.start = a.b.start[lo];
  it.n = a.b.len[lo];
  it.e0 = a.b.entry_off[lo];
  it.o0 = a.obs_off[lo];
  it.O = (int32_t)(a.obs_off[lo + 1] - it.o0);
  it.npages = (it.start + it.n + kPage - 1) / kPage;
  it.nsteps = (it.npages + kStepPages - 1) / kStepPages;
  const int32_t nchunks = (it.nsteps + a.chunk_steps - 1) / a.chunk_steps;
  const int32_t local = rem - a.item_off[lo];
  it.rg = local / nchunks;
  it.chunk = local - it.rg * nchunks;
  // host and device item counts agree by construction; refuse anything else
  const int32_t nrg = (it.O * a.G + kRowsPerGroup - 1) / kRowsPerGroup;
  if (it.n <= 0 || it.O <= 0 || it.rg >= nrg) return false;
  return true;
}

// Issue this wave's share (pages p0, p0+1) of one 8-page step into an LDS buffer.
// Lane t of instruction r fills LDS chunk t%16 of page row 4r + t/16 with global
// chunk (t%16) ^ row, so that a later read of chunk c of row n lands on c ^ (n%16).
__device__ __forceinline__ void issue_step(const ScoreArgs &a, const Item &it, int step, uint8_t *buf,
                                           int wave, int lane) {
  const int32_t *bt = a.b.bt + (int64_t)it.i * a.b.max_pages;
  const int row_in_instr = lane >> 4;
  const int chunk = lane & 15;
#pragma unroll
  for (int pp = 0; pp < 2; ++pp) {
    const int page_in_step = wave * 2 + pp;
    const int lp = step * kStepPages + page_in_step;
    if (lp < it.npages) {
      const int64_t phys = bt[lp];
      const uint16_t *page = a.k + (((int64_t)it.l * a.b.num_pages + phys) * a.b.Hkv + it.g) * kPageElems;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * r + row_in_instr;
        const uint16_t *src = page + row * kHeadDim + ((chunk ^ row) << 3);
        uint8_t *dst = buf + page_in_step * (kPageElems * 2) + r * 1024;
        __builtin_amdgcn_global_load_lds((const void *)src, (lds_void *)dst, 16, 0, 0);
      }
    }
  }
}

__device__ __forceinline__ void store_key(const ScoreArgs &a, const Item &it, int tile, int n,
                                          float v) {
  const int32_t pos = tile * kTileKeys + n;
  const int32_t j = pos - it.start;
  if (j >= 0 && j < it.n) {
    int64_t row = (int64_t)it.l * a.b.Hkv + it.g;
    if (a.partials) row += (int64_t)it.rg * a.b.L * a.b.Hkv;
    a.out[row * a.b.E + it.e0 + j] = v;
  }
}

__global__ __launch_bounds__(kThreads, 2) void score_mfma_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][kStepBytes];
  __shared__ float part[2][kStepTiles][kWaves][kTileKeys];

  Item it;
  if (!decode_item(a, it)) return;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int col = lane & 31;

  const int32_t R = it.O * a.G;
  const int32_t r0 = it.rg * kRowsPerGroup;
  const int32_t rows_here = min(kRowsPerGroup, R - r0);
  const int wpr = (rows_here + kRowsPerWave - 1) / kRowsPerWave;        // waves per row set
  const int nph = wpr == 1 ? 4 : (wpr == 2 ? 2 : 1);                    // tile phases
  const int phase = wave / wpr;
  const int wrow = wave - phase * wpr;
  const bool active = phase < nph;
  const int32_t wr0 = r0 + wrow * kRowsPerWave;
  const bool mt_on0 = active && wr0 < R;
  const bool mt_on1 = active && wr0 + 32 < R;

  // Observer rows of this wave as MFMA A operands: lane (m, h) holds row m,
  // dims 16s + 8h .. +8 for k-step s.  LSE (times log2 e) in the accumulator
  // layout: register k of M tile t holds row 32t + 8(k/4) + 4h + k%4.
  bf16x8 qa[2][8];
  float nl[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int32_t r = wr0 + 32 * t + col;
    const bool ok = active && r < R;
    const uint16_t *qp = a.q;
    if (ok) {
      const int32_t h = it.g * a.G + r / it.O;
      const int32_t o = r % it.O;
      qp = a.q + (((int64_t)it.l * a.Hq + h) * a.obs_total + it.o0 + o) * kHeadDim + 8 * half;
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bf16x8 v = {};
      if (ok) v = *(const bf16x8 *)(qp + 16 * s);
      qa[t][s] = v;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int32_t rr = wr0 + 32 * t + 8 * (k >> 2) + 4 * half + (k & 3);
      float v = __builtin_inff();
      if (active && rr < R) {
        const int32_t h = it.g * a.G + rr / it.O;
        const int32_t o = rr % it.O;
        v = a.lse[((int64_t)it.l * a.Hq + h) * a.obs_total + it.o0 + o] * kLog2e;
      }
      nl[t][k] = -v;
    }
  }

  const int32_t s_begin = it.chunk * a.chunk_steps;
  const int32_t s_end = min(s_begin + a.chunk_steps, it.nsteps);
  const int32_t ntiles = (it.start + it.n + kTileKeys - 1) / kTileKeys;

  issue_step(a, it, s_begin, kbuf[0], wave, lane);
  for (int32_t step = s_begin; step < s_end; ++step) {
    const int cur = (step - s_begin) & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // combine the previous step's per-wave partials (row sets split over waves)
    if (wpr > 1 && step > s_begin && wrow == 0 && active && lane < 32) {
      const int pb = cur ^ 1;
      for (int tt = phase; tt < kStepTiles; tt += nph) {
        const int tile = (step - 1) * kStepTiles + tt;
        if (tile >= ntiles) break;
        float v = 0.f;
        for (int w = 0; w < wpr; ++w) v += part[pb][tt][w][lane];
        store_key(a, it, tile, lane, v);
      }
    }
    if (step + 1 < s_end) issue_step(a, it, step + 1, kbuf[cur ^ 1], wave, lane);
    if (!active) continue;

    const uint8_t *buf = kbuf[cur];
    for (int tt = phase; tt < kStepTiles; tt += nph) {
      const int tile = step * kStepTiles + tt;
      if (tile >= ntiles) break;
      const uint8_t *tb = buf + tt * (kTileKeys * kHeadDim * 2) + col * (kHeadDim * 2);
      bf16x8 kb[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int c = (2 * s + half) ^ (col & 15);
        kb[s] = *(const bf16x8 *)(tb + c * 16);
      }
      float sum = 0.f;
      if (mt_on0) {
        floatx16 acc = {};
#pragma unroll
        for (int s = 0; s < 8; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], kb[s], acc, 0, 0, 0);
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int k = 0; k < 16; k += 2) {
          s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[k], a.alpha, nl[0][k]));
          s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[k + 1], a.alpha, nl[0][k + 1]));
        }
        sum += s0 + s1;
      }
      if (mt_on1) {
        floatx16 acc = {};
#pragma unroll
        for (int s = 0; s < 8; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], kb[s], acc, 0, 0, 0);
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int k = 0; k < 16; k += 2) {
          s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[k], a.alpha, nl[1][k]));
          s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[k + 1], a.alpha, nl[1][k + 1]));
        }
        sum += s0 + s1;
      }
      sum += __shfl_xor(sum, 32);
      if (wpr == 1) {
        if (lane < 32) store_key(a, it, tile, col, sum);
      } else if (lane < 32) {
        part[cur][tt][wrow][lane] = sum;
      }
    }
  }
  if (wpr > 1) {
    __syncthreads();
    const int step = s_end - 1;
    const int pb = (step - s_begin) & 1;
    if (wrow == 0 && active && lane < 32) {
      for (int tt = phase; tt < kStepTiles; tt += nph) {
        const int tile = step * kStepTiles + tt;
        if (tile >= ntiles) break;
        float v = 0.f;
        for (int w = 0; w < wpr; ++w) v += part[pb][tt][w][lane];
        store_key(a, it, tile, lane, v);
      }
    }
  }
}

// VALU path: each wave owns whole 64-key quads (4 pages) of the chunk -- quad q goes
// to wave q % 4 -- and all rows of the row group, so waves never share data and never
// wait on each other.  The wave's LDS buffer is refilled with its next quad as soon as
// the current key rows have been pulled into registers.
__device__ __forceinline__ void issue_quad(const ScoreArgs &a, const Item &it, int32_t quad,
                                           uint8_t *buf, int lane) {
  const int32_t *bt = a.b.bt + (int64_t)it.i * a.b.max_pages;
#pragma unroll
  for (int pp = 0; pp < 4; ++pp) {
    const int32_t lp = quad * 4 + pp;
    if (lp < it.npages) {
      const int64_t phys = bt[lp];
      const uint16_t *page = a.k + (((int64_t)it.l * a.b.num_pages + phys) * a.b.Hkv + it.g) * kPageElems;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * r + (lane >> 4);
        const uint16_t *src = page + row * kHeadDim + (((lane & 15) ^ row) << 3);
        __builtin_amdgcn_global_load_lds((const void *)src,
                                         (lds_void *)(buf + pp * (kPageElems * 2) + r * 1024), 16, 0, 0);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads, 2) void score_valu_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[kWaves][4 * kPageElems * 2];   // 16 KiB per wave

  Item it;
  if (!decode_item(a, it)) return;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int32_t R = it.O * a.G;
  const int32_t r0 = it.rg * kRowsPerGroup;
  const int32_t r1 = min(R, r0 + kRowsPerGroup);
  const int32_t q_end = min(it.chunk * a.chunk_steps + a.chunk_steps, it.nsteps) * 2;
  const int32_t nquads = (it.npages + 3) / 4;
  uint8_t *mybuf = kbuf[wave];

  int32_t quad = it.chunk * a.chunk_steps * 2 + wave;
  if (quad < q_end && quad < nquads) issue_quad(a, it, quad, mybuf, lane);
  for (; quad < q_end && quad < nquads; quad += kWaves) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // lane = key: pull the key row (16 chunks of 16 B) out of the swizzled buffer
    bf16x2 kr[64];
    const uint8_t *rowp = mybuf + lane * (kHeadDim * 2);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const bf16x8 v = *(const bf16x8 *)(rowp + ((c ^ (lane & 15)) << 4));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16x2 p2;
        p2[0] = v[2 * e];
        p2[1] = v[2 * e + 1];
        kr[c * 4 + e] = p2;
      }
    }
    // the reads must have landed before the buffer is refilled
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const int32_t nxt = quad + kWaves;
    if (nxt < q_end && nxt < nquads) issue_quad(a, it, nxt, mybuf, lane);

    float sum = 0.f;
    for (int32_t r = r0; r < r1; ++r) {
      const int32_t h = it.g * a.G + r / it.O;
      const int32_t o = r - (r / it.O) * it.O;
      const int64_t qrow = ((int64_t)it.l * a.Hq + h) * a.obs_total + it.o0 + o;
      const bf16x2 *qp = (const bf16x2 *)(a.q + qrow * kHeadDim);
      float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
      for (int e = 0; e < 64; e += 4) {
        d0 = __builtin_amdgcn_fdot2_f32_bf16(qp[e], kr[e], d0, false);
        d1 = __builtin_amdgcn_fdot2_f32_bf16(qp[e + 1], kr[e + 1], d1, false);
        d2 = __builtin_amdgcn_fdot2_f32_bf16(qp[e + 2], kr[e + 2], d2, false);
        d3 = __builtin_amdgcn_fdot2_f32_bf16(qp[e + 3], kr[e + 3], d3, false);
      }
      const float dot = (d0 + d1) + (d2 + d3);
      sum += __builtin_amdgcn_exp2f(__builtin_fmaf(dot, a.alpha, -a.lse[qrow] * kLog2e));
    }
    const int32_t j = quad * 64 + lane - it.start;
    if (j >= 0 && j < it.n) {
      int64_t row = (int64_t)it.l * a.b.Hkv + it.g;
      if (a.partials) row += (int64_t)it.rg * a.b.L * a.b.Hkv;
      a.out[row * a.b.E + it.e0 + j] = sum;
    }
  }
}

// Sum per-row-group partials into scores (fixed order, deterministic).
__global__ __launch_bounds__(256) void score_combine_kernel(const float *__restrict__ part,
                                                            float *__restrict__ out, int64_t LHE,
                                                            int32_t nrg) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= LHE) return;
  float v = 0.f;
  for (int r = 0; r < nrg; ++r) v += part[(int64_t)r * LHE + idx];
  out[idx] = v;
}

__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ out, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < n) out[idx] = 0.f;
}

// Per-sequence work-item prefix for both paths: item_off_mfma, item_off_valu [S+1].
__global__ __launch_bounds__(256) void score_items_kernel(const int32_t *__restrict__ start,
                                                          const int32_t *__restrict__ len,
                                                          const int64_t *__restrict__ obs_off,
                                                          int32_t S, int32_t G, int32_t chunk_steps,
                                                          int32_t *__restrict__ off_mfma,
                                                          int32_t *__restrict__ off_valu) {
  __shared__ int32_t carry[2];
  __shared__ int32_t wsum[2][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) { carry[0] = 0; carry[1] = 0; }
  __syncthreads();
  for (int32_t base = 0; base < S; base += 256) {
    const int32_t i = base + threadIdx.x;
    int32_t cm = 0, cv = 0;
    if (i < S) {
      const int32_t npages = (start[i] + len[i] + kPage - 1) / kPage;
      const int32_t nsteps = (npages + kStepPages - 1) / kStepPages;
      const int32_t nch = (nsteps + chunk_steps - 1) / chunk_steps;
      const int32_t O = (int32_t)(obs_off[i + 1] - obs_off[i]);
      const int32_t R = O * G;
      const int32_t nrg = (R + kRowsPerGroup - 1) / kRowsPerGroup;
      const int32_t items = (len[i] > 0 && O > 0) ? nch * nrg : 0;
      if (O >= kMfmaMinObservers) cm = items; else cv = items;
    }
    // inclusive wave scans
    int32_t xm = cm, xv = cv;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t ym = __shfl_up(xm, d), yv = __shfl_up(xv, d);
      if (lane >= d) { xm += ym; xv += yv; }
    }
    if (lane == 63) { wsum[0][wave] = xm; wsum[1][wave] = xv; }
    __syncthreads();
    int32_t pm = carry[0], pv = carry[1];
    for (int w = 0; w < wave; ++w) { pm += wsum[0][w]; pv += wsum[1][w]; }
    if (i < S) { off_mfma[i] = pm + xm - cm; off_valu[i] = pv + xv - cv; }
    __syncthreads();
    if (threadIdx.x == 255) { carry[0] = pm + xm; carry[1] = pv + xv; }
    __syncthreads();
  }
  if (threadIdx.x == 0) { off_mfma[S] = carry[0]; off_valu[S] = carry[1]; }
}

struct Plan {
  int32_t chunk_steps;
  int64_t items_mfma, items_valu;   // per (layer, head)
  int32_t max_rg;
  bool any_partial;
  bool need_zero;
};

Plan make_plan(const Batch &b, int32_t G, const int64_t *obs_off_h, const int32_t *len_h,
               const int32_t *start_h) {
  Plan p{};
  int64_t total_steps = 0;
  p.max_rg = 0;
  for (int i = 0; i < b.S; ++i) {
    const int64_t O = obs_off_h[i + 1] - obs_off_h[i];
    if (len_h[i] <= 0 || O <= 0) continue;
    const int32_t npages = (start_h[i] + len_h[i] + kPage - 1) / kPage;
    const int32_t nsteps = (npages + kStepPages - 1) / kStepPages;
    const int32_t nrg = (int32_t)((O * G + kRowsPerGroup - 1) / kRowsPerGroup);
    total_steps += (int64_t)nsteps * nrg;
    p.max_rg = nrg > p.max_rg ? nrg : p.max_rg;
  }
  p.need_zero = false;
  for (int i = 0; i < b.S; ++i) {
    const int64_t O = obs_off_h[i + 1] - obs_off_h[i];
    if (len_h[i] <= 0) continue;
    const int32_t nrg = (int32_t)((O * G + kRowsPerGroup - 1) / kRowsPerGroup);
    if (O <= 0 || nrg < p.max_rg) p.need_zero = true;
  }
  total_steps *= (int64_t)b.L * b.Hkv;
  // aim for ~8 work items per resident workgroup slot (256 CUs x 2)
  int64_t cs = total_steps / (256 * 2 * 8);
  if (cs < 2) cs = 2;
  if (cs > 64) cs = 64;
  p.chunk_steps = (int32_t)cs;
  p.items_mfma = p.items_valu = 0;
  for (int i = 0; i < b.S; ++i) {
    const int64_t O = obs_off_h[i + 1] - obs_off_h[i];
    if (len_h[i] <= 0 || O <= 0) continue;
    const int32_t npages = (start_h[i] + len_h[i] + kPage - 1) / kPage;
    const int32_t nsteps = (npages + kStepPages - 1) / kStepPages;
    const int32_t nch = (nsteps + p.chunk_steps - 1) / p.chunk_steps;
    const int32_t nrg = (int32_t)((O * G + kRowsPerGroup - 1) / kRowsPerGroup);
    if (O >= kMfmaMinObservers) p.items_mfma += (int64_t)nch * nrg; else p.items_valu += (int64_t)nch * nrg;
  }
  p.any_partial = p.max_rg > 1;
  return p;
}

}  // namespace

size_t score_workspace_bytes(const Batch &b, int32_t Hq, const int64_t *obs_off_h,
                             const int32_t *len_h, const int32_t *start_h) {
  const int32_t G = Hq / b.Hkv;
  const Plan p = make_plan(b, G, obs_off_h, len_h, start_h);
  size_t bytes = 2 * ((size_t)b.S + 1) * sizeof(int32_t);
  bytes = (bytes + 255) & ~(size_t)255;
  if (p.any_partial) bytes += (size_t)p.max_rg * b.L * b.Hkv * b.E * sizeof(float);
  return bytes;
}

hipError_t launch_score(const kvs_cache &c, const Batch &b, const kvs_observers &o, float scale,
                        float *scores, void *ws, size_t ws_bytes, const int64_t *obs_off_h,
                        const int32_t *len_h, const int32_t *start_h, hipStream_t st) {
  const int32_t G = o.num_q_heads / b.Hkv;
  const Plan p = make_plan(b, G, obs_off_h, len_h, start_h);
  const int64_t LHE = (int64_t)b.L * b.Hkv * b.E;
  int32_t *off_m = (int32_t *)ws;
  int32_t *off_v = off_m + (b.S + 1);
  size_t head = 2 * ((size_t)b.S + 1) * sizeof(int32_t);
  head = (head + 255) & ~(size_t)255;
  float *partial = p.any_partial ? (float *)((uint8_t *)ws + head) : nullptr;
  (void)ws_bytes;

  // Every live entry of a scored sequence is written by exactly one work item (or,
  // with several row groups, one per group).  Zero-fill is needed only for
  // sequences that are not scored, or that have fewer row groups than the batch.
  if (LHE > 0 && p.need_zero) {
    float *z = p.any_partial ? partial : scores;
    const int64_t nz = p.any_partial ? LHE * p.max_rg : LHE;
    zero_kernel<<<(unsigned)((nz + 255) / 256), 256, 0, st>>>(z, nz);
  }
  if (p.items_mfma + p.items_valu == 0) return hipGetLastError();
  score_items_kernel<<<1, 256, 0, st>>>(b.start, b.len, o.obs_off, b.S, G, p.chunk_steps, off_m, off_v);

  ScoreArgs a{};
  a.k = (const uint16_t *)c.k;
  a.q = (const uint16_t *)o.q;
  a.lse = o.lse;
  a.obs_off = o.obs_off;
  a.out = p.any_partial ? partial : scores;
  a.b = b;
  a.obs_total = o.obs_total;
  a.Hq = o.num_q_heads;
  a.G = G;
  a.chunk_steps = p.chunk_steps;
  a.partials = p.any_partial ? 1 : 0;
  a.alpha = scale * kLog2e;
  const int64_t LH = (int64_t)b.L * b.Hkv;
  if (p.items_mfma > 0) {
    a.item_off = off_m;
    a.items_per_lg = (int32_t)p.items_mfma;
    a.total_items = p.items_mfma * LH;
    a.padded_items = (a.total_items + 7) & ~(int64_t)7;
    score_mfma_kernel<<<(unsigned)a.padded_items, kThreads, 0, st>>>(a);
  }
  if (p.items_valu > 0) {
    a.item_off = off_v;
    a.items_per_lg = (int32_t)p.items_valu;
    a.total_items = p.items_valu * LH;
    a.padded_items = (a.total_items + 7) & ~(int64_t)7;
    score_valu_kernel<<<(unsigned)a.padded_items, kThreads, 0, st>>>(a);
  }
  if (p.any_partial) {
    score_combine_kernel<<<(unsigned)((LHE + 255) / 256), 256, 0, st>>>(partial, scores, LHE, p.max_rg);
  }
  return hipGetLastError();
}

}  // namespace kvs
