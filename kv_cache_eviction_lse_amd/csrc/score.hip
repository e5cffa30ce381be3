// kvs_score kernels: attention recovered from the log-sum-exp, summed per cached entry.
//
// ActKV Dissected, Component 3: the LSE of each query row is a byproduct of paged
// attention, so the probability a row puts on an entry is exp(logit - LSE): no
// softmax pass, no attention matrix.  Component 1: the signal of an entry is the
// attention it receives from all observer (action) tokens, here also summed over
// the query heads of the entry's GQA group.
//
// Work items are chunks of consecutive 4-page steps of one stream and one group of its
// observer rows.  A sequence's rows R = O G decide its path:
//   score_valu_kernel  (R < 16): one key per lane, 64 keys per wave; the key row is
//       pulled from LDS into registers and every observer row (uniform across the wave,
//       so it lives in SGPRs) is dotted with v_dot2c_f32_bf16.  Row groups of 256.
//   score_mfma_kernel  (16 <= R <= 128): QK^T on v_mfma_f32_32x32x16_bf16 with the
//       observer rows on M and the keys on N, so each lane holds one key and 16 rows and
//       the exp and the row sum stay in-lane; 32- or 64-row sets, waves split the tiles.
//   score_pipe_kernel<4> (128 < R <= 256) and score_pipe_kernel<8> (R > 256, row groups
//       of 512): every wave owns 64 rows, so one workgroup stages each K step in LDS
//       once for all its rows; the MFMAs of one key tile overlap the exp work of the
//       previous one.
// K pages stream from HBM straight into LDS (global_load_lds_dwordx4, 1 KiB per
// instruction, XOR-swizzled 16-byte chunks) through a ring of 16 KiB steps.
// All evaluate p = exp2(fma(dot, scale*log2 e, -LSE*log2 e)) and accumulate in fp32.
#include "kvs_internal.h"

#include <type_traits>

namespace kvs {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStepPages = 4;                       // one pipeline step: 4 pages = 64 keys = 16 KiB
constexpr int kStepKeys = kStepPages * kPage;
constexpr int kStepBytes = kStepPages * kPageElems * 2;
constexpr int kRing = 4;                            // LDS ring depth: 3 steps in flight per workgroup
constexpr int kTileKeys = 32;                       // one MFMA N tile (2 pages)
constexpr int kStepTiles = kStepKeys / kTileKeys;   // 2
constexpr int kRowsPerGroup = 256;                  // observer rows of one item (VALU and small MFMA paths)
constexpr int kWideRows = 512;                      // observer rows of one item of score_pipe_kernel<8>
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSmallSeqs = 255;                     // item offsets travel in the kernel arguments
constexpr int kMaxChunkSteps = 128;                 // chunk length limit (block-table slice in LDS)

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
  int32_t rows_per_group;     // observer rows per work item on this path
  float alpha;                // scale * log2(e)
  int32_t use_small;          // 1: item offsets are in small_off (batches of <= 255 sequences)
  int32_t small_off[kSmallSeqs + 1];
};

// The scoring path of a sequence with O observers and R = O G rows.
enum Path : int { kPathValu = 0, kPathMfma = 1, kPathPipe4 = 2, kPathPipe8 = 3, kPaths = 4 };
__host__ __device__ inline int path_of(int64_t O, int64_t R) {
  if (R < kMfmaMinRows) return kPathValu;
  if (R <= 128) return kPathMfma;
  return R <= 256 ? kPathPipe4 : kPathPipe8;
}
__host__ __device__ inline int32_t rows_per_group(int path) {
  return path == kPathPipe8 ? kWideRows : kRowsPerGroup;
}

struct Item {
  int32_t i, l, g, rg, nrg, chunk;
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
  const int32_t *off = a.use_small ? a.small_off : a.item_off;
  int lo = 0, hi = a.b.S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= rem) lo = mid; else hi = mid;
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
  const int32_t local = rem - off[lo];
  // the row groups of one chunk are consecutive items, so they run at the same time on
  // the same XCD and share the chunk's K lines in its L2
  it.nrg = (it.O * a.G + a.rows_per_group - 1) / a.rows_per_group;
  it.chunk = local / it.nrg;
  it.rg = local - it.chunk * it.nrg;
  // host and device item counts agree by construction; refuse anything else
  if (it.n <= 0 || it.O <= 0 || it.chunk >= nchunks) return false;
  return true;
}

// The item's fields are the same in every lane; saying so keeps the loop bounds, page
// indices and branches that derive from them in scalar registers and scalar branches.
__device__ __forceinline__ int64_t uni64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void make_uniform(Item &it) {
  it.i = __builtin_amdgcn_readfirstlane(it.i);
  it.l = __builtin_amdgcn_readfirstlane(it.l);
  it.g = __builtin_amdgcn_readfirstlane(it.g);
  it.rg = __builtin_amdgcn_readfirstlane(it.rg);
  it.nrg = __builtin_amdgcn_readfirstlane(it.nrg);
  it.chunk = __builtin_amdgcn_readfirstlane(it.chunk);
  it.start = __builtin_amdgcn_readfirstlane(it.start);
  it.n = __builtin_amdgcn_readfirstlane(it.n);
  it.O = __builtin_amdgcn_readfirstlane(it.O);
  it.npages = __builtin_amdgcn_readfirstlane(it.npages);
  it.nsteps = __builtin_amdgcn_readfirstlane(it.nsteps);
  it.e0 = uni64(it.e0);
  it.o0 = uni64(it.o0);
}

// One LDS DMA instruction: lane t's 16 bytes from src land at LDS byte address
// lds + 16 t (lds is wave-uniform; M0 carries it).  Written as inline asm because the
// compiler cannot tell which LDS bytes a pending DMA will write, so after the builtin
// form it drains every outstanding vector load before the next LDS read, i.e. the
// whole prefetch ring at every step.  Ordering is explicit instead: a slot is read
// only after the ring barrier's vmcnt wait and s_barrier, and refilled only after
// the barrier that follows the last read of it.  No output registers; the address
// registers are consumed at issue.  M0 is saved and restored around the DMA.  When a
// stream's rows form one row group its K rows are read once per call, so the load is
// marked non-temporal (streaming); with several row groups the other groups' workgroups
// read the same lines, so they stay cacheable.
__device__ __forceinline__ void lds_dma16(const void *src, uint32_t lds, bool stream) {
  uint32_t saved;
  if (stream)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(lds)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, off\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(src), "s"(lds)
        : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const lds_void *)p;
}

// Issue this wave's page (page w of the 4-page step) into an LDS ring slot.  Lane t
// of instruction r fills LDS chunk t%16 of page row 4r + t/16 with global chunk
// (t%16) ^ row, so that a later read of chunk c of row n lands on c ^ (n%16).  Page
// ids come from the chunk's block-table slice staged in LDS, so no global load sits
// between two page loads.  Returns the number of load instructions issued (0 or 4).
__device__ __forceinline__ int issue_step(const ScoreArgs &a, const Item &it, int step, uint8_t *buf,
                                          const int32_t *bt_lds, int32_t page0, int wave, int lane) {
  const int lp = step * kStepPages + wave;
  if (lp >= it.npages) return 0;
  const int64_t phys = __builtin_amdgcn_readfirstlane(bt_lds[lp - page0]);
  const uint16_t *page = a.k + (((int64_t)it.l * a.b.num_pages + phys) * a.b.Hkv + it.g) * kPageElems;
  const int row_in_instr = lane >> 4;
  const int chunk = lane & 15;
  const uint32_t dst0 = __builtin_amdgcn_readfirstlane(lds_addr(buf + wave * (kPageElems * 2)));
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * r + row_in_instr;
    const uint16_t *src = page + row * kHeadDim + ((chunk ^ row) << 3);
    lds_dma16(src, dst0 + r * 1024, it.nrg == 1);
  }
  return 4;
}

// Ring barrier: wait until this wave's loads of the current step have landed,
// leaving `later` loads (of later steps) in flight, and its LDS writes are done;
// then a plain s_barrier.  (A __syncthreads() would also drain every outstanding
// vector memory operation, i.e. the whole prefetch ring, at each step.)  Vector
// loads complete in issue order; stores in between only make the wait longer.
__device__ __forceinline__ void ring_barrier(int later) {
  if (later >= 24) asm volatile("s_waitcnt vmcnt(24) lgkmcnt(0)" ::: "memory");
  else if (later >= 20) asm volatile("s_waitcnt vmcnt(20) lgkmcnt(0)" ::: "memory");
  else if (later >= 16) asm volatile("s_waitcnt vmcnt(16) lgkmcnt(0)" ::: "memory");
  else if (later >= 12) asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)" ::: "memory");
  else if (later >= 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
  else if (later >= 4) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// B operands of one 32-key tile: lane (n, h) gets dims 16s + 8h .. +8 of key n.
__device__ __forceinline__ void read_tile(const uint8_t *buf, int tt, int col, int half, bf16x8 kb[8]) {
  const uint8_t *tb = buf + tt * (kTileKeys * kHeadDim * 2) + col * (kHeadDim * 2);
#pragma unroll
  for (int s = 0; s < 8; ++s) kb[s] = *(const bf16x8 *)(tb + (((2 * s + half) ^ (col & 15)) << 4));
}

__device__ __forceinline__ floatx16 qk_tile(const bf16x8 qa[8], const bf16x8 kb[8]) {
  floatx16 acc = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], kb[s], acc, 0, 0, 0);
  return acc;
}

// sum over the 16 rows a lane holds of exp2(acc * alpha - lse*log2e)
__device__ __forceinline__ float exp_rows(const floatx16 &acc, float alpha, const float nl[16]) {
  float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
  for (int k = 0; k < 16; k += 4) {
    s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[k], alpha, nl[k]));
    s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[k + 1], alpha, nl[k + 1]));
    s2 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[k + 2], alpha, nl[k + 2]));
    s3 += __builtin_amdgcn_exp2f(__builtin_fmaf(acc[k + 3], alpha, nl[k + 3]));
  }
  return (s0 + s1) + (s2 + s3);
}

// Main loop.  NPH = number of tile phases per step (1: every wave takes both tiles of
// a step with its own rows; 2: waves of phase p take tile p).  With NPH = 1 the two
// tiles are software-pipelined (MFMA of tile 1 in flight during the exp of tile 0).
template <int NPH>
__device__ __forceinline__ void score_steps(const ScoreArgs &a, const Item &it, uint8_t (*ring)[kStepBytes],
                                            float (*part)[kStepTiles][kWaves][kTileKeys],
                                            const int32_t *bt_lds, int32_t page0, int wave, int lane,
                                            int wpr, int phase, int wrow, bool active, bool on0,
                                            bool on1, const bf16x8 (*qa)[8], const float (*nl)[16]) {
  constexpr int TPW = kStepTiles / NPH;   // tiles per wave per step
  const int half = lane >> 5;
  const int col = lane & 31;
  const int32_t s_begin = it.chunk * a.chunk_steps;
  const int32_t s_end = min(s_begin + a.chunk_steps, it.nsteps);
  const int32_t ntiles = (it.start + it.n + kTileKeys - 1) / kTileKeys;

  // loads this wave issues for step j (its page of the step, if the page exists)
  auto nloads = [&](int32_t j) -> int { return (j < s_end && j * kStepPages + wave < it.npages) ? 4 : 0; };
  // prologue: kRing - 1 steps in flight
#pragma unroll
  for (int u = 0; u < kRing - 1; ++u)
    if (s_begin + u < s_end) issue_step(a, it, s_begin + u, ring[u], bt_lds, page0, wave, lane);

  for (int32_t step = s_begin; step < s_end; ++step) {
    const int k = step - s_begin;
    const int cur = k & (kRing - 1);
    ring_barrier(nloads(step + 1) + nloads(step + 2));
    // combine the previous step's per-wave partials (row sets split over waves)
    if (wpr > 1 && k > 0 && wrow == 0 && active && lane < 32) {
      const int pb = (k - 1) & 1;
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tt = phase + u * NPH;
        const int tile = (step - 1) * kStepTiles + tt;
        float v = 0.f;
        for (int w = 0; w < wpr; ++w) v += part[pb][tt][w][lane];
        if (tile < ntiles) store_key(a, it, tile, lane, v);
      }
    }
    // refill the slot freed by the previous step
    if (step + kRing - 1 < s_end)
      issue_step(a, it, step + kRing - 1, ring[(k + kRing - 1) & (kRing - 1)], bt_lds, page0, wave, lane);
    if (!active) continue;
    const uint8_t *buf = ring[cur];
    const int tile0 = step * kStepTiles;
    float sums[TPW];
    if (on1) {
      bf16x8 kb[8];
      read_tile(buf, phase, col, half, kb);
      floatx16 a0 = qk_tile(qa[0], kb);
      floatx16 a1 = qk_tile(qa[1], kb);
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        floatx16 b0, b1;
        if (u + 1 < TPW) {
          read_tile(buf, phase + (u + 1) * NPH, col, half, kb);
          b0 = qk_tile(qa[0], kb);
          b1 = qk_tile(qa[1], kb);
        }
        sums[u] = exp_rows(a0, a.alpha, nl[0]) + exp_rows(a1, a.alpha, nl[1]);
        if (u + 1 < TPW) { a0 = b0; a1 = b1; }
      }
    } else if (on0) {
      bf16x8 kb[8];
      read_tile(buf, phase, col, half, kb);
      floatx16 a0 = qk_tile(qa[0], kb);
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        floatx16 b0;
        if (u + 1 < TPW) {
          read_tile(buf, phase + (u + 1) * NPH, col, half, kb);
          b0 = qk_tile(qa[0], kb);
        }
        sums[u] = exp_rows(a0, a.alpha, nl[0]);
        if (u + 1 < TPW) a0 = b0;
      }
    } else {
#pragma unroll
      for (int u = 0; u < TPW; ++u) sums[u] = 0.f;
    }
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int tt = phase + u * NPH;
      const float v = sums[u] + __shfl_xor(sums[u], 32);
      if (lane < 32) {
        if (wpr == 1) {
          if (tile0 + tt < ntiles) store_key(a, it, tile0 + tt, col, v);
        } else {
          part[k & 1][tt][wrow][lane] = v;
        }
      }
    }
  }
  if (wpr > 1) {
    __syncthreads();
    const int k = s_end - 1 - s_begin;
    const int step = s_end - 1;
    if (wrow == 0 && active && lane < 32) {
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const int tt = phase + u * NPH;
        const int tile = step * kStepTiles + tt;
        float v = 0.f;
        for (int w = 0; w < wpr; ++w) v += part[k & 1][tt][w][lane];
        if (tile < ntiles) store_key(a, it, tile, lane, v);
      }
    }
  }
}

// sum over both M tiles of exp2(acc * alpha - lse*log2e): 32 values per lane, four
// independent partial sums, each started from its first term.
__device__ __forceinline__ float exp_rows2(const floatx16 &x0, const floatx16 &x1, float alpha,
                                           const float (*nl)[16]) {
  float s0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x0[0], alpha, nl[0][0]));
  float s1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x0[1], alpha, nl[0][1]));
  float s2 = __builtin_amdgcn_exp2f(__builtin_fmaf(x1[0], alpha, nl[1][0]));
  float s3 = __builtin_amdgcn_exp2f(__builtin_fmaf(x1[1], alpha, nl[1][1]));
#pragma unroll
  for (int k = 2; k < 16; k += 2) {
    s0 += __builtin_amdgcn_exp2f(__builtin_fmaf(x0[k], alpha, nl[0][k]));
    s1 += __builtin_amdgcn_exp2f(__builtin_fmaf(x0[k + 1], alpha, nl[0][k + 1]));
    s2 += __builtin_amdgcn_exp2f(__builtin_fmaf(x1[k], alpha, nl[1][k]));
    s3 += __builtin_amdgcn_exp2f(__builtin_fmaf(x1[k + 1], alpha, nl[1][k + 1]));
  }
  return (s0 + s1) + (s2 + s3);
}

// One LDS DMA instruction with a wave-uniform page base (SGPRs) and a per-lane byte
// offset: lane t's 16 bytes from base + voff land at LDS byte address lds + 16 t.
// Same ordering contract as lds_dma16.
__device__ __forceinline__ void lds_dma16_s(const uint16_t *base, uint32_t voff, uint32_t lds, bool stream) {
  uint32_t saved;
  if (stream)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:0 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(lds)
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 offset:0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(base), "s"(lds)
        : "memory");
}

// One pipeline phase: the QK^T MFMAs of the next key tile (LDS bytes tile_base + rd[s]
// for k-step s) overlapped with the exp/sum of the previous tile's accumulators, for the
// T (1 or 2) 32-row M tiles of the wave.  The scheduling barriers fix the issue order:
// the 8 LDS reads first, then one MFMA per six VALU operations, so that the matrix core
// runs while the exp work issues.  With tile_base a compile-time constant the reads take
// it as their immediate offset.
template <int T>
__device__ __forceinline__ float pipe_phase(const uint8_t *tile_base, const uint32_t rd[8],
                                            const bf16x8 (*qa)[8], floatx16 &n0, floatx16 &n1,
                                            const floatx16 &p0, const floatx16 &p1, float alpha,
                                            const float (*nl)[16]) {
  bf16x8 kb[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) kb[s] = *(const bf16x8 *)(tile_base + rd[s]);
  floatx16 c0 = {}, c1 = {};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], kb[s], c0, 0, 0, 0);
    if constexpr (T == 2) c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], kb[s], c1, 0, 0, 0);
  }
  float v;
  if constexpr (T == 2) v = exp_rows2(p0, p1, alpha, nl);
  else v = exp_rows(p0, alpha, nl[0]);
  n0 = c0;
  if constexpr (T == 2) n1 = c1;
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
  for (int i = 0; i < 8 * T; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
  }
  return v;
}

// ---- The pipelined scorer for more than 128 rows ----
//
// W waves per workgroup and up to 2 W 32-row M tiles of observer rows.  One workgroup
// covers a row group of up to 64 W rows and stages each K step in LDS once for all of
// them.  With W = 8 (one workgroup per CU) tile k goes to wave k mod W, so wave w owns
// rows 32 w + i and 32 (w + W) + i (i < 32) when they exist: dealing the tiles out one
// at a time spreads a partial row group over more waves, hence more SIMDs (10 tiles, R =
// 300, put at most 3 on a SIMD instead of 4).  With W = 4 wave w owns tiles 2w, 2w + 1.  A step is 4 pages (64 keys, two 32-key tiles); waves 0..3 each DMA
// one page of it.  Tile u's MFMAs overlap tile u-1's exp work:
//   phase A of step j:  MFMA(j, tile 1)    || exp(j, tile 0)
//   phase B of step j:  ring barrier(j+1), refill, combine;
//                       MFMA(j+1, tile 0)  || exp(j, tile 1)
// The loop is unrolled over the ring slots, so every LDS read is a per-lane register
// plus an immediate and every DMA a scalar page base plus a per-lane offset computed
// once; control flow in the loop is uniform across the workgroup.  Waves run the loop
// with T = 2, 1 or 0 tiles; those without rows run the same barriers, loads and combines
// without the arithmetic.  Each wave writes its per-lane partial sums (both lane
// halves) to part[step % 2]; after barrier j+1, wave 0 sums tile 0 of step j and
// wave 1 tile 1 of step j-1 in wave order (deterministic), and stores the 32 keys.
// A wave is at most one barrier ahead of another, so two partial buffers suffice.
template <int W>
struct PipeShape {
  static constexpr int kThreads = 64 * W;
  static constexpr int kSlots = W == 8 ? 8 : 4;       // ring depth: kSlots - 1 steps in flight
  static constexpr int kWgPerCu = W == 8 ? 1 : 2;
};

template <int W, int T>
__device__ __forceinline__ void pipe_loop(const ScoreArgs &a, const Item &it, uint8_t (*ring)[kStepBytes],
                                          float (*part)[kStepTiles][W][64], const int32_t *bt_lds, int32_t page0,
                                          int wave, int lane, int nact, const bf16x8 (*qa)[8],
                                          const float (*nl)[16]) {
  constexpr int S = PipeShape<W>::kSlots;
  const int half = lane >> 5;
  const int col = lane & 31;
  const bool stream = it.nrg == 1;
  const bool dma = wave < kStepPages;
  const int32_t s_begin = it.chunk * a.chunk_steps;
  const int32_t s_end = min(s_begin + a.chunk_steps, it.nsteps);
  const int32_t ntiles = (it.start + it.n + kTileKeys - 1) / kTileKeys;
  // this wave's page of step j is logical page 4j + wave
  auto nloads = [&](int32_t j) -> int {
    return (dma && j < s_end && j * kStepPages + wave < it.npages) ? 4 : 0;
  };
  // per-lane source offsets of the 4 DMA instructions of a page (bytes): lane t of
  // instruction r fills LDS chunk t%16 of row 4r + t/16 with global chunk (t%16) ^ row
  uint32_t voff[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * r + (lane >> 4);
    voff[r] = (uint32_t)(row * kHeadDim * 2 + (((lane & 15) ^ row) << 4));
  }
  const int64_t head_base = ((int64_t)it.l * a.b.num_pages) * a.b.Hkv + it.g;
  auto issue = [&](int32_t j, uint8_t *buf) {
    const int lp = j * kStepPages + wave;
    if (!dma || j >= s_end || lp >= it.npages) return;
    const int64_t phys = __builtin_amdgcn_readfirstlane(bt_lds[lp - page0]);
    const uint16_t *page = a.k + (head_base + phys * a.b.Hkv) * kPageElems;
    const uint32_t dst0 = __builtin_amdgcn_readfirstlane(lds_addr(buf + wave * (kPageElems * 2)));
#pragma unroll
    for (int r = 0; r < 4; ++r) lds_dma16_s(page, voff[r], dst0 + r * 1024, stream);
  };
  auto combine = [&](int32_t step, int tt) {
    // the buffer offset goes through an empty asm so that the compiler computes it here
    // instead of keeping one address per (buffer, tile) live across the loop
    int off = ((((step - s_begin) & 1) * kStepTiles + tt) * W) * 64 + lane;
    asm volatile("" : "+v"(off));
    const float *pp = &part[0][0][0][0] + off;
    float v = 0.f;
    for (int w = 0; w < nact; ++w) v += pp[w * 64] + pp[w * 64 + 32];
    const int32_t tile = step * kStepTiles + tt;
    if (tile < ntiles) store_key(a, it, tile, lane, v);
  };
  // B operand k-step s of key n = col: dims 16s + 8h .. +8, stored at chunk (2s+h) ^ (n % 16)
  uint32_t rd[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) rd[s] = (uint32_t)(col * (kHeadDim * 2) + (((2 * s + half) ^ (col & 15)) << 4));

#pragma unroll
  for (int u = 0; u < S - 1; ++u) issue(s_begin + u, ring[u]);
  {
    int later = 0;
#pragma unroll
    for (int u = 1; u < S - 1; ++u) later += nloads(s_begin + u);
    ring_barrier(later);
  }
  issue(s_begin + S - 1, ring[S - 1]);

  constexpr int kTileBytes = kTileKeys * kHeadDim * 2;
  floatx16 t0a = {}, t0b = {}, t1a = {}, t1b = {};
  if constexpr (T > 0) {
    bf16x8 kb[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) kb[s] = *(const bf16x8 *)(ring[0] + rd[s]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      t0a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], kb[s], t0a, 0, 0, 0);
      if constexpr (T == 2) t0b = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], kb[s], t0b, 0, 0, 0);
    }
  }
  // one step with its ring slot fixed at compile time
  auto do_step = [&](auto slot_c, int32_t step) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_c)::value;
    constexpr int NEXT = (SLOT + 1) % S;
    float *mine = &part[(SLOT & 1)][0][wave][0];
    if constexpr (T > 0) mine[lane] = pipe_phase<T>(ring[SLOT] + kTileBytes, rd, qa, t1a, t1b, t0a, t0b, a.alpha, nl);
    if (step + 1 < s_end) {
      int later = 0;
#pragma unroll
      for (int u = 2; u < S; ++u) later += nloads(step + u);
      ring_barrier(later);
      issue(step + S, ring[SLOT]);
      if (lane < 32) {
        if (wave == 0) combine(step, 0);
        else if (wave == 1 && step > s_begin) combine(step - 1, 1);
      }
      if constexpr (T > 0)
        mine[W * 64 + lane] = pipe_phase<T>(ring[NEXT], rd, qa, t0a, t0b, t1a, t1b, a.alpha, nl);
    } else if constexpr (T > 0) {
      mine[W * 64 + lane] = T == 2 ? exp_rows2(t1a, t1b, a.alpha, nl) : exp_rows(t1a, a.alpha, nl[0]);
    }
  };
  for (int32_t step = s_begin; step < s_end; step += S) {
    do_step(std::integral_constant<int, 0>{}, step);
    if (step + 1 >= s_end) break;
    do_step(std::integral_constant<int, 1>{}, step + 1);
    if (step + 2 >= s_end) break;
    do_step(std::integral_constant<int, 2>{}, step + 2);
    if (step + 3 >= s_end) break;
    do_step(std::integral_constant<int, 3>{}, step + 3);
    if constexpr (S == 8) {
      if (step + 4 >= s_end) break;
      do_step(std::integral_constant<int, 4>{}, step + 4);
      if (step + 5 >= s_end) break;
      do_step(std::integral_constant<int, 5>{}, step + 5);
      if (step + 6 >= s_end) break;
      do_step(std::integral_constant<int, 6>{}, step + 6);
      if (step + 7 >= s_end) break;
      do_step(std::integral_constant<int, 7>{}, step + 7);
    }
  }
  __syncthreads();
  if (lane < 32) {
    const int32_t last = s_end - 1;
    if (wave == 0) combine(last, 0);
    else if (wave == 1) combine(last, 1);
    else if (wave == 2 && last > s_begin) combine(last - 1, 1);
  }
}

template <int W>
__global__ __launch_bounds__(PipeShape<W>::kThreads, PipeShape<W>::kWgPerCu) void score_pipe_kernel(ScoreArgs a) {
  constexpr int S = PipeShape<W>::kSlots;
  __shared__ __attribute__((aligned(16))) uint8_t ring[S][kStepBytes];
  __shared__ float part[2][kStepTiles][W][64];
  __shared__ int32_t bt_lds[kMaxChunkSteps * kStepPages];

  Item it;
  if (!decode_item(a, it)) return;
  make_uniform(it);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int col = lane & 31;
  const int32_t R = it.O * a.G;
  const int32_t r0 = it.rg * a.rows_per_group;
  const int32_t rows_here = min(a.rows_per_group, R - r0);
  // 32-row M tiles.  W = 8: tile k of the row group goes to wave k mod W, so this wave's
  // tile t (t < nt) is rows r0 + 32 (wave + W t) + i.  W = 4 (two workgroups per CU):
  // wave w takes tiles 2w and 2w + 1, and a wave with rows always runs both (a partial
  // second tile computes zero rows), which keeps that kernel's code as tuned.
  constexpr bool kDeal = W == 8;
  const int32_t ntr = (rows_here + 31) / 32;
  const int nt = kDeal ? (wave < ntr ? 1 : 0) + (wave + W < ntr ? 1 : 0) : (2 * wave < ntr ? 2 : 0);
  const int nact = kDeal ? (ntr < W ? (int)ntr : W) : (int)((ntr + 1) / 2);   // waves with rows
  auto row_of = [&](int t, int i) -> int32_t {
    return kDeal ? r0 + 32 * (wave + W * t) + i : r0 + 64 * wave + 32 * t + i;
  };

  // Observer rows of this wave as MFMA A operands: lane (m, h) holds row m of the tile,
  // dims 16s + 8h .. +8 for k-step s.  Loads are unconditional (invalid rows read
  // row 0 of the stream and are zeroed) so that they all issue back to back.
  bf16x8 qa[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int32_t r = row_of(t, col);
    const bool ok = t < nt && r < R;
    const int32_t rc = ok ? r : 0;
    const int32_t h = it.g * a.G + rc / it.O;
    const int32_t o = rc - (rc / it.O) * it.O;
    const uint16_t *qp = a.q + (((int64_t)it.l * a.Hq + h) * a.obs_total + it.o0 + o) * kHeadDim + 8 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 v = *(const bf16x8 *)(qp + 16 * s);
      const bf16x8 z = {};
      qa[t][s] = ok ? v : z;
    }
  }
  // LSE of the wave's rows, one per lane (lane 32 t + i: row i of tile t), then spread
  // to the accumulator layout: register k of M tile t holds row 8(k/4) + 4h + k%4 of the
  // tile.  Rows past the end have zero Q and LSE +inf, so they add exactly 0.
  float my_nl;
  {
    const int32_t r = row_of(lane >> 5, lane & 31);
    const bool ok = (lane >> 5) < nt && r < R && r < r0 + rows_here;
    const int32_t rc = ok ? r : 0;
    const int32_t h = it.g * a.G + rc / it.O;
    const int32_t o = rc - (rc / it.O) * it.O;
    const float v = a.lse[((int64_t)it.l * a.Hq + h) * a.obs_total + it.o0 + o] * kLog2e;
    my_nl = ok ? -v : -__builtin_inff();
  }
  const int32_t s_begin = it.chunk * a.chunk_steps;
  const int32_t page0 = s_begin * kStepPages;
  const int32_t page1 = min(it.npages, (s_begin + a.chunk_steps) * kStepPages);
  const int32_t *bt_row = a.b.bt + (int64_t)it.i * a.b.max_pages;
  for (int32_t p = page0 + (int32_t)threadIdx.x; p < page1; p += PipeShape<W>::kThreads) bt_lds[p - page0] = bt_row[p];
  float nl[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int k = 0; k < 16; ++k) nl[t][k] = __shfl(my_nl, 32 * t + 8 * (k >> 2) + 4 * half + (k & 3));
  __syncthreads();
  if (nt == 2)
    pipe_loop<W, 2>(a, it, ring, part, bt_lds, page0, wave, lane, nact, qa, nl);
  else if (kDeal && nt == 1)
    pipe_loop<W, kDeal ? 1 : 2>(a, it, ring, part, bt_lds, page0, wave, lane, nact, qa, nl);
  else
    pipe_loop<W, 0>(a, it, ring, part, bt_lds, page0, wave, lane, nact, qa, nl);
}

__global__ __launch_bounds__(kThreads, 2) void score_mfma_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kRing][kStepBytes];
  __shared__ float part[kRing][kStepTiles][kWaves][kTileKeys];
  __shared__ int32_t bt_lds[kMaxChunkSteps * kStepPages];

  Item it;
  if (!decode_item(a, it)) return;
  make_uniform(it);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5;
  const int col = lane & 31;

  // Row sets (at most 128 rows here): 65..128 rows -> two 64-row sets (2 M tiles per
  // wave); up to 64 rows -> 32-row sets (1 M tile).  Two waves per set; the waves of
  // tile phase p (waves 2p, 2p + 1) take tile p of every step.
  const int32_t R = it.O * a.G;
  const int32_t r0 = it.rg * kRowsPerGroup;
  const int32_t rows_here = min(kRowsPerGroup, R - r0);
  const int rw = rows_here > 64 ? 64 : 32;                              // rows per wave
  const int wpr = (rows_here + rw - 1) / rw;                            // waves per row set
  const int phase = wave / 2;
  const int wrow = wave & 1;
  const bool active = wrow < wpr;
  const int32_t wr0 = r0 + wrow * rw;
  const bool on0 = active && wr0 < R;
  const bool on1 = active && rw == 64 && wr0 + 32 < R;

  // Observer rows of this wave as MFMA A operands: lane (m, h) holds row m,
  // dims 16s + 8h .. +8 for k-step s.  Loads are unconditional (invalid rows read
  // row 0 of the stream and are zeroed) so that they all issue back to back.
  bf16x8 qa[2][8];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int32_t r = wr0 + 32 * t + col;
    const bool ok = active && r < R && (t == 0 || rw == 64);
    const int32_t rc = ok ? r : 0;
    const int32_t h = it.g * a.G + rc / it.O;
    const int32_t o = rc - (rc / it.O) * it.O;
    const uint16_t *qp = a.q + (((int64_t)it.l * a.Hq + h) * a.obs_total + it.o0 + o) * kHeadDim + 8 * half;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 v = *(const bf16x8 *)(qp + 16 * s);
      const bf16x8 z = {};
      qa[t][s] = ok ? v : z;
    }
  }
  // LSE of the wave's rows, one per lane, then spread to the accumulator layout:
  // register k of M tile t holds row 32t + 8(k/4) + 4h + k%4.
  float my_nl;
  {
    const int32_t r = wr0 + lane;
    const bool ok = active && r < R && lane < rw;
    const int32_t rc = ok ? r : 0;
    const int32_t h = it.g * a.G + rc / it.O;
    const int32_t o = rc - (rc / it.O) * it.O;
    const float v = a.lse[((int64_t)it.l * a.Hq + h) * a.obs_total + it.o0 + o] * kLog2e;
    my_nl = ok ? -v : -__builtin_inff();
  }
  // the chunk's slice of the block table
  const int32_t s_begin = it.chunk * a.chunk_steps;
  const int32_t page0 = s_begin * kStepPages;
  const int32_t page1 = min(it.npages, (s_begin + a.chunk_steps) * kStepPages);
  const int32_t *bt_row = a.b.bt + (int64_t)it.i * a.b.max_pages;
  for (int32_t p = page0 + (int32_t)threadIdx.x; p < page1; p += kThreads) bt_lds[p - page0] = bt_row[p];
  float nl[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int k = 0; k < 16; ++k) nl[t][k] = __shfl(my_nl, 32 * t + 8 * (k >> 2) + 4 * half + (k & 3));
  __syncthreads();

  score_steps<2>(a, it, ring, part, bt_lds, page0, wave, lane, wpr, phase, wrow, active, on0, on1, qa, nl);
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
      const uint32_t dst0 = __builtin_amdgcn_readfirstlane(lds_addr(buf + pp * (kPageElems * 2)));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * r + (lane >> 4);
        const uint16_t *src = page + row * kHeadDim + (((lane & 15) ^ row) << 3);
        lds_dma16(src, dst0 + r * 1024, it.nrg == 1);
      }
    }
  }
}

__global__ __launch_bounds__(kThreads, 2) void score_valu_kernel(ScoreArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[kWaves][4 * kPageElems * 2];   // 16 KiB per wave

  Item it;
  if (!decode_item(a, it)) return;
  make_uniform(it);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar branches
  const int lane = threadIdx.x & 63;
  const int32_t R = it.O * a.G;
  const int32_t r0 = it.rg * kRowsPerGroup;
  const int32_t r1 = min(R, r0 + kRowsPerGroup);
  const int32_t q_end = min(it.chunk * a.chunk_steps + a.chunk_steps, it.nsteps);
  const int32_t nquads = (it.npages + 3) / 4;
  uint8_t *mybuf = kbuf[wave];

  int32_t quad = it.chunk * a.chunk_steps + wave;
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

// Per-sequence work-item prefix of every path: item_off[path][S+1].
__global__ __launch_bounds__(256) void score_items_kernel(const int32_t *__restrict__ start,
                                                          const int32_t *__restrict__ len,
                                                          const int64_t *__restrict__ obs_off,
                                                          int32_t S, int32_t G, int32_t chunk_steps,
                                                          int32_t *__restrict__ item_off) {
  __shared__ int32_t carry[kPaths];
  __shared__ int32_t wsum[kPaths][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x < kPaths) carry[threadIdx.x] = 0;
  __syncthreads();
  for (int32_t base = 0; base < S; base += 256) {
    const int32_t i = base + threadIdx.x;
    int32_t c[kPaths] = {0, 0, 0, 0};
    if (i < S) {
      const int32_t npages = (start[i] + len[i] + kPage - 1) / kPage;
      const int32_t nsteps = (npages + kStepPages - 1) / kStepPages;
      const int32_t nch = (nsteps + chunk_steps - 1) / chunk_steps;
      const int32_t O = (int32_t)(obs_off[i + 1] - obs_off[i]);
      const int32_t R = O * G;
      const int path = path_of(O, R);
      const int32_t rpg = rows_per_group(path);
      const int32_t nrg = (R + rpg - 1) / rpg;
      c[path] = (len[i] > 0 && O > 0) ? nch * nrg : 0;
    }
    // inclusive wave scans
    int32_t x[kPaths];
#pragma unroll
    for (int q = 0; q < kPaths; ++q) x[q] = c[q];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
      for (int q = 0; q < kPaths; ++q) {
        const int32_t y = __shfl_up(x[q], d);
        if (lane >= d) x[q] += y;
      }
    }
    if (lane == 63)
#pragma unroll
      for (int q = 0; q < kPaths; ++q) wsum[q][wave] = x[q];
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPaths; ++q) {
      int32_t pre = carry[q];
      for (int w = 0; w < wave; ++w) pre += wsum[q][w];
      if (i < S) item_off[q * (S + 1) + i] = pre + x[q] - c[q];
      x[q] += pre;
    }
    __syncthreads();
    if (threadIdx.x == 255)
#pragma unroll
      for (int q = 0; q < kPaths; ++q) carry[q] = x[q];
    __syncthreads();
  }
  if (threadIdx.x < kPaths) item_off[threadIdx.x * (S + 1) + S] = carry[threadIdx.x];
}

struct Plan {
  int32_t chunk_steps;
  int64_t items[kPaths];   // per (layer, head)
  int32_t max_rg;
  bool any_partial;
  bool need_zero;
};

// Work items of sequence i on its path: (chunks of chunk_steps steps) x (row groups).
inline int64_t seq_items(int32_t start, int32_t len, int64_t O, int32_t G, int32_t chunk_steps) {
  if (len <= 0 || O <= 0) return 0;
  const int32_t npages = (start + len + kPage - 1) / kPage;
  const int32_t nsteps = (npages + kStepPages - 1) / kStepPages;
  const int32_t nch = (nsteps + chunk_steps - 1) / chunk_steps;
  const int32_t rpg = rows_per_group(path_of(O, O * G));
  const int32_t nrg = (int32_t)((O * G + rpg - 1) / rpg);
  return (int64_t)nch * nrg;
}

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
    const int32_t rpg = rows_per_group(path_of(O, O * G));
    const int32_t nrg = (int32_t)((O * G + rpg - 1) / rpg);
    // a 512-row item holds a workgroup of 8 waves, twice the 4-wave items
    total_steps += (int64_t)nsteps * nrg * (rpg == kWideRows ? 2 : 1);
    p.max_rg = nrg > p.max_rg ? nrg : p.max_rg;
  }
  p.need_zero = false;
  for (int i = 0; i < b.S; ++i) {
    const int64_t O = obs_off_h[i + 1] - obs_off_h[i];
    if (len_h[i] <= 0) continue;
    int32_t nrg = 0;
    if (O > 0) {
      const int32_t rpg = rows_per_group(path_of(O, O * G));
      nrg = (int32_t)((O * G + rpg - 1) / rpg);
    }
    if (O <= 0 || nrg < p.max_rg) p.need_zero = true;
  }
  total_steps *= (int64_t)b.L * b.Hkv;
  // aim for ~4 work items per resident 4-wave workgroup slot (256 CUs x 2)
  int64_t cs = total_steps / (256 * 2 * 4);
  if (cs < 4) cs = 4;
  if (cs > kMaxChunkSteps) cs = kMaxChunkSteps;
  p.chunk_steps = (int32_t)cs;
  for (int q = 0; q < kPaths; ++q) p.items[q] = 0;
  for (int i = 0; i < b.S; ++i) {
    const int64_t O = obs_off_h[i + 1] - obs_off_h[i];
    p.items[path_of(O, O * G)] += seq_items(start_h[i], len_h[i], O, G, p.chunk_steps);
  }
  p.any_partial = p.max_rg > 1;
  return p;
}

inline size_t table_bytes(int32_t S) {
  return ((kPaths * ((size_t)S + 1) * sizeof(int32_t)) + 255) & ~(size_t)255;
}

}  // namespace

size_t score_workspace_bytes(const Batch &b, int32_t Hq, const int64_t *obs_off_h,
                             const int32_t *len_h, const int32_t *start_h) {
  const int32_t G = Hq / b.Hkv;
  const Plan p = make_plan(b, G, obs_off_h, len_h, start_h);
  size_t bytes = 0;
  if (b.S > kSmallSeqs) bytes = table_bytes(b.S);
  if (p.any_partial) bytes += (size_t)p.max_rg * b.L * b.Hkv * b.E * sizeof(float);
  return bytes;
}

hipError_t launch_score(const kvs_cache &c, const Batch &b, const kvs_observers &o, float scale,
                        float *scores, void *ws, size_t ws_bytes, const int64_t *obs_off_h,
                        const int32_t *len_h, const int32_t *start_h, hipStream_t st) {
  (void)ws_bytes;
  const int32_t G = o.num_q_heads / b.Hkv;
  const Plan p = make_plan(b, G, obs_off_h, len_h, start_h);
  const int64_t LHE = (int64_t)b.L * b.Hkv * b.E;
  const bool small = b.S <= kSmallSeqs;
  int32_t *table = nullptr;
  size_t head = 0;
  if (!small) {
    table = (int32_t *)ws;
    head = table_bytes(b.S);
  }
  float *partial = p.any_partial ? (float *)((uint8_t *)ws + head) : nullptr;

  // Every live entry of a scored sequence is written by exactly one work item (or,
  // with several row groups, one per group).  Zero-fill is needed only for
  // sequences that are not scored, or that have fewer row groups than the batch.
  if (LHE > 0 && p.need_zero) {
    float *z = p.any_partial ? partial : scores;
    const int64_t nz = p.any_partial ? LHE * p.max_rg : LHE;
    zero_kernel<<<(unsigned)((nz + 255) / 256), 256, 0, st>>>(z, nz);
  }
  int64_t all_items = 0;
  for (int q = 0; q < kPaths; ++q) all_items += p.items[q];
  if (all_items == 0) return hipGetLastError();
  if (!small) score_items_kernel<<<1, 256, 0, st>>>(b.start, b.len, o.obs_off, b.S, G, p.chunk_steps, table);

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
  a.use_small = small ? 1 : 0;
  const int64_t LH = (int64_t)b.L * b.Hkv;
  // the widest items first, so that the long workgroups start early
  const int order[kPaths] = {kPathPipe8, kPathPipe4, kPathMfma, kPathValu};
  for (int oi = 0; oi < kPaths; ++oi) {
    const int path = order[oi];
    const int64_t items = p.items[path];
    if (items == 0) continue;
    if (small) {
      int32_t acc = 0;
      for (int i = 0; i < b.S; ++i) {
        a.small_off[i] = acc;
        const int64_t O = obs_off_h[i + 1] - obs_off_h[i];
        if (path_of(O, O * G) == path) acc += (int32_t)seq_items(start_h[i], len_h[i], O, G, p.chunk_steps);
      }
      a.small_off[b.S] = acc;
    } else {
      a.item_off = table + (size_t)path * (b.S + 1);
    }
    a.rows_per_group = rows_per_group(path);
    a.items_per_lg = (int32_t)items;
    a.total_items = items * LH;
    a.padded_items = (a.total_items + 7) & ~(int64_t)7;
    const unsigned grid = (unsigned)a.padded_items;
    switch (path) {
      case kPathPipe8: score_pipe_kernel<8><<<grid, PipeShape<8>::kThreads, 0, st>>>(a); break;
      case kPathPipe4: score_pipe_kernel<4><<<grid, PipeShape<4>::kThreads, 0, st>>>(a); break;
      case kPathMfma: score_mfma_kernel<<<grid, kThreads, 0, st>>>(a); break;
      default: score_valu_kernel<<<grid, kThreads, 0, st>>>(a); break;
    }
  }
  if (p.any_partial) {
    score_combine_kernel<<<(unsigned)((LHE + 255) / 256), 256, 0, st>>>(partial, scores, LHE, p.max_rg);
  }
  return hipGetLastError();
}

}  // namespace kvs
