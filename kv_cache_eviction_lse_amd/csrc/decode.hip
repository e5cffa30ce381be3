// kvs_decode_attention kernels: paged decode attention that emits each query row's
// log-sum-exp and, on request, adds the attention every cached entry receives into
// the eviction scores.
//
// ActKV Dissected, Component 3: the LSE is a byproduct of paged attention, and the
// attention a row puts on an entry is its logit minus the LSE, recovered per block
// without gathering or recomputing the attention matrix.  Component 1: an entry's
// signal is the attention it receives from the action tokens.  Here the decode pass
// itself keeps each block's logits (R floats per entry), so once the LSE is known the
// tally reads 4R bytes per entry instead of the 256-byte K row that kvs_score reads.
//
// Three kernels per call:
//   decode_split_kernel  one wave per (stream, split of 512 positions).  Per 64-key
//       tile: QK^T on 16x16x32 bf16 MFMAs (query rows on M, keys on N); online softmax
//       per row; then lane = pair of dimensions for P.V (each V row is one coalesced
//       256-byte load, the tile's probabilities are read from LDS).  Writes the split's
//       (max, sum, accumulator) per row, and the logits when a tally is requested.
//   decode_combine_kernel  merges a stream's splits per row: output and LSE.
//   decode_tally_kernel   s_j += sum_r exp(logit_rj - LSE_r) from the kept logits.
// All arithmetic is fp32 with base-2 exponentials (logits are kept as dot * scale * log2 e).
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kSplit = 512;                     // key positions per split (32 pages)
constexpr int kTile = 64;
constexpr int kPartFloats = 2 + kHeadDim;       // max, sum, accumulator
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct DecodeArgs {
  const uint16_t *k;
  const uint16_t *v;
  const uint16_t *q;          // bf16 [L][Hq][T_tot][128]
  const int64_t *tok_off;     // [S+1]
  float *out;                 // fp32 [L][Hq][T_tot][128]
  float *lse;                 // fp32 [L][Hq][T_tot]
  float *scores;              // fp32 [L][Hkv][E] (tally added) or null
  int64_t *part_off;          // [S+1] per-sequence base of (split, row) partials
  float *part;                // [L*Hkv][P_tot][130]
  float *logits;              // [L*Hkv][E][rmax] (tally only)
  Batch b;
  int64_t t_total;
  int32_t Hq;
  int32_t G;
  int32_t rmax;
  float alpha;                // scale * log2 e
};

__device__ __forceinline__ int32_t seq_splits(const DecodeArgs &a, int32_t i) {
  const int32_t n = a.b.len[i];
  const int64_t T = a.tok_off[i + 1] - a.tok_off[i];
  if (n <= 0 || T <= 0) return 0;
  return (a.b.start[i] + n + kSplit - 1) / kSplit;
}

// part_off[i] = sum over earlier sequences of splits * rows (one block).
__global__ __launch_bounds__(256) void decode_prefix_kernel(DecodeArgs a) {
  __shared__ int64_t wsum[4];
  __shared__ int64_t carry;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int32_t base = 0; base < a.b.S; base += 256) {
    const int32_t i = base + threadIdx.x;
    int64_t c = 0;
    if (i < a.b.S) c = (int64_t)seq_splits(a, i) * (a.G * (a.tok_off[i + 1] - a.tok_off[i]));
    const int64_t incl = wave_scan_u64((uint64_t)c);
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    int64_t before = carry;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    if (i < a.b.S) a.part_off[i] = before + incl - c;
    __syncthreads();
    if (threadIdx.x == 255) carry = before + incl;
    __syncthreads();
  }
  if (threadIdx.x == 0) a.part_off[a.b.S] = carry;
}

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum_f32(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

// LDS written by some lanes of a wave and then read by others: the wave's LDS
// operations complete in order, this keeps the compiler from reordering them.
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Maximum / sum over the 16 lanes of each 16-lane block (xor swizzles stay in the block).
__device__ __forceinline__ float block16_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (8 << 10) | 0x1F)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (4 << 10) | 0x1F)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (2 << 10) | 0x1F)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (1 << 10) | 0x1F)));
  return x;
}
__device__ __forceinline__ float block16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (8 << 10) | 0x1F));
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (4 << 10) | 0x1F));
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (2 << 10) | 0x1F));
  x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (1 << 10) | 0x1F));
  return x;
}

// One wave per (split, sequence, layer x KV head).  QK^T on v_mfma_f32_16x16x32_bf16
// with the query rows on M (padded to 16 with zero rows) and 16 keys on N: lane l
// loads 16 bytes of key l % 16 (dims 8 (l / 16) .. + 8 of each 32-dim slice), so one
// load instruction covers 64 contiguous bytes of 16 key rows, and ends up holding
// rows 4 (l / 16) .. + 4 of key l % 16.  The softmax state of those 4 rows is kept in
// each lane of the 16-lane block (identical across the block).  P.V runs with lane =
// pair of dimensions over the tile's V rows (coalesced 256-byte loads).
// Occupancy: 4 waves per SIMD for up to 4 rows (115 VGPRs), 2 for 8, 1 for 16.
template <int RMAX>
__global__ __launch_bounds__(64, RMAX <= 4 ? 4 : (RMAX <= 8 ? 2 : 1)) void decode_split_kernel(DecodeArgs a) {
  __shared__ float plds[16][kTile];
  __shared__ float corr_lds[16];
  const int32_t s = blockIdx.x, i = blockIdx.y, lg = blockIdx.z;
  if (s >= seq_splits(a, i)) return;
  const int32_t l = lg / a.b.Hkv, g = lg - l * a.b.Hkv;
  const int lane = threadIdx.x;
  const int blk = lane >> 4, n = lane & 15;
  const int32_t start = a.b.start[i], len = a.b.len[i];
  const int64_t t0 = a.tok_off[i];
  const int32_t T = (int32_t)(a.tok_off[i + 1] - t0);
  const int32_t R = a.G * T;                   // <= RMAX <= 16 (host checked)
  const int32_t *bt_row = a.b.bt + (int64_t)i * a.b.max_pages;
  const int32_t p0 = s * kSplit, p1 = min(p0 + kSplit, start + len);
  const float NEG = -__builtin_inff();

  // query rows as MFMA A operands: lane (m = lane % 16, 8-dim block lane / 16)
  bf16x8 qa[4];
  {
    const int m = n;
    const bool ok = m < R;
    const int32_t mc = ok ? m : 0;
    const int32_t h = g * a.G + mc / T, t = mc - (mc / T) * T;
    const uint16_t *qp = a.q + (((int64_t)l * a.Hq + h) * a.t_total + t0 + t) * kHeadDim + 8 * blk;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      const bf16x8 v = *(const bf16x8 *)(qp + 32 * sl);
      const bf16x8 z = {};
      qa[sl] = ok ? v : z;
    }
  }
  float mrun[4], lrun[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) { mrun[e] = NEG; lrun[e] = 0.f; }
  float acc0[RMAX], acc1[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) { acc0[r] = 0.f; acc1[r] = 0.f; }

  // Element offset of (l, physical page, g, row 0) for each of the split's (at most 32)
  // logical pages, lane p % 32 holding page p0 / 16 + p.  Every position visited lies in
  // [p0, p1), so its K and V rows are found with a lane exchange (K, per-lane
  // positions) or a lane read (V, one position per load) instead of a block-table load
  // that the row load would have to wait for.
  const int32_t pg0 = p0 >> 4, pg_last = (p1 - 1) >> 4;
  int64_t pbase;
  {
    const int32_t pg = pg0 + (lane & 31);
    const int64_t page = pg <= pg_last ? bt_row[pg] : 0;
    pbase = ((int64_t)l * a.b.num_pages + page) * a.b.Hkv * (kPage * kHeadDim) + (int64_t)g * (kPage * kHeadDim);
  }
  const int32_t pb_lo = (int32_t)(uint32_t)pbase, pb_hi = (int32_t)(pbase >> 32);
  auto page_base_of = [&](int32_t pos) {       // pos per lane, in [p0, p1)
    const int src = (pos >> 4) - pg0;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, pb_lo);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, pb_hi);
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  auto page_base_uniform = [&](int32_t pos) {  // pos the same in every lane, in [p0, p1)
    const int src = (pos >> 4) - pg0;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane(pb_lo, src);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane(pb_hi, src);
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };

  // tiles that lie wholly before the first live position are skipped, so every tile
  // visited holds a live key
  const int32_t tbeg = p0 + ((max(start, p0) - p0) / kTile) * kTile;
  for (int32_t tp = tbeg; tp < p1; tp += kTile) {
    // ---- logits of the tile's 64 keys (4 groups of 16) ----
    floatx4 d[4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int32_t pos = min(max(tp + 16 * kg + n, start), p1 - 1);
      const uint16_t *kr = a.k + page_base_of(pos) + (pos & 15) * kHeadDim + 8 * blk;
      d[kg] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < 4; ++sl)
        d[kg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[sl], *(const bf16x8 *)(kr + 32 * sl), d[kg], 0, 0, 0);
    }
    // ---- online softmax of rows 4 blk + e (state replicated over the 16 lanes) ----
    float x[4][4];
#pragma unroll
    for (int kg = 0; kg < 4; ++kg) {
      const int32_t pos = tp + 16 * kg + n;
      const bool valid = pos >= start && pos < p1;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[kg][e] = valid ? d[kg][e] * a.alpha : NEG;
      if (a.logits && valid) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * blk + e;
          if (r < R) a.logits[((int64_t)lg * a.b.E + a.b.entry_off[i] + (pos - start)) * a.rmax + r] = x[kg][e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float mt = block16_max(fmaxf(fmaxf(x[0][e], x[1][e]), fmaxf(x[2][e], x[3][e])));
      const float mn = fmaxf(mrun[e], mt);              // finite: the tile has a live key
      const float corr = mrun[e] == NEG ? 0.f : __builtin_amdgcn_exp2f(mrun[e] - mn);
      const float mref = mn == NEG ? 0.f : mn;
      float ps = 0.f;
#pragma unroll
      for (int kg = 0; kg < 4; ++kg) {
        const float p = __builtin_amdgcn_exp2f(x[kg][e] - mref);  // 0 for dead keys
        ps += p;
        plds[4 * blk + e][16 * kg + n] = p;
      }
      lrun[e] = lrun[e] * corr + block16_sum(ps);
      mrun[e] = mn;
      if (n == 0) corr_lds[4 * blk + e] = corr;
    }
    wave_lds_order();
    // ---- P.V: lane = dimensions 2 lane, 2 lane + 1 (same wave: LDS in order) ----
    uint32_t vw[kTile];
#pragma unroll
    for (int q = 0; q < kTile; ++q) {
      const int32_t kp = min(max(tp + q, start), p1 - 1);
      vw[q] = ((const uint32_t *)(a.v + page_base_uniform(kp) + (kp & 15) * kHeadDim))[lane];
    }
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r < R) {
        const float c = corr_lds[r];
        acc0[r] *= c;
        acc1[r] *= c;
      }
    }
#pragma unroll
    for (int q = 0; q < kTile; ++q) {
      const float v0 = __uint_as_float(vw[q] << 16), v1 = __uint_as_float(vw[q] & 0xFFFF0000u);
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        if (r < R) {
          const float p = plds[r][q];
          acc0[r] = __builtin_fmaf(p, v0, acc0[r]);
          acc1[r] = __builtin_fmaf(p, v1, acc1[r]);
        }
      }
    }
    wave_lds_order();
  }
  // ---- the split's partials ----
  const int64_t base = (int64_t)lg * a.part_off[a.b.S] + a.part_off[i] + (int64_t)s * R;
  if (n == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * blk + e;
      if (r < R) {
        float *pp = a.part + (base + r) * kPartFloats;
        pp[0] = mrun[e];
        pp[1] = lrun[e];
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (r < R) {
      float *pp = a.part + (base + r) * kPartFloats;
      pp[2 + 2 * lane] = acc0[r];
      pp[3 + 2 * lane] = acc1[r];
    }
  }
}

// Merge the splits of one (stream, row): output = sum_s acc_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),
// LSE = (M + log2 sum) ln 2.  One wave per (sequence, layer x KV head, row): lanes take
// the splits for M and the sum (their weights go to LDS), then lane = pair of dimensions
// for the accumulators, 8 splits in flight.
constexpr int kMaxSplits = 8192;
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float f_lds[kMaxSplits];
  const int32_t i = blockIdx.x, lg = blockIdx.y, r = blockIdx.z;
  const int64_t t0 = a.tok_off[i];
  const int32_t T = (int32_t)(a.tok_off[i + 1] - t0);
  const int32_t R = a.G * T;
  if (r >= R) return;
  const int32_t ns = seq_splits(a, i);
  const int32_t l = lg / a.b.Hkv, g = lg - l * a.b.Hkv;
  const int lane = threadIdx.x;
  const float NEG = -__builtin_inff();
  const int32_t h = g * a.G + r / T, t = r - (r / T) * T;
  const int64_t orow = ((int64_t)l * a.Hq + h) * a.t_total + t0 + t;
  const float *pb = a.part + ((int64_t)lg * a.part_off[a.b.S] + a.part_off[i] + r) * kPartFloats;
  const int64_t sstride = (int64_t)R * kPartFloats;        // from split s to s + 1
  float M = NEG;
  for (int32_t s = lane; s < ns; s += 64) M = fmaxf(M, pb[s * sstride]);
  M = wave_max_f32(M);
  float Ls = 0.f;
  for (int32_t s = lane; s < ns; s += 64) {
    const float ms = pb[s * sstride];
    const float f = ms == NEG ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    f_lds[s] = f;
    Ls = __builtin_fmaf(pb[s * sstride + 1], f, Ls);
  }
  const float L = wave_sum_f32(Ls);
  float o0 = 0.f, o1 = 0.f;
  int32_t s = 0;
  for (; s + 8 <= ns; s += 8) {
    float2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *(const float2 *)(pb + (s + u) * sstride + 2 + 2 * lane);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float f = f_lds[s + u];
      o0 = __builtin_fmaf(v[u].x, f, o0);
      o1 = __builtin_fmaf(v[u].y, f, o1);
    }
  }
  for (; s < ns; ++s) {
    const float2 v = *(const float2 *)(pb + s * sstride + 2 + 2 * lane);
    const float f = f_lds[s];
    o0 = __builtin_fmaf(v.x, f, o0);
    o1 = __builtin_fmaf(v.y, f, o1);
  }
  const bool any = ns > 0 && M != NEG;
  *(float2 *)(a.out + orow * kHeadDim + 2 * lane) = any ? float2{o0 / L, o1 / L} : float2{0.f, 0.f};
  if (lane == 0) a.lse[orow] = any ? (M + __builtin_amdgcn_logf(L)) * kLn2 : NEG;
}

// s_j += sum_r 2^(logit2_rj - LSE_r log2 e) over the stream's rows.  256 threads, four
// entries per thread (256 apart); the rows' LSEs are loaded once per block, the logits
// of an entry as float4s when the row count per entry is a multiple of 4.
constexpr int kTallyPer = 4;
template <int RMAX>
__global__ __launch_bounds__(256) void decode_tally_kernel(DecodeArgs a) {
  const int32_t i = blockIdx.y, lg = blockIdx.z;
  const int32_t n = a.b.len[i];
  const int32_t j0 = blockIdx.x * (256 * kTallyPer) + threadIdx.x;
  if (blockIdx.x * (256 * kTallyPer) >= n) return;
  const int64_t t0 = a.tok_off[i];
  const int32_t T = (int32_t)(a.tok_off[i + 1] - t0);
  const int32_t R = a.G * T;                   // <= RMAX (host checked)
  if (R == 0) return;
  const int32_t l = lg / a.b.Hkv, g = lg - l * a.b.Hkv;
  float lse2[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    lse2[r] = __builtin_inff();                  // rows beyond R contribute 2^(-inf) = 0
    if (r < R) {
      const int32_t h = g * a.G + r / T, t = r - (r / T) * T;
      lse2[r] = a.lse[((int64_t)l * a.Hq + h) * a.t_total + t0 + t] * kLog2e;
    }
  }
  const int64_t ebase = (int64_t)lg * a.b.E + a.b.entry_off[i];
  float x[kTallyPer][RMAX];
#pragma unroll
  for (int u = 0; u < kTallyPer; ++u) {
    const int32_t j = min(j0 + 256 * u, n - 1);
    const float *lp = a.logits + (ebase + j) * a.rmax;
    if (a.rmax % 4 == 0) {
#pragma unroll
      for (int r4 = 0; r4 < RMAX; r4 += 4) {
        float4 v = {0.f, 0.f, 0.f, 0.f};
        if (r4 < R) v = *(const float4 *)(lp + r4);
        // logits of rows beyond this sequence's R were never written
        x[u][r4] = v.x;
        x[u][r4 + 1] = r4 + 1 < R ? v.y : 0.f;
        x[u][r4 + 2] = r4 + 2 < R ? v.z : 0.f;
        x[u][r4 + 3] = r4 + 3 < R ? v.w : 0.f;
      }
    } else {
#pragma unroll
      for (int r = 0; r < RMAX; ++r) x[u][r] = r < R ? lp[r] : 0.f;
    }
  }
#pragma unroll
  for (int u = 0; u < kTallyPer; ++u) {
    const int32_t j = j0 + 256 * u;
    float sum = 0.f;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) sum += __builtin_amdgcn_exp2f(x[u][r] - lse2[r]);
    if (j < n) a.scores[ebase + j] += sum;
  }
}

}  // namespace

size_t decode_workspace_bytes(const Batch &b, int32_t G, const int64_t *tok_off_h, const int32_t *len_h,
                              const int32_t *start_h, bool tally, int32_t *rmax_out) {
  int64_t parts = 0;
  int32_t rmax = 0;
  for (int32_t i = 0; i < b.S; ++i) {
    const int64_t T = tok_off_h[i + 1] - tok_off_h[i];
    const int32_t R = (int32_t)(G * T);
    rmax = R > rmax ? R : rmax;
    if (len_h[i] <= 0 || T <= 0) continue;
    parts += (int64_t)((start_h[i] + len_h[i] + kSplit - 1) / kSplit) * R;
  }
  if (rmax_out) *rmax_out = rmax;
  size_t bytes = (((size_t)b.S + 1) * sizeof(int64_t) + 255) & ~(size_t)255;
  bytes += (((size_t)b.L * b.Hkv * parts * kPartFloats * sizeof(float)) + 255) & ~(size_t)255;
  if (tally) bytes += (size_t)b.L * b.Hkv * b.E * rmax * sizeof(float);
  return bytes;
}

int32_t decode_max_rows() { return 16; }
int64_t decode_max_positions() { return (int64_t)kMaxSplits * kSplit; }

hipError_t launch_decode(const kvs_cache &c, const Batch &b, const kvs_observers &o, float scale, float *out,
                         float *lse, float *scores, void *ws, const int64_t *tok_off_h, const int32_t *len_h,
                         const int32_t *start_h, hipStream_t st) {
  const int32_t G = o.num_q_heads / b.Hkv;
  int32_t rmax = 0;
  (void)decode_workspace_bytes(b, G, tok_off_h, len_h, start_h, scores != nullptr, &rmax);
  int32_t max_splits = 0;
  for (int32_t i = 0; i < b.S; ++i) {
    if (len_h[i] <= 0 || tok_off_h[i + 1] <= tok_off_h[i]) continue;
    const int32_t ns = (start_h[i] + len_h[i] + kSplit - 1) / kSplit;
    max_splits = ns > max_splits ? ns : max_splits;
  }
  DecodeArgs a{};
  a.k = (const uint16_t *)c.k;
  a.v = (const uint16_t *)c.v;
  a.q = (const uint16_t *)o.q;
  a.tok_off = o.obs_off;
  a.out = out;
  a.lse = lse;
  a.scores = scores;
  uint8_t *w = (uint8_t *)ws;
  a.part_off = (int64_t *)w;
  w += (((size_t)b.S + 1) * sizeof(int64_t) + 255) & ~(size_t)255;
  a.part = (float *)w;
  int64_t parts = 0;
  for (int32_t i = 0; i < b.S; ++i) {
    const int64_t T = tok_off_h[i + 1] - tok_off_h[i];
    if (len_h[i] <= 0 || T <= 0) continue;
    parts += (int64_t)((start_h[i] + len_h[i] + kSplit - 1) / kSplit) * G * T;
  }
  w += (((size_t)b.L * b.Hkv * parts * kPartFloats * sizeof(float)) + 255) & ~(size_t)255;
  a.logits = scores ? (float *)w : nullptr;
  a.b = b;
  a.t_total = o.obs_total;
  a.Hq = o.num_q_heads;
  a.G = G;
  a.rmax = rmax > 0 ? rmax : 1;
  a.alpha = scale * kLog2e;
  const int32_t LH = b.L * b.Hkv;
  decode_prefix_kernel<<<1, 256, 0, st>>>(a);
  if (max_splits > 0) {
    const dim3 grid((unsigned)max_splits, (unsigned)b.S, (unsigned)LH);
    if (rmax <= 4) decode_split_kernel<4><<<grid, 64, 0, st>>>(a);
    else if (rmax <= 8) decode_split_kernel<8><<<grid, 64, 0, st>>>(a);
    else decode_split_kernel<16><<<grid, 64, 0, st>>>(a);
  }
  decode_combine_kernel<<<dim3((unsigned)b.S, (unsigned)LH, (unsigned)(rmax > 0 ? rmax : 1)), 64, 0, st>>>(a);
  int32_t max_len = 0;
  for (int32_t i = 0; i < b.S; ++i) max_len = len_h[i] > max_len ? len_h[i] : max_len;
  if (scores && max_len > 0) {
    const dim3 tg((unsigned)((max_len + 256 * kTallyPer - 1) / (256 * kTallyPer)), (unsigned)b.S, (unsigned)LH);
    if (rmax <= 4) decode_tally_kernel<4><<<tg, 256, 0, st>>>(a);
    else if (rmax <= 8) decode_tally_kernel<8><<<tg, 256, 0, st>>>(a);
    else decode_tally_kernel<16><<<tg, 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace kvs
