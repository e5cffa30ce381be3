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
//   decode_split_kernel  one wave per (stream, split of 256 positions).  Per 64-key
//       tile: lane = key for the logits (its K row in VGPRs, v_dot2 with the query
//       rows, which are wave-uniform and come through scalar loads); online softmax
//       per row; then lane = pair of dimensions for P.V (each V row is one coalesced
//       256-byte load, the tile's probabilities are read from LDS).  Writes the split's
//       (max, sum, accumulator) per row, and the logits when a tally is requested.
//   decode_combine_kernel  merges a stream's splits per row: output and LSE.
//   decode_tally_kernel   s_j += sum_r exp(logit_rj - LSE_r) from the kept logits.
// All arithmetic is fp32 with base-2 exponentials (logits are kept as dot * scale * log2 e).
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kSplit = 256;                     // key positions per split (16 pages)
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

// Address (in elements) of the row of key position pos of stream (l, g).
__device__ __forceinline__ int64_t row_elem(const DecodeArgs &a, const int32_t *bt_row, int32_t l, int32_t g,
                                            int32_t pos) {
  const int64_t page = bt_row[pos >> 4];
  return ((((int64_t)l * a.b.num_pages + page) * a.b.Hkv + g) * kPage + (pos & 15)) * kHeadDim;
}

template <int RMAX>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  __shared__ float plds[RMAX][kTile];
  const int32_t s = blockIdx.x, i = blockIdx.y, lg = blockIdx.z;
  if (s >= seq_splits(a, i)) return;
  const int32_t l = lg / a.b.Hkv, g = lg - l * a.b.Hkv;
  const int lane = threadIdx.x;
  const int32_t start = a.b.start[i], n = a.b.len[i];
  const int64_t t0 = a.tok_off[i];
  const int32_t T = (int32_t)(a.tok_off[i + 1] - t0);
  const int32_t R = a.G * T;                   // <= RMAX (host checked)
  const int32_t *bt_row = a.b.bt + (int64_t)i * a.b.max_pages;
  const int32_t p0 = s * kSplit, p1 = min(p0 + kSplit, start + n);
  const float NEG = -__builtin_inff();

  float m[RMAX], lsum[RMAX], acc0[RMAX], acc1[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) { m[r] = NEG; lsum[r] = 0.f; acc0[r] = 0.f; acc1[r] = 0.f; }

  for (int32_t tp = p0; tp < p1; tp += kTile) {
    // ---- logits: lane = key ----
    const int32_t pos = tp + lane;
    const bool valid = pos >= start && pos < p1;
    const int32_t pc = valid ? pos : max(start, tp);      // clamped to a live position
    const uint4 *kr = (const uint4 *)(a.k + row_elem(a, bt_row, l, g, pc));
    bf16x2 kv[64];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint4 x = kr[c];
      const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[c * 4 + e] = __builtin_bit_cast(bf16x2, w4[e]);
    }
    float lg2[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      lg2[r] = NEG;
      if (r < R) {
        const int32_t h = g * a.G + r / T, t = r - (r / T) * T;
        const bf16x2 *qp = (const bf16x2 *)(a.q + (((int64_t)l * a.Hq + h) * a.t_total + t0 + t) * kHeadDim);
        float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
#pragma unroll
        for (int e = 0; e < 64; e += 4) {
          d0 = __builtin_amdgcn_fdot2_f32_bf16(qp[e], kv[e], d0, false);
          d1 = __builtin_amdgcn_fdot2_f32_bf16(qp[e + 1], kv[e + 1], d1, false);
          d2 = __builtin_amdgcn_fdot2_f32_bf16(qp[e + 2], kv[e + 2], d2, false);
          d3 = __builtin_amdgcn_fdot2_f32_bf16(qp[e + 3], kv[e + 3], d3, false);
        }
        lg2[r] = valid ? ((d0 + d1) + (d2 + d3)) * a.alpha : NEG;
        if (a.logits && valid)
          a.logits[((int64_t)lg * a.b.E + a.b.entry_off[i] + (pos - start)) * a.rmax + r] = lg2[r];
      }
    }
    // ---- online softmax per row; tile probabilities to LDS ----
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r < R) {
        const float mt = wave_max_f32(lg2[r]);
        const float mn = fmaxf(m[r], mt);                 // finite: the tile has a live key
        const float corr = m[r] == NEG ? 0.f : __builtin_amdgcn_exp2f(m[r] - mn);
        const float p = valid ? __builtin_amdgcn_exp2f(lg2[r] - mn) : 0.f;
        lsum[r] = lsum[r] * corr + wave_sum_f32(p);
        acc0[r] *= corr;
        acc1[r] *= corr;
        m[r] = mn;
        plds[r][lane] = p;
      }
    }
    // ---- P.V: lane = dimensions 2 lane, 2 lane + 1 ----
    const int32_t nk = min(kTile, p1 - tp);
    for (int32_t q = 0; q < nk; ++q) {
      const int32_t kp = tp + q;
      if (kp < start) continue;                           // wave-uniform
      const uint32_t vw = ((const uint32_t *)(a.v + row_elem(a, bt_row, l, g, kp)))[lane];
      const float v0 = __uint_as_float(vw << 16), v1 = __uint_as_float(vw & 0xFFFF0000u);
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        if (r < R) {
          const float p = plds[r][q];
          acc0[r] = __builtin_fmaf(p, v0, acc0[r]);
          acc1[r] = __builtin_fmaf(p, v1, acc1[r]);
        }
      }
    }
  }
  // ---- the split's partials ----
  const int64_t base = (int64_t)lg * a.part_off[a.b.S] + a.part_off[i] + (int64_t)s * R;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (r < R) {
      float *pp = a.part + (base + r) * kPartFloats;
      if (lane == 0) {
        pp[0] = m[r];
        pp[1] = lsum[r];
      }
      pp[2 + 2 * lane] = acc0[r];
      pp[3 + 2 * lane] = acc1[r];
    }
  }
}

// Merge the splits of one (stream, row): output = sum_s acc_s 2^(m_s - M) / sum_s l_s 2^(m_s - M),
// LSE = (M + log2 sum) ln 2.  One wave per (sequence, layer x KV head), rows in turn.
__global__ __launch_bounds__(64) void decode_combine_kernel(DecodeArgs a) {
  const int32_t i = blockIdx.x, lg = blockIdx.y;
  const int32_t ns = seq_splits(a, i);
  const int64_t t0 = a.tok_off[i];
  const int32_t T = (int32_t)(a.tok_off[i + 1] - t0);
  const int32_t R = a.G * T;
  const int32_t l = lg / a.b.Hkv, g = lg - l * a.b.Hkv;
  const int lane = threadIdx.x;
  const float NEG = -__builtin_inff();
  for (int32_t r = 0; r < R; ++r) {
    const int32_t h = g * a.G + r / T, t = r - (r / T) * T;
    const int64_t orow = ((int64_t)l * a.Hq + h) * a.t_total + t0 + t;
    float M = NEG;
    for (int32_t s = 0; s < ns; ++s)
      M = fmaxf(M, a.part[((int64_t)lg * a.part_off[a.b.S] + a.part_off[i] + (int64_t)s * R + r) * kPartFloats]);
    float L = 0.f, o0 = 0.f, o1 = 0.f;
    for (int32_t s = 0; s < ns; ++s) {
      const float *pp = a.part + ((int64_t)lg * a.part_off[a.b.S] + a.part_off[i] + (int64_t)s * R + r) * kPartFloats;
      const float ms = pp[0];
      const float f = ms == NEG ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      L = __builtin_fmaf(pp[1], f, L);
      o0 = __builtin_fmaf(pp[2 + 2 * lane], f, o0);
      o1 = __builtin_fmaf(pp[3 + 2 * lane], f, o1);
    }
    const bool any = ns > 0 && M != NEG;
    a.out[orow * kHeadDim + 2 * lane] = any ? o0 / L : 0.f;
    a.out[orow * kHeadDim + 2 * lane + 1] = any ? o1 / L : 0.f;
    if (lane == 0) a.lse[orow] = any ? (M + __builtin_amdgcn_logf(L)) * kLn2 : NEG;
  }
}

// s_j += sum_r 2^(logit2_rj - LSE_r log2 e) over the stream's rows.
__global__ __launch_bounds__(256) void decode_tally_kernel(DecodeArgs a) {
  const int32_t i = blockIdx.y, lg = blockIdx.z;
  const int32_t n = a.b.len[i];
  const int32_t j = blockIdx.x * 256 + threadIdx.x;
  if (j >= n) return;
  const int64_t t0 = a.tok_off[i];
  const int32_t T = (int32_t)(a.tok_off[i + 1] - t0);
  const int32_t R = a.G * T;
  if (R == 0) return;
  const int32_t l = lg / a.b.Hkv, g = lg - l * a.b.Hkv;
  const int64_t e = (int64_t)lg * a.b.E + a.b.entry_off[i] + j;
  float s = 0.f;
  for (int32_t r = 0; r < R; ++r) {
    const int32_t h = g * a.G + r / T, t = r - (r / T) * T;
    const float lse2 = a.lse[((int64_t)l * a.Hq + h) * a.t_total + t0 + t] * kLog2e;
    s += __builtin_amdgcn_exp2f(a.logits[e * a.rmax + r] - lse2);
  }
  a.scores[e] += s;
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
  decode_combine_kernel<<<dim3((unsigned)b.S, (unsigned)LH), 64, 0, st>>>(a);
  int32_t max_len = 0;
  for (int32_t i = 0; i < b.S; ++i) max_len = len_h[i] > max_len ? len_h[i] : max_len;
  if (scores && max_len > 0)
    decode_tally_kernel<<<dim3((unsigned)((max_len + 255) / 256), (unsigned)b.S, (unsigned)LH), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
