// kvs_token_confidence kernels: per decode step, the mean negative log-probability
// of the step's k most probable tokens.
//
// ActKV Dissected, Component 2: hesitation is read from the output distribution of
// each step through its top-20 tokens.  With z the step's logits over the
// vocabulary, p = softmax(z) and T the k largest logits,
//     conf = (1/k) sum_{j in T} -ln p_j = LSE(z) - mean_{j in T} z_j
//          = ln S + (1/k) sum_{j in T} (M - z_j),   M = max z,  S = sum_j exp(z_j - M).
//
// One workgroup takes a chunk of 32 768 logits of one row (64 per thread, held in
// VGPRs) and produces (M, S) and the chunk's k largest values; a row of a
// 128 256-token vocabulary is 4 chunks.  The chunk's top k come without a sort:
//   * the k-th largest of the 512 per-thread maxima, M_k, is found by a radix
//     search over order-preserving integer keys (4 passes of 8 bits);
//   * at least k values are >= M_k (one per thread whose maximum is >= M_k), and
//     values > M_k only occur in the at most k-1 threads whose maximum is > M_k,
//     so there are at most (k-1)*64 of them: they are compacted into LDS;
//   * if there are k or more, each is ranked among them (value, then position);
//     otherwise the rest of the top k are copies of M_k.
// A second kernel merges the chunks of a row: M = max M_c, S = sum S_c exp(M_c - M),
// and the top k of the chunks' top-k lists.  Reading and reduction orders are fixed,
// so results are deterministic.
#include "kvs_device.h"

namespace kvs {
namespace {

constexpr int kConfThreads = 512;
constexpr int kConfWaves = kConfThreads / 64;
constexpr int kConfPer = 64;                                 // logits per thread
constexpr int kConfChunk = kConfThreads * kConfPer;          // logits per workgroup
constexpr int kConfMaxK = 64;
constexpr int kCandCap = (kConfMaxK - 1) * kConfPer;         // values above M_k, at most
constexpr int kCombineThreads = 256;
constexpr int kConfMaxChunks = 32;                           // vocabularies up to 2^20
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct ConfArgs {
  const void *logits;
  int64_t rows;
  int64_t vocab;
  int64_t stride;    // elements between rows
  int32_t k;
  int32_t chunks;    // per row
  float *conf;       // [rows], written directly when chunks == 1
  float *part;       // [rows][chunks][2 + k]: M, S, then the chunk's top k values
};

// Order-preserving map of fp32 bit patterns to unsigned keys (NaN excluded).
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_f(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__device__ __forceinline__ float bf16_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ float wave_sum_f32(float x) {
  x += __shfl_xor(x, 32);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 8);
  x += __shfl_xor(x, 4);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 1);
  return x;
}

// Block sum of a float in wave order (deterministic).  scratch: one float per wave.
__device__ __forceinline__ float block_sum_f32(float x, float *scratch) {
  x = wave_sum_f32(x);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) scratch[wave] = x;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += scratch[w];
  __syncthreads();
  return t;
}

// The key of rank `need` (1 = largest) among one key per thread: radix search, 8 bits
// per pass, over a 256-bin LDS histogram.  Every thread must call it.
__device__ __forceinline__ uint32_t block_kth_key(uint32_t key, int need, uint32_t *hist, uint32_t *bcast) {
  uint32_t prefix = 0, mask = 0;
  const int lane = threadIdx.x & 63;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = threadIdx.x; b < 256; b += blockDim.x) hist[b] = 0;
    __syncthreads();
    if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l owns bins 4l .. 4l+3; count strictly above them, from the top
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      const uint32_t incl = wave_scan_u32(mine);
      const uint32_t total = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
      const uint32_t above = total - incl;       // keys in bins above lane l's four
      if (above < (uint32_t)need && (uint32_t)need <= above + mine) {
        uint32_t cum = above;
        int d = 4 * lane + 3;
        const uint32_t c[4] = {c0, c1, c2, c3};
        for (int b = 3; b >= 0; --b) {
          if (cum + c[b] >= (uint32_t)need) { d = 4 * lane + b; break; }
          cum += c[b];
        }
        bcast[0] = (uint32_t)d;
        bcast[1] = cum;
      }
    }
    __syncthreads();
    prefix |= bcast[0] << shift;
    mask |= 255u << shift;
    need -= (int)bcast[1];
    __syncthreads();
  }
  return prefix;
}

// One (row, chunk) per workgroup.  BF16: logits are bf16, else fp32.  VEC: rows are
// 16-byte aligned, so whole 16-byte vectors are loaded where they lie inside the row.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kConfThreads) void conf_chunk_kernel(ConfArgs a) {
  __shared__ float red[kConfWaves];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t bcast[2];
  __shared__ uint32_t ncand;
  __shared__ uint32_t cand[kCandCap];
  __shared__ float topv[kConfMaxK];

  const int64_t blk = blockIdx.x;
  const int64_t row = blk / a.chunks;
  const int32_t chunk = (int32_t)(blk - row * a.chunks);
  if (row >= a.rows) return;
  const int t = threadIdx.x;
  const int64_t c0 = (int64_t)chunk * kConfChunk;     // first logit of the chunk
  const int64_t rem = a.vocab - c0;                     // logits left in the row
  const int64_t nvalid = rem < kConfChunk ? rem : kConfChunk;
  const float NEG = -__builtin_inff();

  // ---- load 64 logits per thread; positions past the row end are -inf ----
  float x[kConfPer];
  if (BF16) {
    const uint16_t *src = (const uint16_t *)a.logits + row * a.stride + c0;
    if (VEC) {
      // vector u (of 8 logits) of thread t starts at logit (u * 512 + t) * 8
#pragma unroll
      for (int u = 0; u < kConfPer / 8; ++u) {
        const int64_t e = ((int64_t)u * kConfThreads + t) * 8;
        if (e + 8 <= nvalid) {
          const uint4 v = *(const uint4 *)(src + e);
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            x[u * 8 + 2 * q] = __uint_as_float(w[q] << 16);
            x[u * 8 + 2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) x[u * 8 + q] = (e + q < nvalid) ? bf16_f(src[e + q]) : NEG;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kConfPer; ++u) {
        const int64_t e = (int64_t)u * kConfThreads + t;
        x[u] = e < nvalid ? bf16_f(src[e]) : NEG;
      }
    }
  } else {
    const float *src = (const float *)a.logits + row * a.stride + c0;
    if (VEC) {
#pragma unroll
      for (int u = 0; u < kConfPer / 4; ++u) {
        const int64_t e = ((int64_t)u * kConfThreads + t) * 4;
        if (e + 4 <= nvalid) {
          const float4 v = *(const float4 *)(src + e);
          x[u * 4] = v.x;
          x[u * 4 + 1] = v.y;
          x[u * 4 + 2] = v.z;
          x[u * 4 + 3] = v.w;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) x[u * 4 + q] = (e + q < nvalid) ? src[e + q] : NEG;
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < kConfPer; ++u) {
        const int64_t e = (int64_t)u * kConfThreads + t;
        x[u] = e < nvalid ? src[e] : NEG;
      }
    }
  }

  // ---- maximum and sum of exp(z - M) ----
  float tmax = NEG;
#pragma unroll
  for (int u = 0; u < kConfPer; ++u) tmax = fmaxf(tmax, x[u]);
  // exp(z - tmax) as 2^((z - tmax) log2 e): the difference first, so that the rounding
  // of the exponent scales with |z - tmax| and not with |z|
  float tsum = 0.f;
  if (tmax != NEG) {
#pragma unroll
    for (int u = 0; u < kConfPer; ++u) tsum += __builtin_amdgcn_exp2f((x[u] - tmax) * kLog2e);
  }
  const uint32_t tkey = fkey(tmax);
  const float M = key_f(block_max_u32(tkey, (uint32_t *)red));
  const float S = block_sum_f32(tmax != NEG ? tsum * __builtin_amdgcn_exp2f((tmax - M) * kLog2e) : 0.f, red);

  // ---- the chunk's k largest values ----
  const int k = a.k;
  const uint32_t mk = block_kth_key(tkey, k, hist, bcast);
  if (t == 0) ncand = 0;
  __syncthreads();
  uint32_t cnt = 0;
#pragma unroll
  for (int u = 0; u < kConfPer; ++u) cnt += fkey(x[u]) > mk ? 1u : 0u;
  const uint32_t incl = wave_scan_u32(cnt);
  const uint32_t wtot = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
  uint32_t base = 0;
  if ((t & 63) == 63 && wtot) base = atomicAdd(&ncand, wtot);
  base = (uint32_t)__builtin_amdgcn_readlane((int)base, 63);
  if (cnt) {
    uint32_t pos = base + incl - cnt;
#pragma unroll
    for (int u = 0; u < kConfPer; ++u) {
      const uint32_t kx = fkey(x[u]);
      if (kx > mk) cand[pos++] = kx;      // pos < kCandCap: see the bound above
    }
  }
  __syncthreads();
  const int nc = (int)ncand;
  if (nc >= k) {
    // rank each candidate: larger keys first, then lower position
    for (int i = t; i < nc; i += kConfThreads) {
      const uint32_t ki = cand[i];
      int rank = 0;
      for (int j = 0; j < nc; ++j) {
        const uint32_t kj = cand[j];
        rank += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
      }
      if (rank < k) topv[rank] = key_f(ki);
    }
  } else {
    for (int i = t; i < k; i += kConfThreads) topv[i] = i < nc ? key_f(cand[i]) : key_f(mk);
  }
  __syncthreads();

  if (a.chunks == 1) {
    if (t < 64) {
      const float d = wave_sum_f32(t < k ? M - topv[t] : 0.f);
      if (t == 0) a.conf[row] = __builtin_amdgcn_logf(S) * kLn2 + d / (float)k;
    }
  } else {
    float *p = a.part + (row * a.chunks + chunk) * (int64_t)(2 + k);
    if (t == 0) {
      p[0] = M;
      p[1] = S;
    }
    if (t < k) p[2 + t] = topv[t];
  }
}

// Merge the chunks of one row (one workgroup per row).
__global__ __launch_bounds__(kCombineThreads) void conf_combine_kernel(ConfArgs a) {
  __shared__ float red[kCombineThreads / 64];
  __shared__ float topv[kConfMaxK];
  __shared__ uint32_t keys[kConfMaxChunks * kConfMaxK];
  const int64_t row = blockIdx.x;
  if (row >= a.rows) return;
  const int t = threadIdx.x;
  const int k = a.k;
  const int C = a.chunks;
  const int64_t w = 2 + k;
  const float *p = a.part + row * C * w;
  const float NEG = -__builtin_inff();
  // M over the chunks (every thread reads the C maxima)
  float M = NEG;
  for (int c = 0; c < C; ++c) M = fmaxf(M, p[c * w]);
  float s = 0.f;
  for (int c = t; c < C; c += kCombineThreads) {
    const float mc = p[c * w];
    s += mc != NEG ? p[c * w + 1] * __builtin_amdgcn_exp2f((mc - M) * kLog2e) : 0.f;
  }
  const float S = block_sum_f32(s, red);
  // the top k of the C*k chunk values, ranked by (value, position)
  const int n = C * k;
  for (int i = t; i < n; i += kCombineThreads) keys[i] = fkey(p[(i / k) * w + 2 + (i % k)]);
  __syncthreads();
  for (int i = t; i < n; i += kCombineThreads) {
    const uint32_t ki = keys[i];
    int rank = 0;
    for (int j = 0; j < n; ++j) {
      const uint32_t kj = keys[j];
      rank += (kj > ki || (kj == ki && j < i)) ? 1 : 0;
    }
    if (rank < k) topv[rank] = key_f(ki);
  }
  __syncthreads();
  if (t < 64) {
    const float d = wave_sum_f32(t < k ? M - topv[t] : 0.f);
    if (t == 0) a.conf[row] = __builtin_amdgcn_logf(S) * kLn2 + d / (float)k;
  }
}

}  // namespace

int64_t conf_max_vocab() { return (int64_t)kConfMaxChunks * kConfChunk; }
int32_t conf_max_k() { return kConfMaxK; }

int32_t conf_chunks(int64_t vocab) { return (int32_t)((vocab + kConfChunk - 1) / kConfChunk); }

size_t conf_workspace_bytes(int64_t rows, int64_t vocab, int32_t k) {
  const int32_t C = conf_chunks(vocab);
  if (C <= 1) return 0;
  return (size_t)rows * C * (2 + k) * sizeof(float);
}

hipError_t launch_confidence(const void *logits, bool bf16, int64_t rows, int64_t vocab, int64_t stride,
                             int32_t k, float *conf, void *ws, hipStream_t st) {
  ConfArgs a{};
  a.logits = logits;
  a.rows = rows;
  a.vocab = vocab;
  a.stride = stride;
  a.k = k;
  a.chunks = conf_chunks(vocab);
  a.conf = conf;
  a.part = (float *)ws;
  const size_t es = bf16 ? 2 : 4;
  const bool vec = ((uintptr_t)logits % 16 == 0) && ((size_t)stride * es) % 16 == 0;
  const unsigned blocks = (unsigned)(rows * a.chunks);
  if (bf16) {
    if (vec) conf_chunk_kernel<true, true><<<blocks, kConfThreads, 0, st>>>(a);
    else conf_chunk_kernel<true, false><<<blocks, kConfThreads, 0, st>>>(a);
  } else {
    if (vec) conf_chunk_kernel<false, true><<<blocks, kConfThreads, 0, st>>>(a);
    else conf_chunk_kernel<false, false><<<blocks, kConfThreads, 0, st>>>(a);
  }
  if (a.chunks > 1) conf_combine_kernel<<<(unsigned)rows, kCombineThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace kvs
