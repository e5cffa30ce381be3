// Internal declarations shared by the libkvs translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/kvs.h"

namespace kvs {

// Raises the dynamic-LDS limit of the n kernels in fns to `bytes`.  The attribute belongs
// to a device, so it is set once per device (the current one), under a lock; `done`
// holds one flag per device for this group of kernels.
inline hipError_t raise_lds_limit(const void *const *fns, int n, int bytes, bool (&done)[64]) {
  static std::mutex mu;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (done[dev]) return hipSuccess;
  for (int k = 0; k < n; ++k) {
    e = hipFuncSetAttribute(fns[k], hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
  }
  done[dev] = true;
  return hipSuccess;
}

constexpr int kHeadDim = 128;
constexpr int kPage = 16;
constexpr int kPageElems = kPage * kHeadDim;          // bf16 elements in one (layer, page, head) block
constexpr int64_t kMaxLen = int64_t(1) << 24;         // live entries per sequence
constexpr int kMfmaMinRows = 16;                      // MFMA scorer when observer rows R = O G >= 16

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((address_space(3))) void lds_void;

// Flattened batch description passed by value to every kernel.
struct Batch {
  const int32_t *bt;         // [S][max_pages]
  const int32_t *start;      // [S]
  const int32_t *len;        // [S]
  const int64_t *entry_off;  // [S+1]
  int64_t num_pages;
  int64_t E;                 // entries per (layer, head) row of per-entry arrays
  int32_t S;
  int32_t max_pages;
  int32_t L;
  int32_t Hkv;
};

// ---- launchers (defined in the .hip files, called by api.hip after validation) ----
hipError_t launch_score(const kvs_cache &c, const Batch &b, const kvs_observers &o, float scale,
                        float *scores, void *ws, size_t ws_bytes, const int64_t *obs_off_h,
                        const int32_t *len_h, const int32_t *start_h, hipStream_t st);
size_t score_workspace_bytes(const Batch &b, int32_t Hq, const int64_t *obs_off_h,
                             const int32_t *len_h, const int32_t *start_h);

hipError_t launch_lrfu(const kvs_cache &c, const Batch &b, const float *scores, uint32_t num,
                       uint32_t den, const float *decay, const int32_t *n_prev, uint8_t *hit,
                       int32_t max_len, hipStream_t st);

// keys (nullable): per-entry fp32 keys [L*Hkv][E] that take the CRF's place in the order.
hipError_t launch_select(const kvs_cache &c, const Batch &b, const float *scores,
                         const int32_t *budget, uint8_t *keep, int32_t max_len, hipStream_t st,
                         const float *keys = nullptr);

// Register-resident cut + LRFU and/or top-B for streams of at most 32768 entries.
// launch_stream_reg_plan: the fused cut, LRFU update and keep set, then the slot plan
// (pairs, pair counts) in the same workgroup.
hipError_t launch_stream_reg_plan(const kvs_cache &c, const Batch &b, const float *scores, uint32_t num,
                                  uint32_t den, const float *decay, const int32_t *n_prev, uint8_t *hit,
                                  const int32_t *budget, uint8_t *keep, int32_t *pairs, int32_t *pair_count,
                                  int64_t pair_cap, hipStream_t st);
bool stream_reg_fits(int32_t max_len, int64_t num_pages, int32_t Hkv);
hipError_t launch_stream_reg(const kvs_cache &c, const Batch &b, const float *scores, bool lrfu, bool select,
                             uint32_t num, uint32_t den, const float *decay, const int32_t *n_prev,
                             uint8_t *hit, const int32_t *budget, uint8_t *keep, hipStream_t st,
                             const float *keys = nullptr);

hipError_t launch_plan(const Batch &b, const uint8_t *keep, const int32_t *budget, int32_t *pairs,
                       int32_t *pair_count, int64_t pair_cap, hipStream_t st);


hipError_t launch_compact(const kvs_cache &c, const Batch &b, const int32_t *pairs,
                          const int32_t *pair_count, int64_t pair_cap, hipStream_t st);

// Paged decode attention with LSE and an optional attention tally.
int32_t decode_max_rows();
int64_t decode_max_positions();   // start + length of a sequence, at most
size_t decode_workspace_bytes(const Batch &b, int32_t G, const int64_t *tok_off_h, const int32_t *len_h,
                              const int32_t *start_h, bool tally, int32_t *rmax_out);
hipError_t launch_decode(const kvs_cache &c, const Batch &b, const kvs_observers &o, float scale, float *out,
                         float *lse, float *scores, void *ws, const int64_t *tok_off_h, const int32_t *len_h,
                         const int32_t *start_h, hipStream_t st);

// Step-aware ranking keys (StepKV): c_j = beta U_step(j) + (1 - beta) s_j into keys.
hipError_t launch_step_keys(const Batch &b, const float *scores, const int64_t *step_off, const int32_t *first,
                            int64_t num_steps, float beta, float *keys, float *utility, hipStream_t st);

// Beacon k-means: Lloyd iterations over P problems of N bf16 points (128 dims), K <= 16.
int32_t kmeans_max_k();
int32_t kmeans_max_points();
hipError_t launch_kmeans(const uint16_t *points, int64_t P, int32_t N, int32_t K, int32_t T, float *centroids,
                         int32_t *assign, uint16_t *beacons, hipStream_t st);
int32_t kmeans_seed_max_points();
hipError_t launch_kmeanspp(const uint16_t *points, int64_t P, int32_t N, int32_t K, const float *uniforms,
                           float *centroids, int32_t *rows, hipStream_t st);

// Token confidence (mean NLL of the k most probable tokens per logits row).
int64_t conf_max_vocab();
int32_t conf_max_k();
int32_t conf_chunks(int64_t vocab, bool bf16, int32_t k);
size_t conf_workspace_bytes(int64_t rows, int64_t vocab, int32_t k);
// kvs_token_confidence_static: the size of the library's per-device partial-result
// buffer, and its device address on the current device.
constexpr size_t kConfScratchBytes = (size_t)16 << 20;
hipError_t conf_scratch(void **out);
hipError_t launch_confidence(const void *logits, bool bf16, int64_t rows, int64_t vocab, int64_t stride,
                             int32_t k, float *conf, void *ws, hipStream_t st);

}  // namespace kvs
