// libkvs C ABI: host-side validation, launch planning and the host-only outputs.
// Every entry point checks its arguments before any HIP call; on error it enqueues
// nothing and returns a status (detail in kvs_last_error()).
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "kvs_internal.h"

namespace {

thread_local char g_err[512] = "";

kvs_status fail(kvs_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

kvs_status ok() {
  g_err[0] = 0;
  return KVS_OK;
}

kvs_status check_cache(const kvs_cache *c, bool need_kv, bool need_crf) {
  if (!c) return fail(KVS_ERR_NULL, "cache is NULL");
  if (c->head_dim != kvs::kHeadDim) return fail(KVS_ERR_UNSUPPORTED, "head_dim %d != 128", c->head_dim);
  if (c->page_size != kvs::kPage) return fail(KVS_ERR_UNSUPPORTED, "page_size %d != 16", c->page_size);
  if (c->num_layers <= 0 || c->num_kv_heads <= 0 || c->num_pages <= 0)
    return fail(KVS_ERR_SHAPE, "num_layers, num_kv_heads and num_pages must be > 0");
  if (c->num_pages > (int64_t(1) << 31))
    return fail(KVS_ERR_UNSUPPORTED, "num_pages %lld exceeds 2^31", (long long)c->num_pages);
  if (need_kv && (!c->k || !c->v)) return fail(KVS_ERR_NULL, "cache k/v is NULL");
  if (need_crf && !c->crf) return fail(KVS_ERR_NULL, "cache crf is NULL");
  return KVS_OK;
}

// Checks the batch against the pool; optionally that no physical page is used twice
// (required by the calls that write the pools in place).
kvs_status check_seqs(const kvs_seqs *s, int64_t num_pages, bool unique_pages) {
  if (!s) return fail(KVS_ERR_NULL, "seqs is NULL");
  if (s->num_seqs < 0 || s->max_pages < 0) return fail(KVS_ERR_SHAPE, "num_seqs/max_pages < 0");
  if (s->num_seqs == 0) return KVS_OK;
  if (!s->block_table || !s->block_table_h || !s->start || !s->start_h || !s->len || !s->len_h ||
      !s->entry_off || !s->entry_off_h)
    return fail(KVS_ERR_NULL, "a seqs array is NULL");
  if (s->entry_off_h[0] < 0) return fail(KVS_ERR_SHAPE, "entry_off[0] < 0");
  std::vector<uint8_t> used;
  if (unique_pages) used.assign((size_t)num_pages, 0);
  for (int32_t i = 0; i < s->num_seqs; ++i) {
    const int32_t st = s->start_h[i], n = s->len_h[i];
    if (st < 0 || st >= kvs::kPage) return fail(KVS_ERR_SHAPE, "start[%d] = %d not in [0, 16)", i, st);
    if (n < 0 || n > kvs::kMaxLen) return fail(KVS_ERR_SHAPE, "len[%d] = %d out of range", i, n);
    if (s->entry_off_h[i + 1] - s->entry_off_h[i] != n)
      return fail(KVS_ERR_SHAPE, "entry_off[%d+1] - entry_off[%d] != len[%d]", i, i, i);
    const int64_t npg = n == 0 ? 0 : (st + (int64_t)n + kvs::kPage - 1) / kvs::kPage;
    if (npg > s->max_pages) return fail(KVS_ERR_SHAPE, "sequence %d needs %lld pages > max_pages", i, (long long)npg);
    const int32_t *row = s->block_table_h + (int64_t)i * s->max_pages;
    for (int64_t p = 0; p < npg; ++p) {
      const int32_t pg = row[p];
      if (pg < 0 || pg >= num_pages)
        return fail(KVS_ERR_SHAPE, "block_table[%d][%lld] = %d outside the pool", i, (long long)p, pg);
      if (unique_pages) {
        if (used[pg]) return fail(KVS_ERR_SHAPE, "page %d is used twice (in-place update needs distinct pages)", pg);
        used[pg] = 1;
      }
    }
  }
  return KVS_OK;
}

kvs::Batch make_batch(const kvs_cache *c, const kvs_seqs *s) {
  kvs::Batch b{};
  b.bt = s->block_table;
  b.start = s->start;
  b.len = s->len;
  b.entry_off = s->entry_off;
  b.num_pages = c->num_pages;
  b.E = s->num_seqs ? s->entry_off_h[s->num_seqs] : 0;
  b.S = s->num_seqs;
  b.max_pages = s->max_pages;
  b.L = c->num_layers;
  b.Hkv = c->num_kv_heads;
  return b;
}

int32_t max_len_of(const kvs_seqs *s) {
  int32_t m = 0;
  for (int32_t i = 0; i < s->num_seqs; ++i) m = s->len_h[i] > m ? s->len_h[i] : m;
  return m;
}

kvs_status check_obs(const kvs_observers *o, const kvs_seqs *s, int32_t Hkv) {
  if (!o) return fail(KVS_ERR_NULL, "observers is NULL");
  if (o->num_q_heads <= 0 || o->num_q_heads % Hkv != 0)
    return fail(KVS_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d", o->num_q_heads, Hkv);
  if (o->num_q_heads / Hkv > 64) return fail(KVS_ERR_UNSUPPORTED, "GQA group larger than 64");
  if (o->obs_total < 0) return fail(KVS_ERR_SHAPE, "obs_total < 0");
  if (s->num_seqs == 0) return KVS_OK;
  if (!o->obs_off || !o->obs_off_h) return fail(KVS_ERR_NULL, "obs_off is NULL");
  if (o->obs_off_h[0] < 0) return fail(KVS_ERR_SHAPE, "obs_off[0] < 0");
  for (int32_t i = 0; i < s->num_seqs; ++i) {
    const int64_t O = o->obs_off_h[i + 1] - o->obs_off_h[i];
    if (O < 0) return fail(KVS_ERR_SHAPE, "obs_off not monotone at %d", i);
    if (O > 65536) return fail(KVS_ERR_UNSUPPORTED, "sequence %d has %lld observers (max 65536)", i, (long long)O);
  }
  if (o->obs_off_h[s->num_seqs] > o->obs_total) return fail(KVS_ERR_SHAPE, "obs_off exceeds obs_total");
  if (o->obs_off_h[s->num_seqs] > o->obs_off_h[0] && (!o->q || !o->lse))
    return fail(KVS_ERR_NULL, "q/lse is NULL");
  return KVS_OK;
}

int64_t pair_cap_of(const kvs_seqs *s, const int32_t *budget_h) {
  int64_t P = 0;
  for (int32_t i = 0; i < s->num_seqs; ++i) {
    const int32_t n = s->len_h[i];
    const int32_t b = budget_h[i];
    const int32_t K = b < n ? b : n;
    const int64_t c = (n - K) < K ? (n - K) : K;
    P = c > P ? c : P;
  }
  return P;
}

kvs_status hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(KVS_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
}

}  // namespace

extern "C" {

const char *kvs_status_string(kvs_status s) {
  switch (s) {
    case KVS_OK: return "KVS_OK";
    case KVS_ERR_NULL: return "KVS_ERR_NULL";
    case KVS_ERR_SHAPE: return "KVS_ERR_SHAPE";
    case KVS_ERR_UNSUPPORTED: return "KVS_ERR_UNSUPPORTED";
    case KVS_ERR_WORKSPACE: return "KVS_ERR_WORKSPACE";
    case KVS_ERR_HIP: return "KVS_ERR_HIP";
  }
  return "KVS_ERR_UNKNOWN";
}

const char *kvs_last_error(void) { return g_err; }

const char *kvs_version(void) { return "kvs 0.1.0 (gfx950)"; }

size_t kvs_score_workspace_size(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_observers *obs) {
  if (check_cache(cache, false, false) != KVS_OK) return 0;
  if (check_seqs(seqs, cache->num_pages, false) != KVS_OK) return 0;
  if (check_obs(obs, seqs, cache->num_kv_heads) != KVS_OK) return 0;
  if (seqs->num_seqs == 0) return 0;
  const kvs::Batch b = make_batch(cache, seqs);
  ok();
  if (b.E == 0) return 0;
  return kvs::score_workspace_bytes(b, obs->num_q_heads, obs->obs_off_h, seqs->len_h, seqs->start_h);
}

kvs_status kvs_score(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_observers *obs, float scale,
                     float *scores, void *workspace, size_t workspace_bytes, void *stream) {
  kvs_status st;
  if ((st = check_cache(cache, true, false)) != KVS_OK) return st;
  if ((st = check_seqs(seqs, cache->num_pages, false)) != KVS_OK) return st;
  if ((st = check_obs(obs, seqs, cache->num_kv_heads)) != KVS_OK) return st;
  if (!std::isfinite(scale)) return fail(KVS_ERR_SHAPE, "scale is not finite");
  if (seqs->num_seqs == 0) return ok();
  const kvs::Batch b = make_batch(cache, seqs);
  if (b.E == 0) return ok();
  if (!scores) return fail(KVS_ERR_NULL, "scores is NULL");
  const size_t need = kvs::score_workspace_bytes(b, obs->num_q_heads, obs->obs_off_h, seqs->len_h, seqs->start_h);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KVS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  return hip_status(kvs::launch_score(*cache, b, *obs, scale, scores, workspace, workspace_bytes,
                                      obs->obs_off_h, seqs->len_h, seqs->start_h, (hipStream_t)stream));
}

float kvs_lrfu_decay(double lambda, int32_t dt) { return (float)std::exp2(-lambda * (double)dt); }

kvs_status kvs_lrfu_update(const kvs_cache *cache, const kvs_seqs *seqs, const float *scores, uint32_t mass_num,
                           uint32_t mass_den, const float *decay, const int32_t *n_prev, uint8_t *hit,
                           void *stream) {
  kvs_status st;
  if ((st = check_cache(cache, false, true)) != KVS_OK) return st;
  if ((st = check_seqs(seqs, cache->num_pages, true)) != KVS_OK) return st;
  if (mass_den == 0 || mass_num > mass_den)
    return fail(KVS_ERR_SHAPE, "mass fraction %u/%u must satisfy 0 <= num <= den, den > 0", mass_num, mass_den);
  if (seqs->num_seqs == 0) return ok();
  const kvs::Batch b = make_batch(cache, seqs);
  if (b.E == 0) return ok();
  if (!scores || !decay || !n_prev) return fail(KVS_ERR_NULL, "scores/decay/n_prev is NULL");
  const int32_t max_len = max_len_of(seqs);
  if (kvs::stream_reg_fits(max_len, cache->num_pages, cache->num_kv_heads))
    return hip_status(kvs::launch_stream_reg(*cache, b, scores, true, false, mass_num, mass_den, decay, n_prev, hit,
                                             nullptr, nullptr, (hipStream_t)stream));
  return hip_status(kvs::launch_lrfu(*cache, b, scores, mass_num, mass_den, decay, n_prev, hit, max_len,
                                     (hipStream_t)stream));
}

kvs_status kvs_select(const kvs_cache *cache, const kvs_seqs *seqs, const float *scores, const int32_t *budget,
                      const int32_t *budget_h, uint8_t *keep, void *stream) {
  kvs_status st;
  if ((st = check_cache(cache, false, true)) != KVS_OK) return st;
  if ((st = check_seqs(seqs, cache->num_pages, false)) != KVS_OK) return st;
  if (seqs->num_seqs == 0) return ok();
  if (!budget || !budget_h) return fail(KVS_ERR_NULL, "budget is NULL");
  for (int32_t i = 0; i < seqs->num_seqs; ++i)
    if (budget_h[i] < 0) return fail(KVS_ERR_SHAPE, "budget[%d] = %d < 0", i, budget_h[i]);
  const kvs::Batch b = make_batch(cache, seqs);
  if (b.E == 0) return ok();
  if (!scores || !keep) return fail(KVS_ERR_NULL, "scores/keep is NULL");
  const int32_t max_len = max_len_of(seqs);
  if (kvs::stream_reg_fits(max_len, cache->num_pages, cache->num_kv_heads))
    return hip_status(kvs::launch_stream_reg(*cache, b, scores, false, true, 0, 1, nullptr, nullptr, nullptr,
                                             budget, keep, (hipStream_t)stream));
  return hip_status(kvs::launch_select(*cache, b, scores, budget, keep, max_len, (hipStream_t)stream));
}

namespace {

// Step boundaries: step_off[0] = 0, non-decreasing; per sequence with steps,
// first[step_off[i]] = 0 <= first[...] non-decreasing <= len[i]; a sequence with live
// entries has at least one step.
kvs_status check_steps(const kvs_steps *t, const kvs_seqs *s) {
  if (!t) return fail(KVS_ERR_NULL, "steps is NULL");
  if (!t->step_off || !t->step_off_h) return fail(KVS_ERR_NULL, "step_off is NULL");
  if (t->step_off_h[0] != 0) return fail(KVS_ERR_SHAPE, "step_off[0] != 0");
  const int64_t M = t->step_off_h[s->num_seqs];
  if (M > (int64_t(1) << 31)) return fail(KVS_ERR_UNSUPPORTED, "%lld steps (max 2^31)", (long long)M);
  if (M > 0 && (!t->first || !t->first_h)) return fail(KVS_ERR_NULL, "first is NULL");
  for (int32_t i = 0; i < s->num_seqs; ++i) {
    const int64_t k0 = t->step_off_h[i], k1 = t->step_off_h[i + 1];
    if (k1 < k0) return fail(KVS_ERR_SHAPE, "step_off not monotone at %d", i);
    const int32_t n = s->len_h[i];
    if (k1 == k0) {
      if (n > 0) return fail(KVS_ERR_SHAPE, "sequence %d has live entries but no step", i);
      continue;
    }
    if (t->first_h[k0] != 0) return fail(KVS_ERR_SHAPE, "the first step of sequence %d does not start at slot 0", i);
    for (int64_t k = k0 + 1; k < k1; ++k)
      if (t->first_h[k] < t->first_h[k - 1] || t->first_h[k] > n)
        return fail(KVS_ERR_SHAPE, "step %lld of sequence %d starts at %d: not in [%d, %d]", (long long)(k - k0), i,
                    t->first_h[k], t->first_h[k - 1], n);
  }
  return KVS_OK;
}

}  // namespace

namespace {

// The combined keys of every entry, fp32 [L][Hkv][E].
size_t step_ws_bytes(const kvs::Batch &b) { return (size_t)b.L * b.Hkv * (size_t)b.E * sizeof(float); }

}  // namespace

size_t kvs_step_select_workspace_size(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_steps *steps) {
  if (check_cache(cache, false, false) != KVS_OK) return 0;
  if (check_seqs(seqs, cache->num_pages, false) != KVS_OK) return 0;
  if (seqs->num_seqs == 0) return 0;
  if (check_steps(steps, seqs) != KVS_OK) return 0;
  const kvs::Batch b = make_batch(cache, seqs);
  ok();
  return step_ws_bytes(b);
}

kvs_status kvs_step_select(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_steps *steps,
                           const float *scores, float beta, const int32_t *budget, const int32_t *budget_h,
                           uint8_t *keep, float *utility, void *workspace, size_t workspace_bytes,
                           void *stream) {
  kvs_status st;
  if ((st = check_cache(cache, false, false)) != KVS_OK) return st;
  if ((st = check_seqs(seqs, cache->num_pages, false)) != KVS_OK) return st;
  if (!(beta >= 0.f && beta <= 1.f)) return fail(KVS_ERR_SHAPE, "beta = %g not in [0, 1]", (double)beta);
  if ((int64_t)cache->num_layers * cache->num_kv_heads > 65535)
    return fail(KVS_ERR_UNSUPPORTED, "num_layers x num_kv_heads exceeds 65535");
  if (seqs->num_seqs == 0) return ok();
  if ((st = check_steps(steps, seqs)) != KVS_OK) return st;
  if (!budget || !budget_h) return fail(KVS_ERR_NULL, "budget is NULL");
  for (int32_t i = 0; i < seqs->num_seqs; ++i)
    if (budget_h[i] < 0) return fail(KVS_ERR_SHAPE, "budget[%d] = %d < 0", i, budget_h[i]);
  const kvs::Batch b = make_batch(cache, seqs);
  if (b.E == 0) return ok();
  if (!scores || !keep) return fail(KVS_ERR_NULL, "scores/keep is NULL");
  const size_t need = step_ws_bytes(b);
  if (!workspace || workspace_bytes < need)
    return fail(KVS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  const hipStream_t hs = (hipStream_t)stream;
  float *keys = (float *)workspace;
  hipError_t e = kvs::launch_step_keys(b, scores, steps->step_off, steps->first, steps->step_off_h[seqs->num_seqs],
                                       beta, keys, utility, hs);
  if (e != hipSuccess) return hip_status(e);
  const int32_t max_len = max_len_of(seqs);
  if (kvs::stream_reg_fits(max_len, cache->num_pages, cache->num_kv_heads))
    return hip_status(kvs::launch_stream_reg(*cache, b, scores, false, true, 0, 1, nullptr, nullptr, nullptr,
                                             budget, keep, hs, keys));
  return hip_status(kvs::launch_select(*cache, b, scores, budget, keep, max_len, hs, keys));
}

kvs_status kvs_beacon_seed(const void *points, int64_t num_problems, int32_t num_points, int32_t k,
                           const float *uniforms, float *centroids, int32_t *rows, void *stream) {
  if (num_problems < 0 || num_problems > INT32_MAX)
    return fail(KVS_ERR_SHAPE, "num_problems = %lld not in [0, 2^31)", (long long)num_problems);
  if (num_points < 1) return fail(KVS_ERR_SHAPE, "num_points = %d < 1", num_points);
  if (num_points > kvs::kmeans_seed_max_points())
    return fail(KVS_ERR_UNSUPPORTED, "num_points = %d > %d", num_points, kvs::kmeans_seed_max_points());
  if (k < 1 || k > kvs::kmeans_max_k())
    return fail(KVS_ERR_UNSUPPORTED, "k = %d not in [1, %d]", k, kvs::kmeans_max_k());
  if (num_problems == 0) return ok();
  if (!points || !uniforms || !centroids) return fail(KVS_ERR_NULL, "points/uniforms/centroids is NULL");
  return hip_status(kvs::launch_kmeanspp((const uint16_t *)points, num_problems, num_points, k, uniforms, centroids,
                                         rows, (hipStream_t)stream));
}

kvs_status kvs_beacon_kmeans(const void *points, int64_t num_problems, int32_t num_points, int32_t k, int32_t iters,
                             float *centroids, int32_t *assign, void *beacons, void *stream) {
  if (num_problems < 0 || num_problems > INT32_MAX)
    return fail(KVS_ERR_SHAPE, "num_problems = %lld not in [0, 2^31)", (long long)num_problems);
  if (num_points < 1) return fail(KVS_ERR_SHAPE, "num_points = %d < 1", num_points);
  if (k < 1 || k > kvs::kmeans_max_k())
    return fail(KVS_ERR_UNSUPPORTED, "k = %d not in [1, %d]", k, kvs::kmeans_max_k());
  if (num_points > kvs::kmeans_max_points())
    return fail(KVS_ERR_UNSUPPORTED, "num_points = %d > %d", num_points, kvs::kmeans_max_points());
  if (iters < 0) return fail(KVS_ERR_SHAPE, "iters = %d < 0", iters);
  if (num_problems == 0) return ok();
  if (!points || !centroids) return fail(KVS_ERR_NULL, "points/centroids is NULL");
  return hip_status(kvs::launch_kmeans((const uint16_t *)points, num_problems, num_points, k, iters, centroids,
                                       assign, (uint16_t *)beacons, (hipStream_t)stream));
}

kvs_status kvs_lrfu_select(const kvs_cache *cache, const kvs_seqs *seqs, const float *scores, uint32_t mass_num,
                           uint32_t mass_den, const float *decay, const int32_t *n_prev, uint8_t *hit,
                           const int32_t *budget, const int32_t *budget_h, uint8_t *keep, void *stream) {
  kvs_status st;
  if ((st = check_cache(cache, false, true)) != KVS_OK) return st;
  if ((st = check_seqs(seqs, cache->num_pages, true)) != KVS_OK) return st;
  if (mass_den == 0 || mass_num > mass_den)
    return fail(KVS_ERR_SHAPE, "mass fraction %u/%u must satisfy 0 <= num <= den, den > 0", mass_num, mass_den);
  if (seqs->num_seqs == 0) return ok();
  if (!budget || !budget_h) return fail(KVS_ERR_NULL, "budget is NULL");
  for (int32_t i = 0; i < seqs->num_seqs; ++i)
    if (budget_h[i] < 0) return fail(KVS_ERR_SHAPE, "budget[%d] = %d < 0", i, budget_h[i]);
  const kvs::Batch b = make_batch(cache, seqs);
  if (b.E == 0) return ok();
  if (!scores || !decay || !n_prev || !keep) return fail(KVS_ERR_NULL, "scores/decay/n_prev/keep is NULL");
  const int32_t max_len = max_len_of(seqs);
  if (kvs::stream_reg_fits(max_len, cache->num_pages, cache->num_kv_heads))
    return hip_status(kvs::launch_stream_reg(*cache, b, scores, true, true, mass_num, mass_den, decay, n_prev, hit,
                                             budget, keep, (hipStream_t)stream));
  hipError_t e = kvs::launch_lrfu(*cache, b, scores, mass_num, mass_den, decay, n_prev, hit, max_len,
                                  (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(kvs::launch_select(*cache, b, scores, budget, keep, max_len, (hipStream_t)stream));
}

int64_t kvs_pair_capacity(const kvs_seqs *seqs, const int32_t *budget_h) {
  if (!seqs) { fail(KVS_ERR_NULL, "seqs is NULL"); return -1; }
  if (seqs->num_seqs < 0) { fail(KVS_ERR_SHAPE, "num_seqs < 0"); return -1; }
  if (seqs->num_seqs == 0) { ok(); return 0; }
  if (!seqs->len_h || !budget_h) { fail(KVS_ERR_NULL, "len_h/budget_h is NULL"); return -1; }
  for (int32_t i = 0; i < seqs->num_seqs; ++i)
    if (budget_h[i] < 0 || seqs->len_h[i] < 0) { fail(KVS_ERR_SHAPE, "negative budget or length"); return -1; }
  ok();
  return pair_cap_of(seqs, budget_h);
}

kvs_status kvs_plan_host(const kvs_seqs *seqs, const int32_t *budget_h, int32_t *shift_h, int32_t *new_start_h,
                         int32_t *new_len_h, int32_t *freed_h, int64_t freed_capacity, int64_t *freed_count_h) {
  kvs_status st;
  if ((st = check_seqs(seqs, (int64_t(1) << 31), false)) != KVS_OK) return st;
  if (seqs->num_seqs > 0 && !budget_h) return fail(KVS_ERR_NULL, "budget_h is NULL");
  for (int32_t i = 0; i < seqs->num_seqs; ++i)
    if (budget_h[i] < 0) return fail(KVS_ERR_SHAPE, "budget[%d] = %d < 0", i, budget_h[i]);
  int64_t nfreed = 0;
  for (int32_t i = 0; i < seqs->num_seqs; ++i) {
    const int32_t n = seqs->len_h[i];
    const int32_t K = budget_h[i] < n ? budget_h[i] : n;
    nfreed += (seqs->start_h[i] + n - K) / kvs::kPage;
  }
  if (freed_h && nfreed > freed_capacity)
    return fail(KVS_ERR_SHAPE, "freed capacity %lld < %lld freed pages", (long long)freed_capacity, (long long)nfreed);
  int64_t w = 0;
  for (int32_t i = 0; i < seqs->num_seqs; ++i) {
    const int32_t n = seqs->len_h[i];
    const int32_t K = budget_h[i] < n ? budget_h[i] : n;
    const int32_t D = n - K;
    const int32_t shift = (seqs->start_h[i] + D) / kvs::kPage;
    if (shift_h) shift_h[i] = shift;
    if (new_start_h) new_start_h[i] = (seqs->start_h[i] + D) % kvs::kPage;
    if (new_len_h) new_len_h[i] = K;
    if (freed_h)
      for (int32_t p = 0; p < shift; ++p) freed_h[w++] = seqs->block_table_h[(int64_t)i * seqs->max_pages + p];
  }
  if (freed_count_h) *freed_count_h = nfreed;
  return ok();
}

kvs_status kvs_plan(const kvs_seqs *seqs, int32_t num_layers, int32_t num_kv_heads, const uint8_t *keep,
                    const int32_t *budget, const int32_t *budget_h, int32_t *pairs, int32_t *pair_count,
                    int32_t *shift_h, int32_t *new_start_h, int32_t *new_len_h, int32_t *freed_h,
                    int64_t freed_capacity, int64_t *freed_count_h, void *stream) {
  if (!seqs) return fail(KVS_ERR_NULL, "seqs is NULL");
  if (num_layers <= 0 || num_kv_heads <= 0) return fail(KVS_ERR_SHAPE, "num_layers/num_kv_heads must be > 0");
  kvs_status st;
  // page ids are not touched by the plan: check the structure only (pool size unknown here)
  if ((st = check_seqs(seqs, (int64_t(1) << 31), false)) != KVS_OK) return st;
  if (seqs->num_seqs > 0 && (!budget || !budget_h)) return fail(KVS_ERR_NULL, "budget is NULL");
  for (int32_t i = 0; i < seqs->num_seqs; ++i)
    if (budget_h[i] < 0) return fail(KVS_ERR_SHAPE, "budget[%d] = %d < 0", i, budget_h[i]);
  const int64_t P = seqs->num_seqs ? pair_cap_of(seqs, budget_h) : 0;
  if (seqs->num_seqs > 0 && (!keep || !pair_count || (P > 0 && !pairs)))
    return fail(KVS_ERR_NULL, "keep/pairs/pair_count is NULL");
  if ((st = kvs_plan_host(seqs, budget_h, shift_h, new_start_h, new_len_h, freed_h, freed_capacity,
                          freed_count_h)) != KVS_OK)
    return st;
  if (seqs->num_seqs == 0) return ok();
  kvs_cache dummy{};
  dummy.num_layers = num_layers;
  dummy.num_kv_heads = num_kv_heads;
  dummy.num_pages = 1;
  const kvs::Batch b = make_batch(&dummy, seqs);
  return hip_status(kvs::launch_plan(b, keep, budget, pairs, pair_count, P, (hipStream_t)stream));
}

kvs_status kvs_compact(const kvs_cache *cache, const kvs_seqs *seqs, const int32_t *budget_h, const int32_t *pairs,
                       const int32_t *pair_count, void *stream) {
  kvs_status st;
  if ((st = check_cache(cache, true, true)) != KVS_OK) return st;
  if ((st = check_seqs(seqs, cache->num_pages, true)) != KVS_OK) return st;
  if (seqs->num_seqs == 0) return ok();
  if (!budget_h) return fail(KVS_ERR_NULL, "budget_h is NULL");
  for (int32_t i = 0; i < seqs->num_seqs; ++i)
    if (budget_h[i] < 0) return fail(KVS_ERR_SHAPE, "budget[%d] = %d < 0", i, budget_h[i]);
  const int64_t P = pair_cap_of(seqs, budget_h);
  if (P == 0) return ok();
  if (!pairs || !pair_count) return fail(KVS_ERR_NULL, "pairs/pair_count is NULL");
  const kvs::Batch b = make_batch(cache, seqs);
  return hip_status(kvs::launch_compact(*cache, b, pairs, pair_count, P, (hipStream_t)stream));
}

kvs_status kvs_plan_compact(const kvs_cache *cache, const kvs_seqs *seqs, const uint8_t *keep, const int32_t *budget,
                            const int32_t *budget_h, int32_t *pairs, int32_t *pair_count, int32_t *shift_h,
                            int32_t *new_start_h, int32_t *new_len_h, int32_t *freed_h, int64_t freed_capacity,
                            int64_t *freed_count_h, void *stream) {
  kvs_status st;
  if ((st = check_cache(cache, true, true)) != KVS_OK) return st;
  if ((st = check_seqs(seqs, cache->num_pages, true)) != KVS_OK) return st;
  if (seqs->num_seqs > 0 && (!budget || !budget_h)) return fail(KVS_ERR_NULL, "budget is NULL");
  for (int32_t i = 0; i < seqs->num_seqs; ++i)
    if (budget_h[i] < 0) return fail(KVS_ERR_SHAPE, "budget[%d] = %d < 0", i, budget_h[i]);
  const int64_t P = seqs->num_seqs ? pair_cap_of(seqs, budget_h) : 0;
  if (seqs->num_seqs > 0 && (!keep || !pair_count || (P > 0 && !pairs)))
    return fail(KVS_ERR_NULL, "keep/pairs/pair_count is NULL");
  if ((st = kvs_plan_host(seqs, budget_h, shift_h, new_start_h, new_len_h, freed_h, freed_capacity,
                          freed_count_h)) != KVS_OK)
    return st;
  if (seqs->num_seqs == 0) return ok();
  const kvs::Batch b = make_batch(cache, seqs);
  hipError_t e = kvs::launch_plan(b, keep, budget, pairs, pair_count, P, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e);
  if (P == 0) return ok();
  return hip_status(kvs::launch_compact(*cache, b, pairs, pair_count, P, (hipStream_t)stream));
}

kvs_status kvs_lrfu_select_compact(const kvs_cache *cache, const kvs_seqs *seqs, const float *scores,
                                   uint32_t mass_num, uint32_t mass_den, const float *decay, const int32_t *n_prev,
                                   uint8_t *hit, const int32_t *budget, const int32_t *budget_h, uint8_t *keep,
                                   int32_t *pairs, int32_t *pair_count, int32_t *shift_h, int32_t *new_start_h,
                                   int32_t *new_len_h, int32_t *freed_h, int64_t freed_capacity,
                                   int64_t *freed_count_h, void *stream) {
  kvs_status st;
  if ((st = check_cache(cache, true, true)) != KVS_OK) return st;
  if ((st = check_seqs(seqs, cache->num_pages, true)) != KVS_OK) return st;
  if (mass_den == 0 || mass_num > mass_den)
    return fail(KVS_ERR_SHAPE, "mass fraction %u/%u must satisfy 0 <= num <= den, den > 0", mass_num, mass_den);
  if (seqs->num_seqs > 0 && (!budget || !budget_h)) return fail(KVS_ERR_NULL, "budget is NULL");
  for (int32_t i = 0; i < seqs->num_seqs; ++i)
    if (budget_h[i] < 0) return fail(KVS_ERR_SHAPE, "budget[%d] = %d < 0", i, budget_h[i]);
  const int64_t P = seqs->num_seqs ? pair_cap_of(seqs, budget_h) : 0;
  if (seqs->num_seqs > 0 && (!keep || !pair_count || (P > 0 && !pairs)))
    return fail(KVS_ERR_NULL, "keep/pairs/pair_count is NULL");
  if ((st = kvs_plan_host(seqs, budget_h, shift_h, new_start_h, new_len_h, freed_h, freed_capacity,
                          freed_count_h)) != KVS_OK)
    return st;
  if (seqs->num_seqs == 0) return ok();
  const kvs::Batch b = make_batch(cache, seqs);
  if (b.E > 0 && (!scores || !decay || !n_prev)) return fail(KVS_ERR_NULL, "scores/decay/n_prev is NULL");
  if (b.E > 0 && kvs::stream_reg_fits(max_len_of(seqs), cache->num_pages, cache->num_kv_heads)) {
    // selection and slot plan in one kernel, then the moves
    hipError_t e = kvs::launch_stream_reg_plan(*cache, b, scores, mass_num, mass_den, decay, n_prev, hit, budget,
                                               keep, pairs, pair_count, P, (hipStream_t)stream);
    if (e != hipSuccess || P == 0) return hip_status(e);
    return hip_status(kvs::launch_compact(*cache, b, pairs, pair_count, P, (hipStream_t)stream));
  }
  // otherwise the two calls in turn (the host outputs are already written)
  if ((st = kvs_lrfu_select(cache, seqs, scores, mass_num, mass_den, decay, n_prev, hit, budget, budget_h, keep,
                            stream)) != KVS_OK)
    return st;
  return kvs_plan_compact(cache, seqs, keep, budget, budget_h, pairs, pair_count, nullptr, nullptr, nullptr,
                          nullptr, 0, nullptr, stream);
}

kvs_status kvs_budget_ratchet(int32_t *budget_h, const uint8_t *flag_h, int32_t num_seqs, int32_t num, int32_t den,
                              int32_t cap) {
  if (num_seqs < 0) return fail(KVS_ERR_SHAPE, "num_seqs < 0");
  if (num_seqs == 0) return ok();
  if (!budget_h || !flag_h) return fail(KVS_ERR_NULL, "budget_h/flag_h is NULL");
  if (den <= 0 || num < den || cap < 0) return fail(KVS_ERR_SHAPE, "ratchet needs num >= den > 0 and cap >= 0");
  for (int32_t i = 0; i < num_seqs; ++i) {
    if (!flag_h[i]) continue;
    const int64_t b = budget_h[i];
    int64_t grown = b * num / den;
    if (grown > cap) grown = cap;
    budget_h[i] = (int32_t)(grown > b ? grown : b);
  }
  return ok();
}

}  // extern "C"

// ---- decode attention ----

namespace {

// Decode queries reuse the observer structure (q, obs_off as token offsets,
// num_q_heads, obs_total); its lse field is not read.
kvs_status check_decode(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_observers *o) {
  kvs_status st;
  if ((st = check_cache(cache, true, false)) != KVS_OK) return st;
  if ((st = check_seqs(seqs, cache->num_pages, false)) != KVS_OK) return st;
  if (!o) return fail(KVS_ERR_NULL, "queries is NULL");
  const int32_t Hkv = cache->num_kv_heads;
  if (o->num_q_heads <= 0 || o->num_q_heads % Hkv != 0)
    return fail(KVS_ERR_SHAPE, "num_q_heads %d is not a positive multiple of num_kv_heads %d", o->num_q_heads, Hkv);
  const int32_t G = o->num_q_heads / Hkv;
  if (o->obs_total < 0) return fail(KVS_ERR_SHAPE, "token total < 0");
  if (seqs->num_seqs == 0) return KVS_OK;
  if (!o->obs_off || !o->obs_off_h) return fail(KVS_ERR_NULL, "token offsets are NULL");
  if (o->obs_off_h[0] < 0) return fail(KVS_ERR_SHAPE, "token offset[0] < 0");
  for (int32_t i = 0; i < seqs->num_seqs; ++i) {
    const int64_t T = o->obs_off_h[i + 1] - o->obs_off_h[i];
    if (T < 0) return fail(KVS_ERR_SHAPE, "token offsets not monotone at %d", i);
    if ((int64_t)G * T > kvs::decode_max_rows())
      return fail(KVS_ERR_UNSUPPORTED, "sequence %d has %lld query rows per KV head (max %d)", i,
                  (long long)(G * T), kvs::decode_max_rows());
    if ((int64_t)seqs->start_h[i] + seqs->len_h[i] > kvs::decode_max_positions())
      return fail(KVS_ERR_UNSUPPORTED, "sequence %d ends at position %lld (max %lld)", i,
                  (long long)seqs->start_h[i] + seqs->len_h[i], (long long)kvs::decode_max_positions());
  }
  if (o->obs_off_h[seqs->num_seqs] > o->obs_total) return fail(KVS_ERR_SHAPE, "token offsets exceed the total");
  if (o->obs_off_h[seqs->num_seqs] > o->obs_off_h[0] && !o->q) return fail(KVS_ERR_NULL, "q is NULL");
  return KVS_OK;
}

}  // namespace

extern "C" {

size_t kvs_decode_workspace_size(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_observers *queries,
                                 int32_t tally) {
  if (check_decode(cache, seqs, queries) != KVS_OK) return 0;
  if (seqs->num_seqs == 0) return 0;
  const kvs::Batch b = make_batch(cache, seqs);
  return kvs::decode_workspace_bytes(b, queries->num_q_heads / cache->num_kv_heads, queries->obs_off_h,
                                     seqs->len_h, seqs->start_h, tally != 0, nullptr);
}

kvs_status kvs_decode_attention(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_observers *queries,
                                float scale, float *out, float *lse, float *scores, void *workspace,
                                size_t workspace_bytes, void *stream) {
  kvs_status st;
  if ((st = check_decode(cache, seqs, queries)) != KVS_OK) return st;
  if (!std::isfinite(scale)) return fail(KVS_ERR_SHAPE, "scale is not finite");
  if (seqs->num_seqs == 0 || queries->obs_off_h[seqs->num_seqs] == queries->obs_off_h[0]) return ok();
  if (!out || !lse) return fail(KVS_ERR_NULL, "out/lse is NULL");
  const kvs::Batch b = make_batch(cache, seqs);
  const size_t need = kvs::decode_workspace_bytes(b, queries->num_q_heads / cache->num_kv_heads,
                                                  queries->obs_off_h, seqs->len_h, seqs->start_h,
                                                  scores != nullptr, nullptr);
  if (!workspace || workspace_bytes < need)
    return fail(KVS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  return hip_status(kvs::launch_decode(*cache, b, *queries, scale, out, lse, scores, workspace,
                                       queries->obs_off_h, seqs->len_h, seqs->start_h, (hipStream_t)stream));
}

}  // extern "C"

// ---- confidence monitor ----

namespace {

kvs_status check_confidence(int32_t dtype, int64_t rows, int64_t vocab, int64_t row_stride, int32_t k) {
  if (dtype != KVS_DTYPE_F32 && dtype != KVS_DTYPE_BF16) return fail(KVS_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (rows < 0) return fail(KVS_ERR_SHAPE, "rows < 0");
  if (vocab <= 0 || vocab > kvs::conf_max_vocab())
    return fail(vocab <= 0 ? KVS_ERR_SHAPE : KVS_ERR_UNSUPPORTED, "vocab %lld not in [1, %lld]", (long long)vocab,
                (long long)kvs::conf_max_vocab());
  if (k < 1 || k > kvs::conf_max_k()) return fail(KVS_ERR_UNSUPPORTED, "k %d not in [1, %d]", k, kvs::conf_max_k());
  if (k > vocab) return fail(KVS_ERR_SHAPE, "k %d > vocab %lld", k, (long long)vocab);
  if (row_stride < vocab) return fail(KVS_ERR_SHAPE, "row_stride %lld < vocab", (long long)row_stride);
  if (rows * (int64_t)kvs::conf_chunks(vocab, false, k) > ((int64_t)1 << 40))
    return fail(KVS_ERR_UNSUPPORTED, "rows x chunks exceeds the grid limit");
  return KVS_OK;
}

}  // namespace

extern "C" {

size_t kvs_token_confidence_workspace_size(int64_t rows, int64_t vocab, int32_t k) {
  if (check_confidence(KVS_DTYPE_F32, rows, vocab, vocab, k) != KVS_OK) return 0;
  return kvs::conf_workspace_bytes(rows, vocab, k);
}

kvs_status kvs_token_confidence(const void *logits, int32_t dtype, int64_t rows, int64_t vocab, int64_t row_stride,
                                int32_t k, float *conf, void *workspace, size_t workspace_bytes, void *stream) {
  kvs_status st;
  if ((st = check_confidence(dtype, rows, vocab, row_stride, k)) != KVS_OK) return st;
  if (rows == 0) return ok();
  if (!logits || !conf) return fail(KVS_ERR_NULL, "logits/conf is NULL");
  const size_t need = kvs::conf_workspace_bytes(rows, vocab, k);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KVS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  return hip_status(kvs::launch_confidence(logits, dtype == KVS_DTYPE_BF16, rows, vocab, row_stride, k, conf,
                                           workspace, (hipStream_t)stream));
}

kvs_status kvs_token_confidence_static(const void *logits, int32_t dtype, int64_t rows, int64_t vocab,
                                       int64_t row_stride, int32_t k, float *conf, void *stream) {
  kvs_status st;
  if ((st = check_confidence(dtype, rows, vocab, row_stride, k)) != KVS_OK) return st;
  if (rows == 0) return ok();
  if (!logits || !conf) return fail(KVS_ERR_NULL, "logits/conf is NULL");
  const size_t need = kvs::conf_workspace_bytes(rows, vocab, k);
  if (need > kvs::kConfScratchBytes)
    return fail(KVS_ERR_UNSUPPORTED, "partial results need %zu bytes > the %zu-byte static buffer", need,
                kvs::kConfScratchBytes);
  void *ws = nullptr;
  if (need > 0) {
    const hipError_t e = kvs::conf_scratch(&ws);
    if (e != hipSuccess) return hip_status(e);
  }
  return hip_status(kvs::launch_confidence(logits, dtype == KVS_DTYPE_BF16, rows, vocab, row_stride, k, conf,
                                           ws, (hipStream_t)stream));
}

kvs_status kvs_confidence_trend(const float *conf_h, int64_t n, int32_t window, int32_t stride, int64_t fit_last,
                                double *pooled_h, int64_t *pooled_count_h, double *slope_h, int32_t *flag_h) {
  if (n < 0 || window < 1 || stride < 1 || fit_last < 0)
    return fail(KVS_ERR_SHAPE, "need n >= 0, window >= 1, stride >= 1, fit_last >= 0");
  if (n > 0 && !conf_h) return fail(KVS_ERR_NULL, "conf_h is NULL");
  if (!flag_h) return fail(KVS_ERR_NULL, "flag_h is NULL");
  const int64_t P = n >= window ? (n - window) / stride + 1 : 0;
  if (pooled_count_h) *pooled_count_h = P;
  // minimum of each full window, windows starting every `stride` values
  std::vector<double> pooled((size_t)P);
  for (int64_t w = 0; w < P; ++w) {
    double m = (double)conf_h[w * stride];
    for (int64_t j = 1; j < window; ++j) m = std::fmin(m, (double)conf_h[w * stride + j]);
    pooled[(size_t)w] = m;
  }
  if (pooled_h)
    for (int64_t w = 0; w < P; ++w) pooled_h[w] = pooled[(size_t)w];
  // least-squares slope against the window index over the last fit_last values (0 = all)
  const int64_t first = (fit_last > 0 && fit_last < P) ? P - fit_last : 0;
  const int64_t m = P - first;
  *flag_h = 0;
  if (slope_h) *slope_h = std::nan("");
  if (m < 2) return ok();
  double xb = 0.0, yb = 0.0;
  for (int64_t i = 0; i < m; ++i) {
    xb += (double)i;
    yb += pooled[(size_t)(first + i)];
  }
  xb /= (double)m;
  yb /= (double)m;
  double sxy = 0.0, sxx = 0.0;
  for (int64_t i = 0; i < m; ++i) {
    const double dx = (double)i - xb;
    sxy += dx * (pooled[(size_t)(first + i)] - yb);
    sxx += dx * dx;
  }
  const double slope = sxy / sxx;
  if (slope_h) *slope_h = slope;
  *flag_h = slope < 0.0 ? 1 : 0;
  return ok();
}

}  // extern "C"

// ---- one eviction round, pipelined over layer chunks ----
namespace {

// Per device: a non-blocking side stream at the default priority and a pool of events,
// created once and reused (an event may be recorded again once the waits on its previous
// record are enqueued).  The mutex is held while a round is enqueued.
struct RoundRes {
  hipStream_t side = nullptr;
  std::vector<hipEvent_t> ev;
};
std::mutex g_round_mu;
std::vector<RoundRes> g_round_res;

hipError_t round_resources(int32_t n_events, RoundRes **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((size_t)dev >= g_round_res.size()) g_round_res.resize((size_t)dev + 1);
  RoundRes &r = g_round_res[dev];
  if (!r.side && (e = hipStreamCreateWithFlags(&r.side, hipStreamNonBlocking)) != hipSuccess) return e;
  while ((int32_t)r.ev.size() < n_events) {
    hipEvent_t x = nullptr;
    if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess) return e;
    r.ev.push_back(x);
  }
  *out = &r;
  return hipSuccess;
}

// Every per-layer array has the layer outermost, so layers [l0, l0 + n) of the batch
// are a contiguous sub-array of each: the same kernels run on a chunk through offset
// pointers and num_layers = n.
struct RoundArgs {
  kvs_cache cache;
  kvs_observers obs;
  float scale;
  uint32_t mass_num, mass_den;
  const float *decay;
  const int32_t *n_prev, *budget;
  float *scores;
  uint8_t *hit, *keep;
  int32_t *pairs, *pair_count;
  int64_t pair_cap;
  int32_t max_len;
  void *ws;
  size_t ws_bytes;
};

RoundArgs layer_chunk(const RoundArgs &r, const kvs_seqs *seqs, int32_t l0, int32_t n) {
  RoundArgs c = r;
  const int64_t P = r.cache.num_pages, Hkv = r.cache.num_kv_heads, S = seqs->num_seqs;
  const int64_t E = S ? seqs->entry_off_h[S] : 0;
  const int64_t Hq = r.obs.num_q_heads, O = r.obs.obs_total;
  c.cache.num_layers = n;
  c.cache.k = (uint16_t *)r.cache.k + l0 * P * Hkv * kvs::kPageElems;
  c.cache.v = (uint16_t *)r.cache.v + l0 * P * Hkv * kvs::kPageElems;
  c.cache.crf = r.cache.crf + l0 * P * Hkv * kvs::kPage;
  c.obs.q = (const uint16_t *)r.obs.q + l0 * Hq * O * kvs::kHeadDim;
  c.obs.lse = r.obs.lse + l0 * Hq * O;
  c.scores = r.scores + l0 * Hkv * E;
  c.keep = r.keep + l0 * Hkv * E;
  c.hit = r.hit ? r.hit + l0 * Hkv * E : nullptr;
  c.pairs = r.pairs ? r.pairs + l0 * Hkv * S * r.pair_cap * 2 : nullptr;
  c.pair_count = r.pair_count + l0 * Hkv * S;
  return c;
}

hipError_t round_score(const RoundArgs &r, const kvs_seqs *seqs, hipStream_t st) {
  const kvs::Batch b = make_batch(&r.cache, seqs);
  return kvs::launch_score(r.cache, b, r.obs, r.scale, r.scores, r.ws, r.ws_bytes, r.obs.obs_off_h, seqs->len_h,
                           seqs->start_h, st);
}

hipError_t round_select_move(const RoundArgs &r, const kvs_seqs *seqs, hipStream_t st) {
  const kvs::Batch b = make_batch(&r.cache, seqs);
  hipError_t e;
  if (kvs::stream_reg_fits(r.max_len, r.cache.num_pages, r.cache.num_kv_heads)) {
    e = kvs::launch_stream_reg_plan(r.cache, b, r.scores, r.mass_num, r.mass_den, r.decay, r.n_prev, r.hit,
                                    r.budget, r.keep, r.pairs, r.pair_count, r.pair_cap, st);
  } else {
    e = kvs::launch_lrfu(r.cache, b, r.scores, r.mass_num, r.mass_den, r.decay, r.n_prev, r.hit, r.max_len, st);
    if (e == hipSuccess) e = kvs::launch_select(r.cache, b, r.scores, r.budget, r.keep, r.max_len, st);
    if (e == hipSuccess) e = kvs::launch_plan(b, r.keep, r.budget, r.pairs, r.pair_count, r.pair_cap, st);
  }
  if (e != hipSuccess || r.pair_cap == 0) return e;
  return kvs::launch_compact(r.cache, b, r.pairs, r.pair_count, r.pair_cap, st);
}

}  // namespace

extern "C" {

kvs_status kvs_eviction_round(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_observers *obs, float scale,
                              uint32_t mass_num, uint32_t mass_den, const float *decay, const int32_t *n_prev,
                              const int32_t *budget, const int32_t *budget_h, float *scores, uint8_t *hit,
                              uint8_t *keep, int32_t *pairs, int32_t *pair_count, void *workspace,
                              size_t workspace_bytes, int32_t layer_chunks, int32_t *shift_h, int32_t *new_start_h,
                              int32_t *new_len_h, int32_t *freed_h, int64_t freed_capacity, int64_t *freed_count_h,
                              void *stream) {
  kvs_status st;
  if ((st = check_cache(cache, true, true)) != KVS_OK) return st;
  if ((st = check_seqs(seqs, cache->num_pages, true)) != KVS_OK) return st;
  if ((st = check_obs(obs, seqs, cache->num_kv_heads)) != KVS_OK) return st;
  if (!std::isfinite(scale)) return fail(KVS_ERR_SHAPE, "scale is not finite");
  if (mass_den == 0 || mass_num > mass_den)
    return fail(KVS_ERR_SHAPE, "mass fraction %u/%u must satisfy 0 <= num <= den, den > 0", mass_num, mass_den);
  if (layer_chunks < 1) return fail(KVS_ERR_SHAPE, "layer_chunks = %d < 1", layer_chunks);
  if (seqs->num_seqs > 0 && (!budget || !budget_h)) return fail(KVS_ERR_NULL, "budget is NULL");
  for (int32_t i = 0; i < seqs->num_seqs; ++i)
    if (budget_h[i] < 0) return fail(KVS_ERR_SHAPE, "budget[%d] = %d < 0", i, budget_h[i]);
  if ((st = kvs_plan_host(seqs, budget_h, shift_h, new_start_h, new_len_h, freed_h, freed_capacity,
                          freed_count_h)) != KVS_OK)
    return st;
  if (seqs->num_seqs == 0) return ok();
  const kvs::Batch b = make_batch(cache, seqs);
  if (b.E == 0) return ok();
  const int64_t P = pair_cap_of(seqs, budget_h);
  if (!scores || !decay || !n_prev || !keep || !pair_count || (P > 0 && !pairs))
    return fail(KVS_ERR_NULL, "scores/decay/n_prev/keep/pairs/pair_count is NULL");
  const size_t need = kvs::score_workspace_bytes(b, obs->num_q_heads, obs->obs_off_h, seqs->len_h, seqs->start_h);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KVS_ERR_WORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, need);
  RoundArgs r{};
  r.cache = *cache;
  r.obs = *obs;
  r.scale = scale;
  r.mass_num = mass_num;
  r.mass_den = mass_den;
  r.decay = decay;
  r.n_prev = n_prev;
  r.budget = budget;
  r.scores = scores;
  r.hit = hit;
  r.keep = keep;
  r.pairs = pairs;
  r.pair_count = pair_count;
  r.pair_cap = P;
  r.max_len = max_len_of(seqs);
  r.ws = workspace;
  r.ws_bytes = workspace_bytes;
  const hipStream_t main = (hipStream_t)stream;
  const int32_t L = cache->num_layers;
  const int32_t chunks = layer_chunks < L ? layer_chunks : L;
  if (chunks == 1) {
    hipError_t e = round_score(r, seqs, main);
    if (e == hipSuccess) e = round_select_move(r, seqs, main);
    return hip_status(e);
  }
  // Scoring of chunk c + 1 (on the caller's stream) overlaps the cut, keep set and moves
  // of chunk c (on a side stream): different layers, so different memory.
  std::lock_guard<std::mutex> lock(g_round_mu);
  RoundRes *res = nullptr;
  hipError_t e = round_resources(chunks + 2, &res);
  if (e != hipSuccess) return hip_status(e);
  const hipStream_t side = res->side;
  const std::vector<hipEvent_t> &ev = res->ev;
  e = hipEventRecord(ev[0], main);                               // the inputs are ready
  if (e == hipSuccess) e = hipStreamWaitEvent(side, ev[0], 0);
  for (int32_t c = 0; c < chunks && e == hipSuccess; ++c) {
    const int32_t l0 = (int32_t)((int64_t)L * c / chunks), l1 = (int32_t)((int64_t)L * (c + 1) / chunks);
    const RoundArgs rc = layer_chunk(r, seqs, l0, l1 - l0);
    e = round_score(rc, seqs, main);
    if (e == hipSuccess) e = hipEventRecord(ev[c + 1], main);
    if (e == hipSuccess) e = hipStreamWaitEvent(side, ev[c + 1], 0);
    if (e == hipSuccess) e = round_select_move(rc, seqs, side);
  }
  if (e == hipSuccess) e = hipEventRecord(ev[chunks + 1], side);
  if (e == hipSuccess) e = hipStreamWaitEvent(main, ev[chunks + 1], 0);   // the caller's stream sees it all
  return hip_status(e);
}

}  // extern "C"
