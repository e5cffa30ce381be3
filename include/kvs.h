/*
 * kvs.h -- C ABI of libkvs: attention-guided KV eviction and in-place compaction
 * of a paged bf16 KV cache on AMD Instinct MI355X (gfx950).
 *
 * One eviction round is five calls, enqueued in order on one HIP stream:
 *
 *   kvs_score        attention each cached entry receives from a set of observer
 *                    queries, recovered from the decode kernel's log-sum-exp and
 *                    summed over observers and the GQA group
 *   kvs_lrfu_update  the attention-mass cut ("action-critical" hits) and the LRFU
 *                    update of each entry's combined recency-frequency value (CRF)
 *   kvs_select       the per-(layer, KV head) keep set of exactly min(B, n) entries
 *   kvs_lrfu_select  the two calls above fused (same results, one pass over the data)
 *   kvs_plan         the conflict-free slot plan: kept rows outside the tail paired
 *                    with evicted slots inside it; the freed pages (host side)
 *   kvs_compact      one in-place pass that moves K row, V row and CRF per pair
 *   kvs_plan_compact the two calls above fused (same results)
 *
 * kvs_decode_attention is the decode step itself with the same tally folded in:
 * paged attention that emits the LSE and adds the action tokens' attention to the
 * scores (ActKV, Component 3).
 *
 * and, for the budget that the rounds use (ActKV, Component 2):
 *
 *   kvs_token_confidence  per decode step, the mean negative log-probability of
 *                         the k most probable tokens (the model's confidence)
 *   kvs_confidence_trend  min-pooling of those values and the sign of a fitted
 *                         line: the flag for kvs_budget_ratchet (host)
 *
 * Sources, cited by page title and section:
 *   "ActKV Dissected: 99% of an Agent's KV Cache Is Scratch Work, and the Budget
 *   Follows Hesitation" (zhichai.net):  Summary; Component 1 (action-attention-
 *   guided eviction); Component 2 (budget follows hesitation); Component 3
 *   (systems engineering); Lineage.
 *   "BeaconKV Compresses KV Cache for Long-Reasoning Models with Beacon Queries"
 *   (cctest.ai): Key ideas (beacon plus recent queries as the observer set).
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless their name ends in _h (host memory).
 *   - The caller owns and allocates all memory.  No call allocates, frees,
 *     synchronizes, or copies between host and device; every call first
 *     validates its arguments on the host and, on error, enqueues nothing and
 *     returns a non-zero kvs_status (kvs_last_error() then describes it).
 *   - Host mirrors (_h) must hold the same values as their device arrays; they
 *     size the launches and are range-checked so that no kernel reads outside a
 *     pool.  Device contents that disagree with their mirrors are undefined
 *     behaviour.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls on different
 *     streams are independent as long as their outputs are disjoint.
 *   - Layout constants: head_dim = 128 and page_size = 16 only (else
 *     KVS_ERR_UNSUPPORTED).
 */
#ifndef KVS_H
#define KVS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvs_status {
  KVS_OK = 0,
  KVS_ERR_NULL = 1,         /* a required pointer is NULL */
  KVS_ERR_SHAPE = 2,        /* sizes inconsistent or out of range (page id, lengths, budget...) */
  KVS_ERR_UNSUPPORTED = 3,  /* head_dim != 128, page_size != 16, or a limit exceeded */
  KVS_ERR_WORKSPACE = 4,    /* workspace missing or smaller than required */
  KVS_ERR_HIP = 5           /* a HIP runtime error (launch failure) */
} kvs_status;

/*
 * Paged KV cache (ActKV, Component 3: the cache is held in fixed-size blocks of
 * a paged-attention engine).  One (layer, page, KV head) block of K or V is 16
 * rows x 128 bf16 = 4 KiB, contiguous:
 *   k, v : bf16 [num_layers][num_pages][num_kv_heads][16][128]
 *   crf  : fp32 [num_layers][num_pages][num_kv_heads][16]
 * crf is the per-slot LRFU state (ActKV, Component 1); it lives in a paged side
 * pool with the same page ids as K/V so that kvs_compact moves it with its row.
 */
typedef struct kvs_cache {
  void *k;
  void *v;
  float *crf;
  int32_t num_layers;
  int32_t num_kv_heads;
  int32_t head_dim;      /* must be 128 */
  int32_t page_size;     /* must be 16 */
  int64_t num_pages;
} kvs_cache;

/*
 * A batch of sequences.  Sequence i owns logical pages 0..npages_i-1 mapped to
 * physical pages block_table[i][*]; its live entries are slots j = 0..len[i]-1
 * at logical positions start[i] + j (start in 0..15: the first live row inside
 * logical page 0).  npages_i = ceil((start[i] + len[i]) / 16) <= max_pages.
 * Per-entry arrays (scores, hit, keep) are [num_layers][num_kv_heads][E] with
 * E = entry_off[num_seqs]; sequence i's entries sit at entry_off[i] + j, and
 * entry_off[i+1] - entry_off[i] must equal len[i].
 * A *stream* is one (sequence, layer, KV head): its own scores, hits, CRF, keep
 * set and moves.
 */
typedef struct kvs_seqs {
  int32_t num_seqs;
  int32_t max_pages;
  const int32_t *block_table;    /* [num_seqs][max_pages] */
  const int32_t *block_table_h;
  const int32_t *start;          /* [num_seqs] */
  const int32_t *start_h;
  const int32_t *len;            /* [num_seqs] */
  const int32_t *len_h;
  const int64_t *entry_off;      /* [num_seqs + 1] */
  const int64_t *entry_off_h;
} kvs_seqs;

/*
 * Observer queries and their log-sum-exp (ActKV, Component 3: the LSE is a
 * byproduct of paged attention; BeaconKV, Key ideas: beacon queries alongside
 * recent queries -- both are simply observers here, weighted equally).
 *   q   : bf16 [num_layers][num_q_heads][obs_total][128]
 *   lse : fp32 [num_layers][num_q_heads][obs_total], natural log, over the same
 *         live entries and the same scale as kvs_score uses
 * Sequence i's observers are obs_off[i] .. obs_off[i+1]-1.  Query head h reads
 * KV head h / (num_q_heads / num_kv_heads).
 */
typedef struct kvs_observers {
  const void *q;
  const float *lse;
  const int64_t *obs_off;        /* [num_seqs + 1] */
  const int64_t *obs_off_h;
  int32_t num_q_heads;
  int64_t obs_total;
} kvs_observers;

/* Human-readable name of a status code (static storage). */
const char *kvs_status_string(kvs_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *kvs_last_error(void);

/*
 * Bytes of device workspace kvs_score needs for this batch: fp32 partial sums
 * per group of 256 observer rows for every entry when some sequence has more
 * than 256 rows (observers x GQA group), plus two small work-item tables when the
 * batch has more than 255 sequences.  0 otherwise.  Returns 0 (and sets
 * kvs_last_error()) on invalid arguments.
 */
size_t kvs_score_workspace_size(const kvs_cache *cache, const kvs_seqs *seqs,
                                const kvs_observers *obs);

/*
 * kvs_score -- ActKV, Component 3 (attention recovered per block by subtracting
 * the LSE from the query's logits: no gather, no recomputation) and Component 1
 * (each entry's attention tallied over all action tokens).  For every stream
 * (i, l, g) and live slot j:
 *     s_j = sum over observers o of sequence i and query heads h of group g of
 *           exp(scale * <q[l][h][o], k_j> - lse[l][h][o])
 * bf16 inputs, fp32 accumulation.  Writes scores (fp32 [L][Hkv][E]); entries of
 * a sequence with no observers get 0.  Sequences with 16 or more observers use
 * the MFMA kernel, the others a VALU dot-product kernel.
 * workspace: device, >= kvs_score_workspace_size bytes, 256-byte aligned; its
 * contents are scratch (overwritten).
 */
kvs_status kvs_score(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_observers *obs,
                     float scale, float *scores, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * kvs_lrfu_update -- ActKV, Component 1.  Per stream:
 *   1. mass cut: m_j = floor(s_j * 2^32) (integers), M = sum m_j,
 *      T = ceil(mass_num * M / mass_den); hits are the shortest prefix of the
 *      order (s desc, slot asc) whose mass reaches T (no hits if T == 0).
 *      mass_num/mass_den = 9/10 is the pages' "top 90%".
 *   2. LRFU: CRF_j <- fma(decay[i], CRF_j, hit_j) in fp32, with CRF_j taken as 0
 *      for j >= n_prev[i] (entries appended since the last round).
 *      decay[i] = fp32(2^(-lambda * dt_i)); kvs_lrfu_decay() computes it.
 * scores must be finite and >= 0 (as kvs_score produces).  crf is updated in
 * place through the block table.  hit (nullable): uint8 [L][Hkv][E], 1 = hit.
 * decay: fp32 [num_seqs] (device); n_prev: int32 [num_seqs] (device).
 * Requires 0 < mass_den, mass_num <= mass_den.
 */
kvs_status kvs_lrfu_update(const kvs_cache *cache, const kvs_seqs *seqs, const float *scores,
                           uint32_t mass_num, uint32_t mass_den, const float *decay,
                           const int32_t *n_prev, uint8_t *hit, void *stream);

/* fp32(2^(-lambda * dt)) computed in double on the host (LRFU weight of dt steps). */
float kvs_lrfu_decay(double lambda, int32_t dt);

/*
 * kvs_select -- ActKV, Summary/Results (an entry budget per head).  Per stream,
 * keep exactly K = min(budget[i], len[i]) entries: the first K of the order
 * (CRF desc, s desc, slot asc), comparing fp32 values (all >= 0).
 * keep: uint8 [L][Hkv][E] (1 = keep).  budget: int32 [num_seqs] device, with its
 * host mirror budget_h (values >= 0).
 */
kvs_status kvs_select(const kvs_cache *cache, const kvs_seqs *seqs, const float *scores,
                      const int32_t *budget, const int32_t *budget_h, uint8_t *keep,
                      void *stream);

/*
 * kvs_lrfu_select -- kvs_lrfu_update followed by kvs_select in one call, with the
 * same arguments, validation and results (crf, hit and keep are written exactly as
 * the two calls would write them).  Each stream's scores and CRF are read once.
 */
kvs_status kvs_lrfu_select(const kvs_cache *cache, const kvs_seqs *seqs, const float *scores,
                           uint32_t mass_num, uint32_t mass_den, const float *decay,
                           const int32_t *n_prev, uint8_t *hit, const int32_t *budget,
                           const int32_t *budget_h, uint8_t *keep, void *stream);

/*
 * Reasoning steps of each sequence (StepKV, Abstract: cache entries are associated
 * with the step that generated them).  Sequence i's steps are the global step ids
 * step_off[i] .. step_off[i+1]-1; step k covers live slots first[k] .. (first of the
 * next step of the sequence, or len[i]) - 1.  Requirements (checked on the host
 * mirrors): step_off[0] = 0, non-decreasing; within a sequence first[] starts at 0,
 * never decreases and stays <= len[i] (empty steps are allowed); a sequence with live
 * entries has at least one step.  At most 2^31 steps.  The same steps hold for every
 * layer and KV head.
 */
typedef struct kvs_steps {
  const int64_t *step_off;      /* [num_seqs + 1] */
  const int64_t *step_off_h;
  const int32_t *first;         /* [step_off[num_seqs]] */
  const int32_t *first_h;
} kvs_steps;

/* Bytes of workspace kvs_step_select needs (the combined keys, fp32 [L][Hkv][E]); 0 on
 * invalid arguments (kvs_last_error() says which). */
size_t kvs_step_select_workspace_size(const kvs_cache *cache, const kvs_seqs *seqs,
                                      const kvs_steps *steps);

/*
 * kvs_step_select -- StepKV, Abstract: step utility combined with token saliency
 * ranks the prunable entries, and the top ones are kept under the budget.  Per
 * stream (sequence, layer, KV head), with a_j = floor(s_j * 2^32):
 *   U_k = fp32(floor(sum_{j in step k} a_j / |k|) * 2^-32)   (0 for an empty step),
 *   c_j = fma(beta, U_k(j), fp32(fp32(1 - beta) * s_j)),
 *   keep = the first K = min(budget[i], len[i]) entries of (c desc, s desc, slot asc).
 * Every live entry is prunable.  scores: fp32 [L][Hkv][E], finite, >= 0, with the
 * scores of any one step summing to less than 2^32.  beta in [0, 1].
 * keep: uint8 [L][Hkv][E].  utility: fp32 [L][Hkv][num_steps] (U of every step) or
 * NULL.  budget: int32 [num_seqs] device with its host mirror budget_h (>= 0).
 * workspace: device, >= kvs_step_select_workspace_size(), 256-byte aligned; scratch.
 * Exact: the keep set and the utilities are defined to the bit.  cache supplies the
 * shape only (k, v and crf are not read).
 */
kvs_status kvs_step_select(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_steps *steps,
                           const float *scores, float beta, const int32_t *budget,
                           const int32_t *budget_h, uint8_t *keep, float *utility,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * kvs_beacon_seed -- the initial centroids of kvs_beacon_kmeans by k-means++: for each
 * problem, centroid 0 is row floor(u_0 * n); then, with D2_i the squared distance
 * (fp32 sums) from row i to its nearest chosen centroid, centroid c is the first row
 * in row order whose running sum of D2 exceeds u_c * sum(D2) (a draw with probability
 * D2_i / sum(D2)), or row floor(u_c * n) when every D2 is 0.  Rows with D2 = 0 are
 * never drawn otherwise.  points: bf16 [num_problems][num_points][128], finite.
 * uniforms: fp32 [num_problems][k] in [0, 1), the draws (the caller's generator).
 * centroids: fp32 [num_problems][k][128] out (the chosen rows, exact).  rows: int32
 * [num_problems][k] out (the chosen row indices) or NULL.  1 <= k <= 16,
 * 1 <= num_points <= 16384.  One workgroup per problem; no workspace.
 */
kvs_status kvs_beacon_seed(const void *points, int64_t num_problems, int32_t num_points, int32_t k,
                           const float *uniforms, float *centroids, int32_t *rows, void *stream);

/*
 * kvs_beacon_kmeans -- BeaconKV, Key ideas: queries that revisit distant context form
 * a few similarity groups, and one representative per group (a beacon query) joins the
 * recent queries as an observer.  Lloyd's k-means for num_problems independent
 * problems (one per layer and query head, say), each over num_points history queries
 * of 128 bf16 values, from given initial centroids, for iters iterations:
 *   assignment  a_i = the k minimising ||c_k||^2 - 2 <x_i, c_k> (ties to the lower k),
 *               scored in fp32 with each centroid carried to 16 significant bits;
 *   update      c_kd = the mean of the members' coordinates d, rounded once to fp32
 *               (nearest, ties to even); a group without members keeps its centroid.
 *               The sums are exact integers on the 2^-32 grid, so the result is the
 *               exact mean rounded once whenever no member coordinate lies in
 *               0 < |x| < 2^-25 (those are truncated toward zero on the grid, which
 *               moves the mean by less than 2^-32), and never depends on member order.
 * points: bf16 [num_problems][num_points][128], finite with |x| < 2^15.
 * centroids: fp32 [num_problems][k][128], the initial centroids in, the final out.
 * assign: int32 [num_problems][num_points] (the last iteration's assignments; not
 * written when iters = 0) or NULL.  beacons: bf16 [num_problems][k][128] (the final
 * centroids rounded to nearest, ties to even) or NULL.  1 <= k <= 16,
 * 1 <= num_points <= 65536 (KVS_ERR_UNSUPPORTED beyond), iters >= 0.  One workgroup
 * per problem; no workspace.
 */
kvs_status kvs_beacon_kmeans(const void *points, int64_t num_problems, int32_t num_points, int32_t k,
                             int32_t iters, float *centroids, int32_t *assign, void *beacons,
                             void *stream);

/*
 * Per-stream capacity of the move-pair buffer for this batch and budget:
 *   P = max over sequences of min(len_i - K_i, K_i),  K_i = min(budget_h[i], len_i).
 * pairs must hold int32 [num_layers][num_kv_heads][num_seqs][P][2] and pair_count
 * int32 [num_layers][num_kv_heads][num_seqs].  Returns -1 (and sets
 * kvs_last_error()) on invalid arguments.
 */
int64_t kvs_pair_capacity(const kvs_seqs *seqs, const int32_t *budget_h);

/*
 * kvs_plan -- ActKV, Component 3 (survivors skew to the tail, so the tail is the
 * target region; survivors outside it are paired one-to-one with holes inside
 * it).  Per stream, with K = min(budget_i, len_i) and D = len_i - K:
 *   sources      = kept slots j < D, ascending
 *   destinations = evicted slots j >= D, ascending
 * pair t = (source_t, destination_t) is written to
 *   pairs[(((l * Hkv + g) * num_seqs + i) * P + t) * 2 + {0, 1}],  P = kvs_pair_capacity,
 * and pair_count[(l * Hkv + g) * num_seqs + i] receives the number of pairs.
 * keep (uint8 [L][Hkv][E]) must hold exactly K ones per stream, as kvs_select
 * writes; with another count the pairs written stay within the capacity but the
 * plan is meaningless.  budget: int32 [num_seqs] device, budget_h its host mirror.
 * Host outputs (each nullable), computed from host data only, no wait:
 *   shift_h[i]     = (start_i + D) / 16   logical pages freed at the front
 *   new_start_h[i] = (start_i + D) % 16
 *   new_len_h[i]   = K
 *   freed_h        = block_table_h[i][0 .. shift_i-1] for each i in order
 *                    (ActKV, Component 3: freed blocks go back to the scheduler);
 *                    capacity freed_capacity entries, count in *freed_count_h.
 * After kvs_compact has run, the live entries of sequence i are logical
 * positions start_i + D .. start_i + len_i - 1: the caller drops the first
 * shift_i block-table entries and sets start = new_start, len = new_len.  Freed
 * pages may be reused only by work enqueued after kvs_compact on the same
 * stream (it still reads them).
 */
kvs_status kvs_plan(const kvs_seqs *seqs, int32_t num_layers, int32_t num_kv_heads,
                    const uint8_t *keep, const int32_t *budget, const int32_t *budget_h,
                    int32_t *pairs, int32_t *pair_count, int32_t *shift_h, int32_t *new_start_h,
                    int32_t *new_len_h, int32_t *freed_h, int64_t freed_capacity,
                    int64_t *freed_count_h, void *stream);

/*
 * The host outputs of kvs_plan alone (same definitions, same argument rules), for
 * callers that plan page reuse before enqueuing any device work.  Touches no
 * device memory.
 */
kvs_status kvs_plan_host(const kvs_seqs *seqs, const int32_t *budget_h, int32_t *shift_h,
                         int32_t *new_start_h, int32_t *new_len_h, int32_t *freed_h,
                         int64_t freed_capacity, int64_t *freed_count_h);

/*
 * kvs_compact -- ActKV, Component 3 (copied in one parallel pass; no extra KV
 * buffer).  For every pair of every stream, copies the K row (256 B), the V row
 * (256 B) and the CRF value of the source slot onto the destination slot, in
 * place, addressed through the pre-compaction layout in seqs.  Sources and
 * destinations of a plan from kvs_plan are disjoint, so the pairs are applied
 * in any order.  budget_h must be the array given to kvs_plan (it fixes P).
 */
kvs_status kvs_compact(const kvs_cache *cache, const kvs_seqs *seqs, const int32_t *budget_h,
                       const int32_t *pairs, const int32_t *pair_count, void *stream);

/*
 * kvs_lrfu_select_compact -- kvs_lrfu_select followed by kvs_plan_compact in one call, with
 * the union of their arguments and validation, and the same results: hit (optional),
 * keep, the updated CRF, pairs, pair_count, the host outputs, and the moved K/V rows and
 * CRF values.  ActKV Dissected, Component 1 (the 90 % attention-mass cut, LRFU) and
 * Summary (top-B per head), then Component 3 (the slot plan and the one-pass in-place
 * move).  While every stream has at most 32 768 entries, one kernel workgroup per stream
 * selects and plans it (the plan as soon as its keep set is written) and one further
 * kernel moves all pairs; otherwise the two calls run in turn.  Errors as for the two
 * calls; on error nothing is enqueued.
 */
kvs_status kvs_lrfu_select_compact(const kvs_cache *cache, const kvs_seqs *seqs, const float *scores,
                                   uint32_t mass_num, uint32_t mass_den, const float *decay, const int32_t *n_prev,
                                   uint8_t *hit, const int32_t *budget, const int32_t *budget_h, uint8_t *keep,
                                   int32_t *pairs, int32_t *pair_count, int32_t *shift_h, int32_t *new_start_h,
                                   int32_t *new_len_h, int32_t *freed_h, int64_t freed_capacity,
                                   int64_t *freed_count_h, void *stream);

/*
 * kvs_plan_compact -- kvs_plan followed by kvs_compact in one call, with the union of
 * their arguments and validation, and the same results (pairs, pair_count, the host
 * outputs and the moved K/V rows and CRF values).
 */
kvs_status kvs_plan_compact(const kvs_cache *cache, const kvs_seqs *seqs, const uint8_t *keep,
                            const int32_t *budget, const int32_t *budget_h, int32_t *pairs,
                            int32_t *pair_count, int32_t *shift_h, int32_t *new_start_h,
                            int32_t *new_len_h, int32_t *freed_h, int64_t freed_capacity,
                            int64_t *freed_count_h, void *stream);

/*
 * kvs_eviction_round -- the whole round in one call: kvs_score, then kvs_lrfu_select,
 * then kvs_plan_compact, with the union of their arguments and validation and the
 * same results (scores, crf, hit, keep, pairs, pair_count, moved rows, host outputs).
 * ActKV, Component 3: eviction runs beside decoding on the engine's paged blocks.
 * layer_chunks > 1 splits the layers into that many contiguous chunks and overlaps
 * the scoring of chunk c + 1 (on `stream`) with the cut, keep set and moves of chunk c
 * (on a library-owned side stream of the same device, default priority; every array
 * has the layer outermost, so chunks touch disjoint memory).  All work is ordered
 * after what `stream` held at the call and before what it is given next.
 * workspace: >= kvs_score_workspace_size(cache, seqs, obs), as for kvs_score (the
 * chunks use it in turn).  Calls that overlap on one device share the side stream.
 */
kvs_status kvs_eviction_round(const kvs_cache *cache, const kvs_seqs *seqs, const kvs_observers *obs,
                              float scale, uint32_t mass_num, uint32_t mass_den, const float *decay,
                              const int32_t *n_prev, const int32_t *budget, const int32_t *budget_h,
                              float *scores, uint8_t *hit, uint8_t *keep, int32_t *pairs,
                              int32_t *pair_count, void *workspace, size_t workspace_bytes,
                              int32_t layer_chunks, int32_t *shift_h, int32_t *new_start_h,
                              int32_t *new_len_h, int32_t *freed_h, int64_t freed_capacity,
                              int64_t *freed_count_h, void *stream);

/*
 * Host-side budget ratchet (ActKV, Component 2 and Lineage): for each sequence
 * whose flag_h is non-zero, budget_h[i] <- max(budget_h[i],
 * min(cap, floor(budget_h[i] * num / den))).  The pages' ratchet is num/den = 7/4,
 * cap = 30000, starting from 512; the budget never shrinks.
 */
kvs_status kvs_budget_ratchet(int32_t *budget_h, const uint8_t *flag_h, int32_t num_seqs,
                              int32_t num, int32_t den, int32_t cap);

/*
 * Bytes of device workspace kvs_decode_attention needs (tally != 0: with the
 * per-entry logits kept for the score tally, 4 x rows bytes per entry).  Returns 0
 * (and sets kvs_last_error()) on invalid arguments.
 */
size_t kvs_decode_workspace_size(const kvs_cache *cache, const kvs_seqs *seqs,
                                 const kvs_observers *queries, int32_t tally);

/*
 * kvs_decode_attention -- ActKV, Component 3 (the log-sum-exp is a byproduct of
 * paged attention, and each block's attention is recovered from it without
 * gathering or recomputing the attention matrix) and Component 1 (an entry's signal
 * is the attention it receives from the action tokens).  For every sequence i, KV
 * head g and query row r = (query head h of g's group, token t of the call):
 *     logit_rj = scale * <q_r, k_j> over the n_i live entries j (no mask),
 *     lse_r    = ln sum_j exp(logit_rj),
 *     out_r    = sum_j exp(logit_rj - lse_r) v_j,
 * and, when scores is not NULL (the call's tokens are action tokens),
 *     scores_j += sum over the rows of g of exp(logit_rj - lse_r)
 * -- the quantity kvs_score computes for observers given their LSE.
 * queries: the observer structure holding the call's decode tokens: q bf16
 *   [L][Hq][T_tot][128], obs_off = token offsets [num_seqs + 1] (with host mirror),
 *   num_q_heads, obs_total = T_tot; its lse field is not read.  At most 16 rows per
 *   (sequence, KV head): Hq / Hkv x tokens <= 16, and start + length of every
 *   sequence <= 4 194 304 positions (else KVS_ERR_UNSUPPORTED).
 * out: fp32 [L][Hq][T_tot][128]; lse: fp32 [L][Hq][T_tot] (sequences with no live
 *   entries get out = 0 and lse = -inf).  scores: fp32 [L][Hkv][E] or NULL.
 * workspace: device, >= kvs_decode_workspace_size(..., scores != NULL), 256-byte
 *   aligned; scratch.  fp32 arithmetic with bf16 inputs.
 */
kvs_status kvs_decode_attention(const kvs_cache *cache, const kvs_seqs *seqs,
                                const kvs_observers *queries, float scale, float *out, float *lse,
                                float *scores, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Logit element types for kvs_token_confidence.
 */
enum { KVS_DTYPE_F32 = 0, KVS_DTYPE_BF16 = 1 };

/*
 * Bytes of device workspace kvs_token_confidence needs: (2 + k) fp32 partial
 * results per (row, chunk), chunks of 16 384 logits for k <= 32 and of 8 192 above;
 * 0 when a row is one chunk.  Sized for fp32 logits (bf16 chunks are twice as long,
 * so bf16 rows need at most this).  Returns 0 (and sets kvs_last_error()) on invalid
 * arguments.
 */
size_t kvs_token_confidence_workspace_size(int64_t rows, int64_t vocab, int32_t k);

/*
 * kvs_token_confidence -- ActKV, Component 2 (the model's hesitation at each step,
 * read from the top-20 tokens of the step's output distribution).  For every row r
 * (one decode step's logits z over the vocabulary, softmax at temperature 1):
 *     conf[r] = (1/k) * sum over the k largest z_j of -ln softmax(z)_j
 *             = LSE(z) - mean of the k largest z_j
 * i.e. the mean negative log-probability of the k most probable tokens (the pages:
 * k = 20).  A peaked distribution gives a large value, a flat one a value near
 * ln(vocab).  fp32 arithmetic; which of several equal logits fill the k-th place
 * does not change the result.
 * logits: device, [rows][row_stride] elements of type dtype (KVS_DTYPE_F32 or
 *   KVS_DTYPE_BF16), the first vocab of each row used.  -inf logits are tokens of
 *   probability 0 (a row needs at least one finite logit; fewer than k finite ones
 *   give +inf); NaN is undefined.
 * conf: device fp32 [rows].  1 <= k <= 64, k <= vocab <= 2^20 (else
 *   KVS_ERR_SHAPE / KVS_ERR_UNSUPPORTED).  workspace: device, at least
 *   kvs_token_confidence_workspace_size bytes (scratch, overwritten), 4-byte aligned.
 */
kvs_status kvs_token_confidence(const void *logits, int32_t dtype, int64_t rows, int64_t vocab,
                                int64_t row_stride, int32_t k, float *conf, void *workspace,
                                size_t workspace_bytes, void *stream);

/*
 * kvs_token_confidence_static -- kvs_token_confidence for callers that cannot
 * allocate device memory (code under graph capture, serving loops that forbid
 * allocation): the same computation and results, with the partial results in a
 * buffer the library holds instead of a caller workspace.  Same arguments as
 * kvs_token_confidence without workspace/workspace_bytes.  The buffer is a static
 * device array of 16 MiB, one per GPU the library runs on, held until the process
 * ends; its address is looked up once per device on the first call with that device
 * current.  Calls whose partial results need more (kvs_token_confidence_workspace_size
 * above 16 MiB, e.g. 4 096 rows at a vocabulary above 2^17 with k = 20) return
 * KVS_ERR_UNSUPPORTED.  This call allocates nothing, and nothing in the buffer must
 * start at zero.  Every call on one GPU shares that GPU's buffer: calls that overlap
 * on one GPU (concurrent streams, or threads) race and give undefined results.
 */
kvs_status kvs_token_confidence_static(const void *logits, int32_t dtype, int64_t rows, int64_t vocab,
                                       int64_t row_stride, int32_t k, float *conf, void *stream);

/*
 * kvs_confidence_trend (host) -- ActKV, Component 2 (token-level confidence
 * min-pooled over sliding windows into a trajectory-level series; a fitted line
 * with negative slope means the budget is too small).  From n token confidences
 * conf_h (host, in step order):
 *   pooled[w] = min(conf_h[w*stride .. w*stride + window - 1]), for every full
 *               window, P = (n - window) / stride + 1 of them (0 if n < window);
 *               the pages: window 64, stride 8;
 *   slope     = ordinary least-squares slope of the last fit_last pooled values
 *               (0 = all P) against their index 0, 1, ..., in fp64;
 *   flag      = 1 if slope < 0, else 0 (also 0 when fewer than two values are fitted,
 *               and then slope = NaN).
 * pooled_h (nullable): host double [P]; pooled_count_h, slope_h (nullable): host.
 * flag_h: host int32, feed it to kvs_budget_ratchet.
 */
kvs_status kvs_confidence_trend(const float *conf_h, int64_t n, int32_t window, int32_t stride,
                                int64_t fit_last, double *pooled_h, int64_t *pooled_count_h,
                                double *slope_h, int32_t *flag_h);

/* Library version string. */
const char *kvs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVS_H */
