/*
 * kvc.h -- fixed-budget KV-cache decode step (attend, score, aggregate, select,
 * fold, compact) and LaProx prefill scoring, as hand-written HIP for MI355X
 * (gfx950). C ABI: plain pointers and sizes, no C++ or torch types.
 *
 * Sources (the pages these operations are defined on):
 *   MomentKV  -- "MOMENTKV: Closing the Directional Gap in KV Cache Eviction for
 *                Long-Context Inference" (summary page): moment statistics §4.1,
 *                moment-informed eviction and corrected inference §4.2,
 *                Algorithm 1, Appendix A.1.
 *   InertiaKV -- "Key factors of KV cache eviction under aggressive decoding:
 *                temporal aggregation and rank preservation" (translated
 *                article): per-token score §3.1 eq. (1), utility rules eqs. (2)-(4),
 *                budget §3.
 *   KeepKV    -- reading notes on "KeepKV: Achieving Periodic Lossless KV Cache
 *                Compression": attention eq. (1), votes eqs. (6)-(7), ZIP merge
 *                eqs. (8)-(12), numerical-stability guard, framework integration,
 *                EMA score prediction eqs. (14)-(15), the inference algorithm's
 *                prefill compression.
 *   LaProx    -- notes on "Reformulating KV Cache Eviction Problem for
 *                Long-Context LLM Inference": key designs 1-3, GQA paragraph.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership. Every array argument is DEVICE memory owned by the caller. The
 *   library allocates nothing and keeps no state between calls; scratch lives
 *   in a caller-provided workspace sized by the *_workspace_size helpers.
 * Streams. `stream` is a hipStream_t passed as void* (NULL = default stream).
 *   Calls only enqueue work; results are ready when the stream reaches them.
 * Errors. Each call returns KVC_OK (0) or a negative KVC_ERR_* code after
 *   validating its host-visible arguments; a call that returns an error has
 *   enqueued nothing. Conditions only the device can see (a live length that
 *   exceeds the capacity) are recorded in the workspace status word, readable
 *   with kvc_workspace_status().
 * Units and scopes. A unit is one KV head of one layer of one sequence. A
 *   scope is the set of units that share one slot set: votes, positions,
 *   utilities and the live length are per scope; K and V rows are per unit.
 *   Row r of a unit's K (or V) is at element offset (row_base + r) * head_dim,
 *   with row_base = scope * scope_stride + unit * unit_stride.
 * GQA. Query head h of a layer reads KV head h / G (consecutive grouping);
 *   queries are laid out [scope][unit][G][head_dim].
 * Head dimension. head_dim must be 128 (KVC_ERR_UNSUPPORTED otherwise).
 * Alignment. K, V, q and new-row pointers must be 16-byte aligned (KVC_ERR_ALIGN).
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_VERSION 1

enum kvc_status {
  KVC_OK = 0,
  KVC_ERR_ARG = -1,          /* null pointer, negative size, inconsistent sizes */
  KVC_ERR_DTYPE = -2,        /* dtype is not KVC_BF16 / KVC_F32 */
  KVC_ERR_UNSUPPORTED = -3,  /* head_dim != 128, G not in {1,2,4,8}, shape beyond limits */
  KVC_ERR_CAPACITY = -4,     /* append into a full cache, max_len > capacity, budget < 0 */
  KVC_ERR_ALIGN = -5,        /* K/V/q/new rows not 16-byte aligned */
  KVC_ERR_WORKSPACE = -6,    /* workspace missing or smaller than required */
  KVC_ERR_DEVICE = -7        /* HIP launch failure */
};

enum kvc_dtype { KVC_BF16 = 0, KVC_F32 = 1 };

/* InertiaKV §3.1, eqs. (2)-(4). */
enum kvc_rule { KVC_RULE_SINGLE = 0, KVC_RULE_CUMULATIVE = 1, KVC_RULE_EMA = 2 };

/* Cache descriptor. All pointers are device pointers. */
typedef struct kvc_cache {
  int32_t dtype;            /* enum kvc_dtype of K and V (queries and new rows use it too) */
  int32_t head_dim;         /* must be 128 */
  int32_t capacity;         /* slots per scope */
  int32_t n_scopes;
  int32_t units_per_scope;  /* KV heads sharing one slot set (1: per-head scope) */
  int32_t reserved;
  int64_t scope_stride;     /* rows between the first units of consecutive scopes */
  int64_t unit_stride;      /* rows between consecutive units of one scope */
  void *k, *v;              /* [rows][head_dim] in dtype */
  int32_t *votes;           /* [n_scopes][capacity] KeepKV votes, or NULL (every vote is 1) */
  int32_t *pos;             /* [n_scopes][capacity] token positions (distinct among live slots) */
  float *m;                 /* [n_scopes][capacity] utilities (fp32) */
  int32_t *len;             /* [n_scopes] live slots; slots [0, len) are live */
} kvc_cache;

/* MomentKV running sums per unit (MomentKV §4.1): count, key sum, value sum
 * and value-key outer-product sum S[a][b] = sum_e v_{e,a} k_{e,b}, fp32. */
typedef struct kvc_moments {
  int32_t *n;               /* [n_scopes][units_per_scope] */
  float *sk;                /* [n_scopes][units_per_scope][head_dim] */
  float *sv;                /* [n_scopes][units_per_scope][head_dim] */
  float *S;                 /* [n_scopes][units_per_scope][head_dim][head_dim], row-major */
} kvc_moments;

/* KeepKV ZIP-merge parameters (eqs. (8)-(12), stability guard). The reference
 * logit of an entry is the mean over the group's G query heads of
 * scale * q_g . k, i.e. the logit of the group-mean query. */
typedef struct kvc_merge {
  const void *q;            /* [n_scopes][1][G][head_dim] in the cache dtype */
  int32_t G;
  float scale;
  float eps;                /* guard: |w_e l_e + w_c l_c| < eps falls back to (k_e + k_c)/2 */
  int32_t reserved;
} kvc_merge;

/* ---------------------------------------------------------------------------
 * kvc_decode_attn_score -- append one token, then vote-weighted GQA decode
 * attention and the head-averaged per-token score.
 *
 * KeepKV notes eq. (1) and eq. (6): o_g = sum_i p_i e^{l_{g,i}} v_i / sum_i p_i e^{l_{g,i}},
 * l_{g,i} = scale * q_g . k_i (votes enter as ln p_i added to the logit).
 * InertiaKV §3.1 eq. (1): s(i) = mean over the scope's units*G query heads of
 * a_{g,i} = p_i e^{l_{g,i}} / Z_g.
 *
 * If k_new is non-NULL the new rows (k_new, v_new: [n_scopes][units][head_dim]
 * in the cache dtype) are written at slot len of every scope with vote 1,
 * position t and utility 0, and len is incremented; attention then covers
 * slots [0, len). out: [n_scopes][units][G][head_dim] fp32; lse:
 * [n_scopes][units][G] fp32 (ln Z_g, -inf when Z_g = 0); s: [n_scopes][capacity]
 * fp32 or NULL (only slots < len are written). max_len is a host-side upper
 * bound on the live length after the append, used to size the launch (<= 0:
 * capacity); a device length beyond it is still handled correctly.
 * ------------------------------------------------------------------------- */
int32_t kvc_decode_attn_score(const kvc_cache *cache, const void *k_new, const void *v_new,
                              int32_t t, const void *q, int32_t G, float scale,
                              float *out, float *lse, float *s, int32_t max_len,
                              void *ws, size_t ws_bytes, void *stream);

/* kvc_ema_update -- InertiaKV §3.1 eqs. (2)-(4) on slots [0, len) of every
 * scope: SINGLE m = s; CUMULATIVE m = m + s; EMA m = alpha m + (1 - alpha) s.
 * m, s: [n_scopes][capacity] fp32; len: [n_scopes]. */
int32_t kvc_ema_update(float *m, const float *s, const int32_t *len, int32_t n_scopes,
                       int32_t capacity, int32_t rule, float alpha, void *stream);

/* kvc_select_evict -- InertiaKV §3.1: when a scope holds more than `budget`
 * live entries, the k = len - budget entries of lowest key are evicted;
 * MomentKV Algorithm 1 phase 1 (one at a time) selects the same set when the
 * key does not depend on the evicted set. Ties: (key, pos) ascending, so the
 * lower position goes first; pos NULL uses the slot index. LaProx key design 3
 * (model-wide Top-K) is this call with one scope over the flattened scores and
 * budget = K.
 * key: [n_scopes][capacity] fp32 (finite); len NULL means every slot is live.
 * evict: [n_scopes][capacity] u8, set to 1 on the selected slots and 0 on every
 * other slot < len; n_evict: [n_scopes] int32 or NULL. */
int32_t kvc_select_evict(const float *key, const int32_t *pos, const int32_t *len,
                         int32_t n_scopes, int32_t capacity, int32_t budget,
                         uint8_t *evict, int32_t *n_evict, void *ws, size_t ws_bytes,
                         void *stream);

/* kvc_select_evict_protected -- kvc_select_evict where every entry at a position
 * >= protect_from ranks after every other entry: the order is (protected, key,
 * pos) ascending, so protected entries are evicted only when too few others are
 * left to reach the budget. This is InertiaKV's third lazy-refresh alternative
 * (§3.1, the lazy rule): entries appended since the last score refresh carry no
 * score yet and are protected instead of being evicted on their stale zero
 * utility; protect_from is the position of the first such entry. Positions must
 * be non-negative. pos NULL uses the slot index. One scope of more than 2^20 slots with len NULL (the device-
 * wide path of kvc_select_evict) is KVC_ERR_UNSUPPORTED. Workspace:
 * kvc_select_workspace_size. */
int32_t kvc_select_evict_protected(const float *key, const int32_t *pos, const int32_t *len,
                                   int32_t n_scopes, int32_t capacity, int32_t budget,
                                   int32_t protect_from, uint8_t *evict, int32_t *n_evict,
                                   void *ws, size_t ws_bytes, void *stream);

/* kvc_keep_jaccard -- rank-stability diagnostic (InertiaKV §3.1, the rank-inertia
 * measure of Fig. 1): per scope, the Jaccard similarity |A and B| / |A or B| of two
 * kept sets over the same slots, A = {slots < len with keep_a != 0}, likewise B
 * (1 when both are empty). keep_a, keep_b: [n_scopes][capacity] u8 (e.g. the
 * complement of two kvc_select_evict results on one state under two scorers);
 * len NULL means every slot; out: [n_scopes] fp32. */
int32_t kvc_keep_jaccard(const uint8_t *keep_a, const uint8_t *keep_b, const int32_t *len, int32_t n_scopes,
                         int32_t capacity, float *out, void *stream);

/* kvc_moment_update -- MomentKV §4.1 / Appendix A.1 / Algorithm 1 steps 11-13:
 * for every slot < len flagged in evict (u8 [n_scopes][capacity]), fold its
 * rows into every unit's sums: n += 1, sk += k, sv += v, S += v k^T (fp32).
 * Must run before kvc_compact overwrites the evicted rows. */
int32_t kvc_moment_update(const kvc_cache *cache, const uint8_t *evict, const kvc_moments *mom,
                          void *stream);

/* kvc_moment_correct -- MomentKV normalisation-corrected output (summary page,
 * Algorithm 1 phase 2, §4.2, with the first-order estimate of §4.1). For each
 * unit u (scope-major unit order, as in kvc_moments) and query head g:
 *   if n_e = 0: out = f_R;
 *   else, with k_bar = s_k/n_e, v_bar = s_v/n_e, S_tilde = S - s_v s_k^T/n_e:
 *     Z_E_hat = n_e exp(scale q.k_bar)   (Jensen lower bound of Z_E),
 *     f_E_hat = v_bar + scale S_tilde q / n_e,
 *     w_R = Z_R / (Z_R + Z_E_hat) with Z_R = exp(lse_R),
 *     out = w_R f_R + (1 - w_R) f_E_hat.
 * f_R, lse_R: the attention output and log-partition over the retained set
 * (e.g. kvc_decode_attn_score on the cache after eviction), [n_units][G][128]
 * and [n_units][G] fp32; q: [n_units][G][128] in `dtype` (KVC_BF16 or KVC_F32);
 * out: [n_units][G][128] fp32, may be f_R itself. Arithmetic in float64; the
 * moment matrix must be 16-byte aligned. */
int32_t kvc_moment_correct(const kvc_moments *mom, int32_t n_units, const void *q, int32_t dtype, int32_t G,
                           float scale, const float *f_R, const float *lse_R, float *out, void *stream);

/* kvc_moment_evict -- MomentKV moment-informed eviction (summary page, §4.2
 * "moment residual" and "moment-aware eviction score", Algorithm 1 phase 1),
 * per-KV-head scopes only (units_per_scope = 1, else KVC_ERR_UNSUPPORTED).
 * While a scope holds more than `budget` live entries, every live entry j is
 * scored against the moment model of the evicted set,
 *   r_j = v_j - v_bar - scale S_tilde (k_j - k_bar) / n_e   (r_j = v_j if n_e = 0),
 *   score(j) = alpha_j ||r_j||_2,
 * with k_bar = s_k/n_e, v_bar = s_v/n_e, S_tilde = S - s_v s_k^T/n_e; the
 * lowest score (ties: lower position) is evicted and folded into the sums
 * (n_e += 1, s_k += k, s_v += v, S += v k^T, fp32) before the next one is
 * scored. Do not call kvc_moment_update for these flags again; remove the
 * entries with kvc_compact afterwards.
 * alpha: [n_scopes][capacity] fp32 attention weights of the live entries (e.g.
 * the s of kvc_decode_attn_score after the append; renormalising alpha over
 * the entries left scales every score alike, so it is not redone per round).
 * evict: [n_scopes][capacity] u8, 1 on the evicted slots and 0 on every other
 * slot < len. order: [n_scopes][capacity] int32 or NULL; entry i of a scope
 * receives the slot evicted in round i. score_out: [n_scopes][capacity] fp32
 * or NULL; the first round's scores of slots < len. n_evict: [n_scopes] or NULL.
 * Arithmetic: residuals, norms and scores in float64 (float64 MFMA).
 * Rounds. max_len (<= 0: capacity) bounds the live length on the host; the
 * call runs max(1, max_len - budget) rounds of two kernels, so it is meant for
 * the decode steady state (one eviction per step) and small refresh batches.
 * A scope that needs more rounds than that evicts only as many and sets the
 * workspace status to KVC_ERR_CAPACITY. The moment matrix and the key sums
 * must be 16-byte aligned. Workspace: kvc_moment_evict_workspace_size. */
int32_t kvc_moment_evict(const kvc_cache *cache, const kvc_moments *mom, const float *alpha, float scale,
                         int32_t budget, int32_t max_len, uint8_t *evict, int32_t *order, float *score_out,
                         int32_t *n_evict, void *ws, size_t ws_bytes, void *stream);

/* kvc_keepkv_prefill_merge -- KeepKV prefill compression by greedy all-pairs
 * ZIP merging (reading notes on KeepKV: the inference algorithm's prefill steps
 * 2-5, "candidate choice", eqs. (7), (10), (12) and the numerical-stability
 * guard), per-KV-head scopes only (units_per_scope = 1) of capacity at most
 * 32768 (else KVC_ERR_UNSUPPORTED). While a scope holds more than `budget` live entries,
 * the two entries whose keys have the largest cosine, both at positions below
 * protect_from (the most recent tokens are never merged), are ZIP-merged with
 * the reference logits of merge->q (the mean over its G query heads of
 * scale * q_g . k, recomputed for a merged key) and votes added; the merged
 * rows, rounded to the cache dtype, replace the older entry's rows in its slot
 * (its utility becomes the sum of the two) and the other slot is flagged in
 * evict (u8 [n_scopes][capacity]; 0 on every other slot < len). Remove the
 * flagged slots with kvc_compact (merge NULL). Ties: cosine descending, then
 * the pair's lower position, then its higher one; a zero key has cosine 0.
 * pairs: [n_scopes][capacity][2] int32 or NULL, merge i of a scope as
 * (surviving slot, removed slot); n_merged: [n_scopes] int32 or NULL. votes
 * must be non-NULL. Cosines are float64 (exact products of the cache values).
 * If fewer than two entries may merge before the budget is reached, the scope
 * stops there and the workspace status becomes KVC_ERR_CAPACITY. One
 * workgroup per scope runs the merges in sequence: each merge reads every
 * candidate key once (O(len d)); an entry whose kept partners were all merged
 * away is recomputed (another O(len d), several entries per pass) only when
 * it could take part in the next pair. Workspace:
 * kvc_keepkv_prefill_workspace_size. */
int32_t kvc_keepkv_prefill_merge(const kvc_cache *cache, const kvc_merge *merge, int32_t budget,
                                 int32_t protect_from, uint8_t *evict, int32_t *pairs, int32_t *n_merged,
                                 void *ws, size_t ws_bytes, void *stream);

/* kvc_keepkv_prefill_merge_marked -- kvc_keepkv_prefill_merge, plus stage timing
 * for measurement: events (hipEvent_t handles created by the caller, n_events = 4)
 * are recorded on `stream` before the first kernel and after each of the three
 * (key norms and flags, initial partner lists, the merge loop). events NULL
 * behaves as kvc_keepkv_prefill_merge; n_events other than 4 with events
 * non-NULL is KVC_ERR_ARG. */
int32_t kvc_keepkv_prefill_merge_marked(const kvc_cache *cache, const kvc_merge *merge, int32_t budget,
                                        int32_t protect_from, uint8_t *evict, int32_t *pairs, int32_t *n_merged,
                                        void *ws, size_t ws_bytes, void *stream, void *const *events,
                                        int32_t n_events);

/* kvc_keepkv_refresh -- KeepKV's periodic refresh (reading notes on KeepKV: the
 * inference algorithm's decode step 6g, Figure 4 and the paragraph on periodic
 * refresh): the full KV kept in host memory is loaded back and compressed again,
 * which clears the error the EMA-predicted merges of the decode steps since the
 * last compression have accumulated. Per-KV-head scopes of a bf16 cache
 * (units_per_scope = 1 and capacity <= 32768, else KVC_ERR_UNSUPPORTED; fp32
 * KVC_ERR_DTYPE) with votes and utilities. In stream order:
 *   1. reload: host_k, host_v ([n_scopes][n_tokens][128] bf16, every token so far in
 *      position order) and host_pos ([n_scopes][n_tokens] int32, increasing) are
 *      copied into slots [0, n_tokens) of every scope; those slots get vote 1 and
 *      the live length becomes n_tokens (whatever the cache held before);
 *   2. the utility of every reloaded token is restarted with eq. (15)'s window
 *      form, as kvc_keepkv_ema_init computes it, from q_win ([n_scopes][G][n_win]
 *      [128] bf16, the queries of the last n_win steps, row j standing at the
 *      position of slot n_tokens - n_win + j) and alpha;
 *   3. greedy ZIP merging down to `budget`, as kvc_keepkv_prefill_merge does it,
 *      with the exact group-mean logits of merge->q (the current step's G query
 *      heads, [n_scopes][G][128] bf16) under merge->scale, which step 2 uses too;
 *      entries at positions >= protect_from never merge;
 *   4. the merged-away slots are removed (hole filling, as kvc_compact).
 * pairs ([n_scopes][capacity][2] int32) and n_merged ([n_scopes] int32), or NULL,
 * receive the merges as kvc_keepkv_prefill_merge reports them (slots before step 4).
 * The host buffers should be pinned (hipHostMalloc) for the copies to run
 * asynchronously; they must stay valid until the stream reaches this call's end.
 * A scope that cannot reach its budget stops above it and the workspace status
 * (its first word) becomes KVC_ERR_CAPACITY. 0 < alpha < 1, else KVC_ERR_ARG;
 * 0 < n_win <= n_tokens <= capacity and budget >= 0, else KVC_ERR_CAPACITY.
 * Workspace: kvc_keepkv_refresh_workspace_size, zero-filled once. */
int32_t kvc_keepkv_refresh(const kvc_cache *cache, const void *host_k, const void *host_v, const int32_t *host_pos,
                           int32_t n_tokens, const void *q_win, int32_t n_win, const kvc_merge *merge, float alpha,
                           int32_t budget, int32_t protect_from, int32_t *pairs, int32_t *n_merged, void *ws,
                           size_t ws_bytes, void *stream);

/* kvc_keepkv_refresh_marked -- kvc_keepkv_refresh, plus stage timing for
 * measurement: events (hipEvent_t handles created by the caller, n_events = 5) are
 * recorded on `stream` before the reload and after each of its four steps. events
 * NULL behaves as kvc_keepkv_refresh; n_events other than 5 with events non-NULL is
 * KVC_ERR_ARG. */
int32_t kvc_keepkv_refresh_marked(const kvc_cache *cache, const void *host_k, const void *host_v,
                                  const int32_t *host_pos, int32_t n_tokens, const void *q_win, int32_t n_win,
                                  const kvc_merge *merge, float alpha, int32_t budget, int32_t protect_from,
                                  int32_t *pairs, int32_t *n_merged, void *ws, size_t ws_bytes, void *stream,
                                  void *const *events, int32_t n_events);

/* kvc_keepkv_ema_init -- KeepKV's window initialisation of the EMA utility at the
 * end of prefill (reading notes on KeepKV: EMA score prediction, eq. (15) at t = L,
 * and the inference algorithm's prefill step 4), per-KV-head scopes of a bf16 cache
 * (units_per_scope = 1, else KVC_ERR_UNSUPPORTED; fp32 caches KVC_ERR_DTYPE).
 * Slots [0, n_tokens) of every scope hold the prompt in position order; q_win
 * ([n_scopes][G][n_win][128] bf16, 16-byte aligned) holds the queries of the last
 * n_win prompt tokens, window row j at position n_tokens - n_win + j. For each
 * row, s_j(i) is the mean over the G query heads of the softmax weight of key i
 * under scale * q . k, causal (keys i <= the row's position; 0 beyond). Writes
 * m[s][i] = sum_j (1 - alpha) alpha^(n_win - 1 - j) s_j(i) for i < n_tokens (the
 * page's w is n_win - 1); other slots are untouched. This equals the EMA recursion
 * m <- alpha m + (1 - alpha) s run from zero over the window rows. The bias-
 * corrected prediction m / (1 - alpha^t) is kvc_ema_predict. Logits and softmax statistics
 * are float64 (fp64 MFMA), weights and m fp32. 0 < alpha < 1, else KVC_ERR_ARG;
 * 0 < n_win <= n_tokens <= capacity, else KVC_ERR_CAPACITY. Workspace:
 * kvc_keepkv_ema_init_workspace_size. */
int32_t kvc_keepkv_ema_init(const kvc_cache *cache, const void *q_win, int32_t G, int32_t n_win, int32_t n_tokens,
                            float scale, float alpha, void *ws, size_t ws_bytes, void *stream);

/* kvc_ema_predict -- KeepKV notes, EMA score prediction eq. (14): the
 * bias-corrected predicted score out = m / (1 - alpha^t) of an EMA state m that
 * has taken t updates from zero (eq. (15); t counts the window rows of
 * kvc_keepkv_ema_init plus the decode steps since). The factor is formed in
 * float64; every entry of a step is scaled alike, so rankings are unchanged.
 * m, out: [n_scopes][capacity] fp32 (out may equal m); len: [n_scopes] or NULL
 * (every slot): slots [0, len) are written, others untouched. 0 < alpha < 1 and
 * t >= 1, else KVC_ERR_ARG. */
int32_t kvc_ema_predict(const float *m, const int32_t *len, int32_t n_scopes, int32_t capacity, float alpha,
                        int32_t t, float *out, void *stream);

/* kvc_keepkv_ema_init_marked -- kvc_keepkv_ema_init, plus stage timing for
 * measurement: events (hipEvent_t handles created by the caller, n_events = 5)
 * are recorded on `stream` before the first kernel and after each of the four
 * (window pass 1, row combine, window pass 2, sum over window-row blocks). events
 * NULL behaves as kvc_keepkv_ema_init; n_events other than 5 with events non-NULL
 * is KVC_ERR_ARG. */
int32_t kvc_keepkv_ema_init_marked(const kvc_cache *cache, const void *q_win, int32_t G, int32_t n_win,
                                   int32_t n_tokens, float scale, float alpha, void *ws, size_t ws_bytes,
                                   void *stream, void *const *events, int32_t n_events);

/* kvc_compact -- remove the flagged entries of every scope (MomentKV Algorithm 1
 * step 14; InertiaKV §3: eviction is irreversible). Survivors end in slots
 * [0, len - n_evicted): the j-th evicted slot below the new length receives the
 * j-th surviving slot at or above it (rows of every unit, vote, position and
 * utility move together; slot order is not preserved). len is updated.
 * With merge non-NULL the cache must carry votes (KVC_ERR_ARG otherwise: the
 * merged entry's vote p_e + p_c has to be stored) and each scope at most one
 * flagged entry e (per-head scopes only; a scope with several flags is left
 * untouched and the workspace status word becomes KVC_ERR_UNSUPPORTED); e is
 * first ZIP-merged into the live entry c of largest
 * cos(k_e, k_c) (ties to the lower position): KeepKV eqs. (7), (10), (12):
 * v_c <- (w_e v_e + w_c v_c)/(w_e + w_c), k_c <- eq. (12) with the guard,
 * p_c <- p_e + p_c, m_c <- m_e + m_c, with w_x = p_x e^{l_x}. Merged rows are
 * rounded to the cache dtype (nearest even). */
int32_t kvc_compact(const kvc_cache *cache, const uint8_t *evict, const kvc_merge *merge,
                    void *ws, size_t ws_bytes, void *stream);

/* kvc_decode_step -- the whole decode step, in the order
 * append -> attend -> score -> utility -> select -> fold -> compact
 * (MomentKV Algorithm 1; KeepKV decode steps 6a-6f; InertiaKV §3.1), with the
 * semantics of kvc_decode_attn_score, kvc_ema_update, kvc_select_evict,
 * kvc_moment_update and kvc_compact applied in turn. refresh = 0 skips the
 * score and utility update for this step (lazy refresh: eviction still holds
 * the budget with the stale utility; the appended entry has utility 0).
 * Ranking: the step computes scores and utilities in float64 and selects on
 * (float64 utility, position) ascending before the utilities are stored as
 * fp32, so entries whose utilities lie below float32's range (stored as 0)
 * are still ranked by their float64 values; the selection of kvc_select_evict
 * ranks the fp32 keys it is given.
 * mom NULL skips the fold. evict_out: [n_scopes][capacity] u8 or NULL; when
 * given it receives the flags of the evicted slots as they were before
 * compaction. s may be NULL. Merge mode is kvc_compact's (merge non-NULL; it
 * needs votes, KVC_ERR_ARG otherwise, and one eviction per scope and step).
 *
 * Attention group. Only units [attn_unit0, attn_unit0 + attn_units) of each
 * scope attend and score in this call (attn_units <= 0: every unit); q, out and
 * lse are then [n_scopes][attn_units][G][head_dim] ([..][G] for lse), while
 * the append (k_new, v_new: every unit), the fold and the compaction act on
 * every unit of the scope. This is how one slot set shared by all layers of a
 * sequence is driven layer by layer (InertiaKV §3.1: the utility is updated
 * after every compressed layer); a call whose scope is already within budget
 * only attends, scores and updates the utility. A call with budget >= capacity
 * cannot evict; without an append, evict_out or merge its selection launch is
 * skipped (the later layers of a model-scope step, after the first layer has
 * evicted to the budget).
 *
 * Launches. max_len <= budget + 1 (at most one eviction per scope, the steady
 * state) runs the whole step in one launch. A larger max_len (e.g. the first
 * step after prefill, which compresses to the budget) adds a fixed sequence
 * of device-wide kernels for the scopes that evict more than one entry:
 * radix select, flags, lists, moment fold and row moves; scopes that evict
 * at most one entry finish inside the first launch and the later kernels
 * skip them. */
int32_t kvc_decode_step(const kvc_cache *cache, const void *k_new, const void *v_new, int32_t t,
                        const void *q, int32_t G, float scale, int32_t rule, float alpha,
                        int32_t budget, int32_t refresh, float *out, float *lse, float *s,
                        const kvc_moments *mom, const kvc_merge *merge, uint8_t *evict_out,
                        int32_t attn_unit0, int32_t attn_units, int32_t max_len,
                        void *ws, size_t ws_bytes, void *stream);

/* kvc_decode_groups -- InertiaKV §3.1 (one slot set per sequence shared by
 * every layer, the utility updated after every compressed layer) for the
 * layers of a model-scope step that come after the one that evicted: n_groups
 * consecutive attention groups of group_units units each, units
 * [unit0, unit0 + n_groups * group_units) of every scope, attend over the live
 * entries, score, and update the shared utility group after group, as
 * n_groups calls of kvc_decode_step without append, flags or merge and with a
 * budget no smaller than the live length (attn_unit0 = unit0 + j * group_units,
 * attn_units = group_units, j = 0 .. n_groups - 1) would -- but in three
 * launches for all the groups, with the utility chain in closed form:
 *   single      m = s_{n-1}
 *   cumulative  m = m + sum_j s_j
 *   EMA         m = alpha^n m + sum_j (1 - alpha) alpha^(n-1-j) s_j
 * evaluated in float64 and stored once as float32 (the calls it replaces
 * store m after every group). s_j is group j's head-averaged score (the mean
 * over its group_units * G heads of the vote-weighted attention weights).
 * Nothing is appended, selected or moved; a scope's live length is whatever
 * len holds. q: [n_scopes][n_groups * group_units][G][head_dim] in the cache
 * dtype; out: the same shape, fp32; lse: [n_scopes][n_groups * group_units][G]
 * fp32; s: [n_scopes][capacity] fp32 or NULL, receives the last group's scores
 * (slots < len). refresh == 0 (a lazy step) attends only: m and s are left as
 * they are. max_len (<= 0: capacity) sizes the launches; a longer device
 * length is still covered. Workspace: kvc_decode_workspace_size(cache, G, 0)
 * is enough. Errors: KVC_ERR_ARG for a unit range outside the scope, bad
 * pointers or rule, or refresh without utilities; KVC_ERR_UNSUPPORTED for
 * group_units * G > 64, or n_groups * group_units * G above 4096 (bf16 caches)
 * or 2048 (fp32). */
int32_t kvc_decode_groups(const kvc_cache *cache, const void *q, int32_t G, float scale, int32_t rule,
                          float alpha, int32_t refresh, int32_t unit0, int32_t n_groups, int32_t group_units,
                          float *out, float *lse, float *s, int32_t max_len, void *ws, size_t ws_bytes,
                          void *stream);

/* kvc_decode_plan -- the kernels a call with these shapes runs, without running
 * it: kvc_decode_step (step != 0, with this budget, merge != 0 for a call with a
 * merge descriptor) or kvc_decode_attn_score (step == 0; budget and merge
 * ignored) on `cache` with group size G and max_len (<= 0: capacity). Returns
 *   KVC_PLAN_ONE_LAUNCH: one workgroup per scope does the whole step in one
 *     launch (single-unit scopes, at most one eviction per scope, the per-token
 *     state of max_len tokens fits in LDS, and either at least 128 scopes or at
 *     most 256 KiB of K and V rows per scope);
 *   KVC_PLAN_SPLIT: split-K attention, then the score and finish kernels;
 *   KVC_PLAN_SPLIT_BULK: KVC_PLAN_SPLIT plus the device-wide eviction kernels
 *     (max_len > budget + 1, no merge);
 * or the (negative) error code the call would return for these shapes. Host
 * only: reads the device's LDS size, enqueues nothing. */
enum { KVC_PLAN_ONE_LAUNCH = 1, KVC_PLAN_SPLIT = 2, KVC_PLAN_SPLIT_BULK = 3 };
int32_t kvc_decode_plan(const kvc_cache *cache, int32_t G, int32_t step, int32_t merge, int32_t budget,
                        int32_t max_len);

/* kvc_decode_step_noalloc -- kvc_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments and results, with the workspace
 * replaced by a scratch array of KVC_NOALLOC_SCRATCH_BYTES (128 MiB) that the
 * library's code object holds on each GPU it runs on, for the life of the
 * process. The call allocates nothing (no hipMalloc, no allocating library
 * routine); its first call on a device looks up that device's array.
 * A cache whose decode workspace (kvc_decode_workspace_size) exceeds the scratch
 * size is rejected with KVC_ERR_WORKSPACE before anything is enqueued. status:
 * a caller-owned device int32 that receives the device-detected condition a
 * workspace status word would (KVC_ERR_CAPACITY when a live length exceeds the
 * capacity; the caller zeroes and reads it), or NULL (the condition is then not
 * reported). Every call on one GPU shares that GPU's scratch: calls that can
 * overlap on one GPU (different streams, or different host threads) race and
 * must be serialised by the caller. */
#define KVC_NOALLOC_SCRATCH_BYTES (128u << 20)
int32_t kvc_decode_step_noalloc(const kvc_cache *cache, const void *k_new, const void *v_new, int32_t t,
                                const void *q, int32_t G, float scale, int32_t rule, float alpha,
                                int32_t budget, int32_t refresh, float *out, float *lse, float *s,
                                const kvc_moments *mom, const kvc_merge *merge, uint8_t *evict_out,
                                int32_t attn_unit0, int32_t attn_units, int32_t max_len, int32_t *status,
                                void *stream);

/* kvc_laprox_score -- LaProx prefill score (key design 1), per-layer
 * normalisation (key design 2) and GQA group mean (training-strategy paragraph).
 * For layer l, KV head h, token i < N:
 *   c_i = || mean_{g in group(h)} A_g[:, i] ||_2 over the w window rows, where
 *         window row j sits at position N - w + j and A_g[j, :] is the causal
 *         softmax of scale * q_{g,j} . k_i over i <= N - w + j;
 *   r_i = || v_i W_bar_h ||_2, W_bar_h = sum_{g in group(h)} W_O^g (d x D),
 *         computed as r_i^2 = v_i M_h v_i^T with M_h = W_bar_h W_bar_h^T
 *         (d x d), both on float64 MFMA;
 *   score[l][h][i] = c_i r_i / sum_{h', i'} c_{i'} r_{i'} over layer l.
 * q_win: [n_layers][H][w][d] bf16; k, v: [n_layers][n_kv][N][d] bf16;
 * w_o: [n_layers][H][d][D] bf16; score: [n_layers][n_kv][N] fp32.
 * Shapes: d = 128, G = H / n_kv in {1, 2, 4, 8}, G*w a multiple of 8,
 * 0 < w <= N, D a multiple of 64 (KVC_ERR_UNSUPPORTED otherwise). Logits,
 * W_bar, M_h and r_i^2 are float64.
 * The model-wide Top-K (key design 3) is kvc_select_evict on score with one
 * scope of n_layers*n_kv*N entries and budget K. */
int32_t kvc_laprox_score(const void *q_win, const void *k, const void *v, const void *w_o,
                         int32_t n_layers, int32_t H, int32_t n_kv, int32_t N, int32_t w,
                         int32_t d, int32_t D, float scale, float *score,
                         void *ws, size_t ws_bytes, void *stream);

/* kvc_laprox_score_marked -- kvc_laprox_score, plus stage timing for
 * measurement: events (hipEvent_t handles created by the caller, n_events = 8)
 * are recorded on `stream` before the first kernel and after each of the seven
 * stages (Gram matrices W_bar W_bar^T, window pass 1, row combine, window pass
 * 2, value-output norms v M v^T, product, normalisation). events NULL behaves as
 * kvc_laprox_score;
 * n_events other than 8 with events non-NULL is KVC_ERR_ARG. */
int32_t kvc_laprox_score_marked(const void *q_win, const void *k, const void *v, const void *w_o,
                                int32_t n_layers, int32_t H, int32_t n_kv, int32_t N, int32_t w,
                                int32_t d, int32_t D, float scale, float *score, void *ws,
                                size_t ws_bytes, void *stream, void *const *events, int32_t n_events);

/* Workspace sizes in bytes. The decode and compact workspaces must be zero-filled once
 * before their first use (their first word is the device status word, see
 * kvc_workspace_status); every other byte is written by a call before that
 * call reads it, so one workspace can serve any number of calls on one
 * stream (concurrent calls need separate workspaces). */
size_t kvc_decode_workspace_size(const kvc_cache *cache, int32_t G, int32_t max_len);
size_t kvc_select_workspace_size(int32_t n_scopes, int32_t capacity);
size_t kvc_compact_workspace_size(const kvc_cache *cache);
size_t kvc_moment_evict_workspace_size(const kvc_cache *cache);
size_t kvc_keepkv_prefill_workspace_size(const kvc_cache *cache);
size_t kvc_keepkv_ema_init_workspace_size(const kvc_cache *cache, int32_t G, int32_t n_win, int32_t n_tokens);
size_t kvc_keepkv_refresh_workspace_size(const kvc_cache *cache, int32_t G, int32_t n_win, int32_t n_tokens);
size_t kvc_laprox_workspace_size(int32_t n_layers, int32_t H, int32_t n_kv, int32_t N, int32_t w,
                                 int32_t d, int32_t D);

/* Synchronises `stream`, returns the device status word of a workspace
 * (KVC_OK or KVC_ERR_CAPACITY when a device length exceeded its capacity)
 * and clears it. */
int32_t kvc_workspace_status(void *ws, void *stream);

const char *kvc_status_string(int32_t status);

/* kvc_read_probe -- measurement aid, not part of the method: reads the first
 * bytes / 16 16-byte vectors of buf (device memory, 16-byte aligned) once, each
 * of `workgroups` workgroups (256 threads) one contiguous share with 8 loads in
 * flight per thread (reverse != 0: each share from its end), and writes one
 * word per workgroup to sink[workgroups]. Timing it gives the streaming-read
 * rate a plain kernel attains on the device, the ceiling the decode kernels are
 * compared with beside the published HBM peak. KVC_ERR_ARG for null pointers,
 * workgroups <= 0 or bytes < 16; KVC_ERR_ALIGN for an unaligned buf. */
int32_t kvc_read_probe(const void *buf, size_t bytes, int32_t workgroups, int32_t reverse, uint32_t *sink,
                       void *stream);

/* Synchronises `stream` and reports an asynchronous device error of the work queued
 * on it: KVC_ERR_DEVICE if the stream (or an earlier launch) failed, else KVC_OK. */
int32_t kvc_check(void *stream);
int32_t kvc_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KVC_H */
