// Launch arguments and launchers of the standalone entry-point kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

struct CacheArgs {
  char *k, *v;
  int32_t *votes, *pos;
  float *m;
  int32_t *len;
  int64_t scope_stride, unit_stride;
  int32_t dtype, capacity, n_scopes, units;
};

struct MergeArgs {
  const int32_t *e_slot;    // entry to merge per scope at e_slot[scope * e_stride] (-1: none), or
  int64_t e_stride;         // null: the single flagged slot of the evict flags
  const char *q;
  int32_t G;
  double scale;
  float eps;
  int32_t n_splits;
  double *part_cos;
  int32_t *part_slot;       // (slot, position) of each range's partner
  int32_t *status;          // set to -3 for a scope with several flagged entries (standalone path) or
                            // more than one entry over the budget, -4 for a length over the capacity
  // Non-null: the merge kernels take the decode step's selection themselves (no finish ran):
  // the live length is len + append, and a scope then one entry over `budget` merges the entry
  // of the lowest (utility, position) key over the score kernel's chunk candidates.
  const uint64_t *cand_key;
  const int32_t *cand_slot, *cand_pos;
  int32_t n_score_chunks, score_chunk, append, budget;
  int32_t cand_max;         // chunks of the live-length bound the launch was sized for (loaded at entry)
};

struct MomentArgs {
  const int32_t *n;
  const float *sk, *sv, *S;
};

// MomentKV moment-informed eviction on per-KV-head scopes (one unit per scope).
struct MomentEvictArgs {
  const char *k, *v;
  int64_t scope_stride;
  const int32_t *pos, *len;
  int32_t *mom_n;
  float *sk, *sv, *S;
  const float *alpha;
  double scale;
  int32_t capacity, n_scopes, budget, rounds;
  int32_t n_chunks;         // candidate stride per scope
  int32_t n_chunks_used;    // chunks launched per scope
  int32_t chunk;            // tokens per chunk (a multiple of 64)
  int32_t fused_pick;       // chunk >= capacity: the score kernel picks and folds
  uint8_t *evict;
  int32_t *order, *n_evict;
  float *score_out;
  double *cand_score;
  int32_t *cand_pos, *cand_slot;
  int32_t *status;
};

// KeepKV prefill compression by greedy all-pairs ZIP merging (per-KV-head scopes).
// Candidates per scope that the prefill merging loop keeps listed in LDS.
constexpr int PREFILL_MAX_ROWS = 32768;

struct PrefillMergeArgs {
  char *k, *v;
  int64_t scope_stride;
  int32_t *votes, *pos, *len;
  float *m;
  const char *q;            // [n_scopes][G][head_dim] in the cache dtype
  int32_t G;
  double scale;
  float eps;
  int32_t capacity, n_scopes, budget, protect_from;
  uint8_t *evict;
  int32_t *pairs, *n_merged;
  void *meta;               // [n_scopes][capacity] 16 bytes: key norm (float64), position, candidate flag
  void *rec;                // [n_scopes][capacity] 64-byte partner lists: 4 x (cosine, slot, position)
  void *sum;                // [n_scopes][capacity] 32-byte row summaries the merge loop reads per pass
  int32_t *status;
};

size_t wide_state_bytes();
// One scope of more than 2^20 keys (len = NULL): a device-wide radix select.
hipError_t launch_select_wide(const float *key, const int32_t *pos, int cap, int budget, uint8_t *evict,
                              int32_t *n_evict, void *ws, hipStream_t st);
hipError_t launch_moment_update(const CacheArgs &c, const uint8_t *evict, int32_t *n, float *sk,
                                float *sv, float *S, hipStream_t st);
hipError_t launch_moment_update_mfma(const CacheArgs &c, const uint8_t *evict, int32_t *n, float *sk, float *sv,
                                     float *S, hipStream_t st);
hipError_t launch_merge(const CacheArgs &c, const uint8_t *evict, const MergeArgs &mg, hipStream_t st);
hipError_t launch_moment_correct(const MomentArgs &m, int n_units, const void *q, int dtype, int G, double scale,
                                 const float *f_R, const float *lse_R, float *out, hipStream_t st);
// marks: NULL, or 4 events recorded before the first kernel and after each of the three.
hipError_t launch_prefill_merge(const PrefillMergeArgs &p, int dtype, hipStream_t st, hipEvent_t *marks);

// Periodic refresh: vote 1 on slots [0, n) of every scope and live length n.
hipError_t launch_reload_slots(int32_t *votes, int32_t *len, int n_scopes, int n, int cap, hipStream_t st);
hipError_t launch_moment_evict(const MomentEvictArgs &p, int dtype, int rounds, hipStream_t st);
hipError_t launch_ema_update(float *m, const float *s, const int32_t *len, int n_scopes, int cap,
                             int rule, float alpha, hipStream_t st);
hipError_t launch_ema_predict(const float *m, const int32_t *len, int n_scopes, int cap, float alpha, int t,
                              float *out, hipStream_t st);
// Streaming-read probe (measurement aid).
hipError_t launch_read_probe(const void *buf, size_t bytes, int workgroups, int reverse, uint32_t *sink,
                             hipStream_t st);
hipError_t launch_jaccard(const uint8_t *a, const uint8_t *b, const int32_t *len, int n_scopes, int cap, float *out,
                          hipStream_t st);

}  // namespace kvc
