// Launch arguments of the fused decode-step kernel (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

// Per-scope state of a device-wide eviction of k > 1 entries (the bulk path:
// radix select, evicted and mover lists, split fold and row moves run as
// separate grid-wide kernels after the attention kernel).
struct BulkScope {
  uint64_t prefix, mask;   // cut on the 64-bit key (see the flags kernel)
  uint32_t lprefix, lmask; // cut on the 32-bit tie key (positions) when 64-bit keys tie
  int32_t krem;            // rank of the k-th smallest key inside the current bin
  int32_t done;            // the cut is final
  int32_t L, k;            // live length before eviction, evicted count
  int32_t B;               // survivors at or above B move into the evicted slots below it
  int32_t n_pairs;         // hole-filling moves
  int32_t run;             // the grid-wide kernels act on this scope
  int32_t pad;
};

struct BulkArgs {
  BulkScope *st;           // [n_scopes]
  uint32_t *hpart;         // [n_scopes][n_chunks][256] radix histogram of each chunk (current pass)
  int32_t *cnt;            // [n_scopes][n_chunks][2]: evicted slots, movers
  float *fpart;            // [n_scopes * units][fold_splits][HD*HD + 2*HD] fold partials (fold_splits > 1)
  const float *key;        // selection keys [n_scopes][cap] and positions (null: the slot index)
  const int32_t *pos;
  const double *key64;     // non-null: float64 keys [n_scopes][cap] ranked as (key64, position)
  uint8_t *flags, *flags2; // [n_scopes][cap] evicted flags (selection writes both, if non-null)
  int32_t *list, *list2;   // [n_scopes][cap]: evicted slots ascending; movers ascending
  const int32_t *len;      // live lengths for the standalone paths (null: cap)
  int32_t *n_evict;        // [n_scopes] or null
  int32_t cap, budget, n_scopes;
  int32_t n_chunks, chunk; // slot chunks of the histogram, flag, count and list kernels
  int32_t fold_splits;     // workgroups folding one unit's evicted rows
  int32_t move_blocks;     // workgroups moving one scope's rows
  int32_t protect;         // 1: entries at positions >= protect_from rank after every other entry
  int32_t protect_from;
};

struct StepArgs {
  // cache (scope of `units` units; attention covers units [attn_unit0, attn_unit0 + attn_units))
  char *k, *v;
  int32_t *votes, *pos;
  float *m;
  int32_t *len;
  int64_t scope_stride, unit_stride;
  int32_t capacity, n_scopes, units, attn_unit0, attn_units;
  // step inputs
  const char *k_new, *v_new;
  int32_t t, append;
  const char *q;
  double scale;
  // outputs
  float *out, *lse, *s;
  // step semantics: mode 0 attend (+ score), 1 full step, 2 full step without compaction
  int32_t mode, rule, budget, refresh;
  float alpha;
  int32_t *mom_n;
  float *mom_sk, *mom_sv, *mom_S;
  uint8_t *evict_out;
  // workspace
  int32_t *status;
  double *partM, *partZ;
  float *partO, *fac;
  double *subM;
  float *ews;
  uint8_t *ewsh;     // shift counts of the stored weights (exp_shifted), beside ews
  double *m64;       // float64 utilities of scopes that evict more than one entry [n_scopes][cap]
  uint8_t *flags;
  int32_t *list, *list2;
  int32_t n_splits, nsub_cap;
  int32_t lds_len;   // per-scope kernel: live tokens its LDS holds (at most budget + 1)
  int32_t row_bytes; // bytes of one K (or V) row
  int32_t max_len;   // live length the launch is sized for (a longer device length is still handled)
  // split path: score chunks and each chunk's lowest (m, pos) key
  int32_t score_chunk, n_score_chunks;   // tokens per chunk; chunks per scope the arrays hold
  uint64_t *cand_key;       // orderable float64 utility of each chunk's lowest entry
  int32_t *cand_slot, *cand_pos;
  BulkScope *bulk;   // non-null: scopes evicting k > 1 stop after the utility update
  // per-unit kernel over attention groups: per-token head-summed attention weights
  // (vote-weighted) of unit gu at wsum[gu * wsum_stride + i]
  double *wsum;
  int32_t wsum_stride;
  // split path in merge mode: the merge kernels take the selection from the chunk
  // candidates, so no finish kernel runs (no flags reported, no moments folded)
  int32_t merge_select;
  // finish workgroups per scope (> 1: multi-unit scopes without moments, the hole
  // fill's rows spread over them) and the live length the score kernel saw
  int32_t fin_blocks;
  int32_t *steplen;
};

int decode_chunk_tokens(int dtype);
int decode_unit_chunk_tokens(int dtype);
hipError_t launch_decode(const StepArgs &a, int dtype, int G, hipStream_t st);
hipError_t launch_decode_unit(const StepArgs &a, int dtype, int G, hipStream_t st);
// The per-scope kernel with one workgroup per attention unit of every scope
// (a.attn_units of them), attending only: o, lse and the per-token weight sums.
hipError_t launch_decode_unit_groups(const StepArgs &a, int dtype, int G, hipStream_t st);
// LDS (static + dynamic) of the per-scope kernel for lds_len live tokens
size_t decode_unit_lds_bytes(int dtype, int G, int lds_len, bool votes);
size_t decode_unit_groups_lds_bytes(int dtype, int G, int lds_len, bool votes);
// Device-wide select -> flags -> lists -> fold -> moves for the scopes the
// epilogue handed over (BulkScope::k > 1).
hipError_t launch_bulk(const StepArgs &a, const BulkArgs &b, int dtype, hipStream_t st);
size_t bulk_part_floats();   // floats of one fold partial
// Standalone entry points on the same grid-wide kernels (BulkArgs: key/pos,
// flags, lists, len, budget, n_evict and the chunking filled by the caller).
hipError_t launch_bulk_select(const BulkArgs &b, hipStream_t st);
hipError_t launch_bulk_compact(const StepArgs &a, const BulkArgs &b, int dtype, hipStream_t st);

}  // namespace kvc
