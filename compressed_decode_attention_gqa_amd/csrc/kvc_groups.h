// Launch arguments of the multi-group decode call: consecutive attention groups
// of a scope (the layers after the first of a model-scope step) that attend,
// score and update the shared utility without evicting.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_decode.h"

namespace kvc {

struct GroupsArgs {
  int32_t n_scopes;
  int32_t units;          // attention units per scope in the call (n_groups * group_units)
  int32_t group_units, n_groups;
  int32_t capacity, n_splits, nsub_cap;
  int32_t max_len;        // live-length bound the score grid is sized for (longer lengths are strided)
  const int32_t *len, *votes;
  float *m, *s, *out, *lse;
  double *partM, *partZ;  // split partials; the combine leaves M and 1/Z in split 0's entries
  const float *partO;
  const double *subM;
  const float *ews;
  const uint8_t *ewsh;
  const double *wsum;     // per-unit kernel path: per-token head sums [gu][wsum_stride] (null: split path)
  int32_t wsum_stride;
  int32_t rule;
  double alpha;
};

// Tokens per score workgroup and the dynamic LDS of the score kernel.
int groups_score_chunk(int dtype);
size_t groups_score_lds_bytes(int dtype, int G, int units);

// Split-K attention only (k_decode_split over a.attn_units units of every scope).
hipError_t launch_decode_attention(const StepArgs &a, int dtype, int G, hipStream_t st);
// Per attention head: M, Z, lse and the output over the split partials; then
// (score) the groups' scores and the closed-form utility update.
hipError_t launch_groups_epilogue(const GroupsArgs &g, int dtype, int G, bool score, hipStream_t st);
// After the per-unit kernel (which wrote o, lse and wsum): the groups' scores and
// the closed-form utility update.
hipError_t launch_groups_wscore(const GroupsArgs &g, int G, hipStream_t st);

}  // namespace kvc
