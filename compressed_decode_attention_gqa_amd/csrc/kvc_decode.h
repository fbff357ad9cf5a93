// Launch arguments of the fused decode-step kernel (host and device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

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
  int32_t *status, *counters;
  double *partM, *partZ;
  float *partO, *fac;
  double *subM;
  float *ews;
  uint8_t *flags;
  int32_t *list, *list2;
  int32_t n_splits, nsub_cap;
  int32_t lds_len;   // per-scope kernel: live tokens its LDS holds (at most budget + 1)
};

int decode_chunk_tokens(int dtype);
int decode_unit_chunk_tokens(int dtype);
hipError_t launch_decode(const StepArgs &a, int dtype, int G, hipStream_t st);
hipError_t launch_decode_unit(const StepArgs &a, int dtype, int G, hipStream_t st);
// LDS (static + dynamic) of the per-scope kernel for lds_len live tokens
size_t decode_unit_lds_bytes(int dtype, int G, int lds_len, bool votes);

}  // namespace kvc
