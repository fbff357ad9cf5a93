// KeepKV periodic refresh, device side of the reload (reading notes on KeepKV:
// the inference algorithm's decode step 6g and Figure 4): after the full KV rows
// and positions are copied from host memory into slots [0, n) of every scope,
// every reloaded entry gets vote 1 and the scope's live length becomes n. The
// EMA window initialisation, the greedy ZIP merging and the compaction that
// follow are the prefill kernels.
#include <algorithm>

#include "kvc_device.h"
#include "kvc_kernels.h"

namespace kvc {

namespace {

__global__ __launch_bounds__(WG) void k_reload_slots(int32_t *votes, int32_t *len, int n, int cap) {
  const int scope = blockIdx.y;
  if (votes) {
    int32_t *vrow = votes + int64_t(scope) * cap;
    for (int i = blockIdx.x * WG + threadIdx.x; i < n; i += gridDim.x * WG) vrow[i] = 1;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) len[scope] = n;
}

}  // namespace

hipError_t launch_reload_slots(int32_t *votes, int32_t *len, int n_scopes, int n, int cap, hipStream_t st) {
  const int blocks = std::max(1, std::min(64, (n + WG - 1) / WG));
  hipLaunchKernelGGL(k_reload_slots, dim3(blocks, n_scopes), dim3(WG), 0, st, votes, len, n, cap);
  return hipGetLastError();
}

}  // namespace kvc
