// LaProx prefill scoring: launch interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvc {

// Shapes the kernels take: G = H / n_kv in {1, 2, 4, 8}, G w a multiple of 8,
// 0 < w <= N, D a positive multiple of 64 (head_dim is 128).
bool laprox_shape_supported(int H, int n_kv, int N, int w, int D);
size_t laprox_workspace_bytes(int n_layers, int H, int n_kv, int N, int w, int d, int D);
// marks: NULL, or 8 events recorded on st before the first kernel and after each
// of the seven (Gram matrix W_bar W_bar^T, window pass 1, row combine, window
// pass 2, value-output norms v M v^T, product, normalisation).
constexpr int kLaproxStages = 7;
hipError_t launch_laprox(const void *q_win, const void *k, const void *v, const void *w_o, int n_layers,
                         int H, int n_kv, int N, int w, int D, double scale, float *score, void *ws,
                         hipStream_t st, hipEvent_t *marks);

}  // namespace kvc
