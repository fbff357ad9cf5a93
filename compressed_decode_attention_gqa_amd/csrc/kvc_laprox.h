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

// KeepKV's window initialisation of the EMA utility on the same window passes: for every unit
// (a KV head with G query heads, keys at k + u kstride rows), the w window queries
// q_win[u][g][j] at positions N - w + j (causal over keys [0, N)) give the group-mean softmax
// weights s_j; m[u m_stride + i] = sum_j (1 - alpha) alpha^(w - 1 - j) s_j(i) for i < N.
// marks: NULL, or 5 events (before the first kernel and after each of the four).
constexpr int kEmaStages = 4;
size_t ema_window_workspace_bytes(int units, int G, int N, int w);
hipError_t launch_ema_window(const void *q_win, const void *k, int64_t kstride, int units, int G, int w, int N,
                             double scale, double alpha, float *m, int64_t m_stride, void *ws, hipStream_t st,
                             hipEvent_t *marks);

}  // namespace kvc
