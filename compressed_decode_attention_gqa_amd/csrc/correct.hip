// MomentKV normalisation-corrected output (summary page, Algorithm 1 phase 2
// and §4.2, with the first-order estimate of §4.1): per unit, the retained
// attention output f_R of each query head is mixed with the moment estimate
// of the evicted part,
//   f_E_hat = v_bar + tau (S q - s_v (s_k . q) / n_e) / n_e,
//   ln Z_E_hat = ln n_e + tau (s_k . q) / n_e,
//   w_R = Z_R / (Z_R + Z_E_hat) = 1 / (1 + exp(ln Z_E_hat - lse_R)),
//   out = w_R f_R + (1 - w_R) f_E_hat.
// Four 256-thread workgroups per unit, each owning 32 rows of S (and of the
// output): eight threads form one row of S q for every head from 16 contiguous
// floats each (float64 sums). The moment matrix is read once (64 KB per unit).
// With so little per workgroup the time is the chain of dependent loads, so
// every load that depends on nothing else is issued at entry (the thread's
// moment-matrix floats, its output element's f_R, s_v and lse), s_k . q is a
// lane reduction (one wave per head), and each thread owns at most one output
// element (G * 32 <= 256).
#include "kvc_device.h"
#include "kvc_kernels.h"

namespace kvc {
namespace {

constexpr int RPB = 32;   // rows of the moment matrix (and of the output) per workgroup

template <typename T, int G>
__global__ __launch_bounds__(WG) void k_moment_correct(const int32_t *mom_n, const float *mom_sk,
                                                       const float *mom_sv, const float *mom_S, const T *q,
                                                       double scale, const float *f_R, const float *lse_R,
                                                       float *out) {
  static_assert(G * RPB <= WG, "one output element per thread");
  __shared__ double qs[G][HD];
  __shared__ double sq[G][RPB];
  __shared__ double kq[G];
  const int a0 = blockIdx.y * RPB, u = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t o0 = int64_t(u) * G * HD;
  // this thread's output element (head og, row a0 + orr) and its inputs
  const bool has_o = tid < G * RPB;
  const int og = tid / RPB, orr = tid - og * RPB;
  const int64_t oo = o0 + int64_t(og) * HD + a0 + orr;
  float fr = 0.f, sv = 0.f, lse = 0.f;
  if (has_o) {
    fr = f_R[oo];
    sv = mom_sv[int64_t(u) * HD + a0 + orr];
    lse = lse_R[int64_t(u) * G + og];
  }
  // row a0 + tid / 8 of S, columns [16 h, 16 h + 16) with h = tid % 8
  const int r = tid >> 3, h = tid & 7;
  const float4 *row = reinterpret_cast<const float4 *>(mom_S + (int64_t(u) * HD + a0 + r) * HD + 16 * h);
  float4 s4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) s4[j] = row[j];
  const int n = mom_n[u];
  for (int idx = tid; idx < G * HD; idx += WG) (&qs[0][0])[idx] = double(load_elem<T>(q, o0 + idx));
  // s_k . q_g: wave w takes heads w, w + 4, ...; lane l elements 2 l and 2 l + 1
  const float sk0 = mom_sk[int64_t(u) * HD + 2 * lane], sk1 = mom_sk[int64_t(u) * HD + 2 * lane + 1];
  for (int g = wave; g < G; g += WG / 64) {
    double d = fma(double(sk0), double(load_elem<T>(q, o0 + g * HD + 2 * lane)),
                   double(sk1) * double(load_elem<T>(q, o0 + g * HD + 2 * lane + 1)));
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) d += __shfl_xor(d, o);
    if (lane == 0) kq[g] = d;
  }
  __syncthreads();
  if (n <= 0) {
    if (has_o) out[oo] = fr;
    return;
  }
  double acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = 16 * h + 4 * j;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      acc[g] = fma(double(s4[j].x), qs[g][b], acc[g]);
      acc[g] = fma(double(s4[j].y), qs[g][b + 1], acc[g]);
      acc[g] = fma(double(s4[j].z), qs[g][b + 2], acc[g]);
      acc[g] = fma(double(s4[j].w), qs[g][b + 3], acc[g]);
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) acc[g] += __shfl_xor(acc[g], o);
    if (h == 0) sq[g][r] = acc[g];
  }
  __syncthreads();
  if (has_o) {
    const double inv_n = 1.0 / double(n);
    const double svd = double(sv), kqg = kq[og];
    const double fE = svd * inv_n + scale * (sq[og][orr] - svd * kqg * inv_n) * inv_n;
    const double x = log(double(n)) + scale * kqg * inv_n - double(lse);   // ln(Z_E_hat / Z_R)
    const double wR = x > 0.0 ? exp(-x) / (1.0 + exp(-x)) : 1.0 / (1.0 + exp(x));
    out[oo] = float(wR * double(fr) + (1.0 - wR) * fE);
  }
}

template <typename T>
hipError_t launch_t(const MomentArgs &m, int n_units, const void *q, int G, double scale, const float *f_R,
                    const float *lse_R, float *out, hipStream_t st) {
  const T *qq = static_cast<const T *>(q);
  switch (G) {
    case 1: hipLaunchKernelGGL((k_moment_correct<T, 1>), dim3(n_units, HD / RPB), dim3(WG), 0, st, m.n, m.sk, m.sv, m.S, qq, scale, f_R, lse_R, out); break;
    case 2: hipLaunchKernelGGL((k_moment_correct<T, 2>), dim3(n_units, HD / RPB), dim3(WG), 0, st, m.n, m.sk, m.sv, m.S, qq, scale, f_R, lse_R, out); break;
    case 4: hipLaunchKernelGGL((k_moment_correct<T, 4>), dim3(n_units, HD / RPB), dim3(WG), 0, st, m.n, m.sk, m.sv, m.S, qq, scale, f_R, lse_R, out); break;
    case 8: hipLaunchKernelGGL((k_moment_correct<T, 8>), dim3(n_units, HD / RPB), dim3(WG), 0, st, m.n, m.sk, m.sv, m.S, qq, scale, f_R, lse_R, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_moment_correct(const MomentArgs &m, int n_units, const void *q, int dtype, int G, double scale,
                                 const float *f_R, const float *lse_R, float *out, hipStream_t st) {
  return dtype == 0 ? launch_t<bf16_t>(m, n_units, q, G, scale, f_R, lse_R, out, st)
                    : launch_t<float>(m, n_units, q, G, scale, f_R, lse_R, out, st);
}

}  // namespace kvc
