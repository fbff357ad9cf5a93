// Fused decode step over a fixed-budget cache: append, vote-weighted split-K
// GQA attention, head-averaged score, utility update, selection, moment fold
// and compaction, in one launch. Also serves the attention-only entry point.
//
// Grid: x = split (workgroups sharing one attention unit), y = attention unit.
// Each workgroup streams whole sub-chunks of CH tokens of its unit: every lane
// issues all of its 16-byte K and V loads for the sub-chunk first, then forms
// float64 logits (bf16/fp32 products are exact in float64), the per-head
// sub-chunk maximum, the weights p_i exp(l - M) and the value sums. The last
// workgroup of a scope to finish (device-scope counter) combines the partials
// and runs the scope's score -> utility -> select -> fold -> compact epilogue.
#include <type_traits>

#include "kvc_epilogue.h"

namespace kvc {

template <typename T>
struct Geometry {
  static constexpr int EPV = ElemTraits<T>::EPV;  // elements per lane-vector
  static constexpr int LPT = HD / EPV;            // lanes per token row
  static constexpr int TPI = 64 / LPT;            // tokens per wave per iteration
  static constexpr int UNR = 8;                   // iterations per wave per sub-chunk
  static constexpr int TPW = TPI * UNR;
  static constexpr int CH = (WG / 64) * TPW;      // tokens per sub-chunk
};

int decode_chunk_tokens(int dtype) { return dtype == 0 ? Geometry<bf16_t>::CH : Geometry<float>::CH; }

template <typename T, int G>
struct SplitLds {
  double lgt[G][Geometry<T>::CH];
  float w[Geometry<T>::CH][G];
  double red[4][G];
  double Mrun[G], Zrun[G];
  float ofac[G];
  float ored[4][G][HD];
};

// ---------------------------------------------------------------- split kernel
template <typename T, int G>
__global__ __launch_bounds__(WG) void k_decode(const StepArgs a) {
  using TR = ElemTraits<T>;
  using Geo = Geometry<T>;
  constexpr int EPV = Geo::EPV, LPT = Geo::LPT, TPI = Geo::TPI, UNR = Geo::UNR;
  constexpr int TPW = Geo::TPW, CH = Geo::CH;
  constexpr int NPAIR = CH * G;
  constexpr int RP = (NPAIR + WG - 1) / WG;

  __shared__ union {
    SplitLds<T, G> sp;
    EpiLds ep;
  } lds;
  __shared__ int s_last;
  SplitLds<T, G> &sh = lds.sp;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gu = blockIdx.y;
  const int scope = gu / a.attn_units, ua = gu - scope * a.attn_units;
  const int unit = a.attn_unit0 + ua;
  const int cap = a.capacity;
  int L = a.len[scope] + a.append;
  const bool overflow = L > cap;
  if (overflow) L = 0;

  const int64_t row0 = int64_t(scope) * a.scope_stride + int64_t(unit) * a.unit_stride;
  const char *Kb = a.k + row0 * (HD * int64_t(sizeof(T)));
  const char *Vb = a.v + row0 * (HD * int64_t(sizeof(T)));
  const char *Kn = a.k_new + (int64_t(scope) * a.units + unit) * (HD * int64_t(sizeof(T)));
  const char *Vn = a.v_new + (int64_t(scope) * a.units + unit) * (HD * int64_t(sizeof(T)));
  const int cb = lane % LPT;
  const int tg = lane / LPT;

  double qf[G][EPV];
  {
    const T *qp = reinterpret_cast<const T *>(a.q) + int64_t(gu) * G * HD;
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < EPV; ++j) qf[g][j] = double(load_elem<T>(qp, g * HD + cb * EPV + j));
  }
  float oacc[G][EPV];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < EPV; ++j) oacc[g][j] = 0.f;
  if (tid < G) {
    sh.Mrun[tid] = -INFINITY;
    sh.Zrun[tid] = 0.0;
  }
  __syncthreads();

  const int h = tid % G;
  const int nsub = (L + CH - 1) / CH;
  for (int c = blockIdx.x; c < nsub; c += a.n_splits) {
    const int base = c * CH;
    u32x4 kr[UNR], vr[UNR];
#pragma unroll
    for (int it = 0; it < UNR; ++it) {
      const int tok = base + wave * TPW + it * TPI + tg;
      if (tok < L) {
        const bool isnew = a.append && tok == L - 1;
        const char *ks = isnew ? Kn : Kb + int64_t(tok) * (HD * int64_t(sizeof(T)));
        const char *vs = isnew ? Vn : Vb + int64_t(tok) * (HD * int64_t(sizeof(T)));
        kr[it] = ld16(ks + 16 * cb);
        vr[it] = ld16(vs + 16 * cb);
      } else {
        kr[it] = u32x4(0u);
        vr[it] = u32x4(0u);
      }
    }
    // logits l = scale * q . k, float64 accumulation
#pragma unroll
    for (int it = 0; it < UNR; ++it) {
      double acc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = 0.0;
#pragma unroll
      for (int j = 0; j < EPV; ++j) {
        const double kj = double(TR::get(kr[it], j));
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = fma(qf[g][j], kj, acc[g]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) acc[g] = group_sum_f64<LPT>(acc[g]);
      if (cb == 0) {
        const int tl = wave * TPW + it * TPI + tg;
        const bool valid = base + tl < L;
#pragma unroll
        for (int g = 0; g < G; ++g) sh.lgt[g][tl] = valid ? acc[g] * a.scale : -INFINITY;
      }
    }
    __syncthreads();

    // per-head sub-chunk maximum; thread tid always serves head tid % G
    double lv[RP];
    double mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int p = tid + r * WG;
      lv[r] = p < NPAIR ? sh.lgt[h][p / G] : -INFINITY;
      mx = fmax(mx, lv[r]);
    }
    mx = wave_max_strided<G>(mx);
    if (lane < G) sh.red[wave][lane] = mx;
    __syncthreads();
    const double Mc = fmax(fmax(sh.red[0][h], sh.red[1][h]), fmax(sh.red[2][h], sh.red[3][h]));
    const double Mnew = fmax(sh.Mrun[h], Mc);
    double z = 0.0;
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      const int p = tid + r * WG;
      if (p < NPAIR) {
        const int tl = p / G, tok = base + tl;
        float w = 0.f;
        if (tok < L) {
          const float e = exp_split(lv[r] - Mnew);
          const int pv = (a.append && tok == L - 1) ? 1 : (a.votes ? a.votes[int64_t(scope) * cap + tok] : 1);
          w = float(pv) * e;
          a.ews[(int64_t(gu) * G + h) * cap + tok] = e;
          z += double(w);
        }
        sh.w[tl][h] = w;
      }
    }
    z = wave_sum_strided<G>(z);
    __syncthreads();
    if (lane < G) sh.red[wave][lane] = z;
    __syncthreads();
    if (tid < G) {
      const double zc = sh.red[0][tid] + sh.red[1][tid] + sh.red[2][tid] + sh.red[3][tid];
      const double Mo = sh.Mrun[tid];
      const double f = Mo > -INFINITY ? exp(Mo - Mnew) : 0.0;
      sh.Zrun[tid] = sh.Zrun[tid] * f + zc;
      sh.Mrun[tid] = Mnew;
      sh.ofac[tid] = float(f);
      a.subM[(int64_t(gu) * a.nsub_cap + c) * G + tid] = Mnew;
    }
    __syncthreads();
    // value sums with the weights p_i exp(l - M)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float f = sh.ofac[g];
#pragma unroll
      for (int j = 0; j < EPV; ++j) oacc[g][j] *= f;
    }
#pragma unroll
    for (int it = 0; it < UNR; ++it) {
      const int tl = wave * TPW + it * TPI + tg;
      float wv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) wv[g] = sh.w[tl][g];
#pragma unroll
      for (int j = 0; j < EPV; ++j) {
        const float vj = TR::get(vr[it], j);
#pragma unroll
        for (int g = 0; g < G; ++g) oacc[g][j] = fmaf(wv[g], vj, oacc[g][j]);
      }
    }
    __syncthreads();
  }

  // reduce the value sums over token groups and waves; write this split's partials
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < EPV; ++j) {
      float x = oacc[g][j];
#pragma unroll
      for (int o = LPT; o < 64; o <<= 1) x += __shfl_xor(x, o);
      oacc[g][j] = x;
    }
  if (lane < LPT) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < EPV; ++j) sh.ored[wave][g][cb * EPV + j] = oacc[g][j];
  }
  __syncthreads();
  {
    const int64_t pbase = int64_t(gu) * a.n_splits + blockIdx.x;
    float *po = a.partO + pbase * G * HD;
    for (int idx = tid; idx < G * HD; idx += WG) {
      const int g = idx / HD, e = idx - (idx / HD) * HD;
      po[idx] = sh.ored[0][g][e] + sh.ored[1][g][e] + sh.ored[2][g][e] + sh.ored[3][g][e];
    }
    if (tid < G) {
      a.partM[pbase * G + tid] = sh.Mrun[tid];
      a.partZ[pbase * G + tid] = sh.Zrun[tid];
    }
  }

  // last workgroup of the scope runs the epilogue
  release_device();
  __syncthreads();
  if (tid == 0) {
    release_device();
    const int prev = atomicAdd(a.counters + scope, 1);
    s_last = prev == a.n_splits * a.attn_units - 1;
  }
  __syncthreads();
  if (!s_last) return;
  acquire_device();
  if (overflow) {
    if (tid == 0) {
      a.status[0] = -4;
      a.counters[scope] = 0;
      if (a.bulk) a.bulk[scope].k = 0;
    }
    return;
  }
  decode_epilogue<T, G, CH>(a, scope, L, lds.ep, a.ews + int64_t(scope) * a.attn_units * G * cap, cap,
                            a.subM + int64_t(scope) * a.attn_units * a.nsub_cap * G, a.nsub_cap);
  if (tid == 0) a.counters[scope] = 0;
}

template <typename T>
static hipError_t launch_g(const StepArgs &a, int G, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1: hipLaunchKernelGGL((k_decode<T, 1>), grid, dim3(WG), 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_decode<T, 2>), grid, dim3(WG), 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_decode<T, 4>), grid, dim3(WG), 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_decode<T, 8>), grid, dim3(WG), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode(const StepArgs &a, int dtype, int G, hipStream_t st) {
  dim3 grid(a.n_splits, a.n_scopes * a.attn_units);
  return dtype == 0 ? launch_g<bf16_t>(a, G, grid, st) : launch_g<float>(a, G, grid, st);
}



}  // namespace kvc
