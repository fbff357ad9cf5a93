// Split-K decode attention for launches the per-scope kernel does not take
// (few or multi-unit scopes, long caches, the bulk first step), then the
// scope epilogue as its own launch.
//
// k_decode_split: grid x = split, y = attention unit. Each workgroup streams
// a contiguous range of CHW-token sub-chunks of its unit with the per-scope
// kernel's streaming core: NW waves, each taking every NW-th sub-chunk with
// PF sub-chunks of 16-byte K/V loads in flight; float64 logits with the
// lane-permuted transposed reduction (one head's logit per lane, no selects);
// a per-wave running maximum rescaled only when it moves; one weight
// exp(l - M) per (token, head) formed by one lane. The per-token weights go to
// the workspace (ews, with their shift counts in ewsh for weights below
// float32's range) with the running maximum of each sub-chunk (subM), so
// the epilogue can normalise them into attention weights; the waves'
// (M, Z, value sums) are combined into the workgroup's split partial.
//
// k_epi_score (token chunks x scopes) then k_epi_finish (one workgroup per
// scope): the scope epilogue (score, utility, then select -> fold -> compact,
// or a hand-over of scopes that evict more than one entry to the grid-wide
// bulk kernels).
#include <algorithm>

#include "kvc_epilogue.h"
#include "kvc_groups.h"
#include "kvc_stream.h"

namespace kvc {

int decode_chunk_tokens(int dtype) {
  return dtype == 0 ? UnitGeometry<bf16_t>::CHW : UnitGeometry<float>::CHW;
}

template <typename T, int G>
struct SplitLds {
  using Geo = UnitGeometry<T, G>;
  union {
    struct {
      float w[Geo::NW][Geo::UNR][Geo::TPI][G];   // weights for the value sums
      int vt[Geo::NW][Geo::CHW];                 // votes of the wave's current sub-chunk
    } st;
    struct {
      double pM[Geo::NW][G], pZ[Geo::NW][G];
      float pO[Geo::NW][G][HD];
      float fac[Geo::NW][G];
    } ep;
  };
};

// NTL: the rows load non-temporally (the bulk first step streams the whole prompt once,
// far more than any cache holds; a steady step's keys stay cached for the ZIP merge's
// cosine pass, which re-reads them).
template <typename T, int G, bool VOTES, bool NTL = false>
__global__ __launch_bounds__((UnitGeometry<T, G>::NT), 1) void k_decode_split(const StepArgs a) {
  using TR = ElemTraits<T>;
  using Geo = UnitGeometry<T, G>;
  constexpr int EPV = Geo::EPV, LPT = Geo::LPT, TPI = Geo::TPI, UNR = Geo::UNR;
  constexpr int CHW = Geo::CHW, PF = Geo::PF, NW = Geo::NW, NT = Geo::NT, RB = Geo::RB;
  constexpr int D = LPT / G;                         // lanes sharing one (token, head) logit
  constexpr int ITL = (UNR + D - 1) / D;             // weights a lane forms per sub-chunk
  static_assert(NW * G <= 64, "the combine runs in one wave");

  __shared__ SplitLds<T, G> sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int gu = blockIdx.y;
  const int scope = gu / a.attn_units, ua = gu - scope * a.attn_units;
  const int unit = a.attn_unit0 + ua;
  const int cap = a.capacity;
  const int64_t sc = int64_t(scope) * cap;
  int L = a.len[scope] + a.append;
  if (L > cap) L = 0;   // reported by the epilogue
  const int Lold = L - (L > 0 ? a.append : 0);

  UnitStream<T, VOTES, false, NTL, NTL> W;
  {
    const int64_t row0 = int64_t(scope) * a.scope_stride + int64_t(unit) * a.unit_stride;
    W.Kb = a.k + row0 * RB;
    W.Vb = a.v + row0 * RB;
    W.Kn = a.k_new + (int64_t(scope) * a.units + unit) * RB;
    W.Vn = a.v_new + (int64_t(scope) * a.units + unit) * RB;
    W.mrow = nullptr;
    W.vrow = VOTES ? a.votes + sc : nullptr;
    W.L = L;
    W.Lold = Lold;
    W.append = a.append;
    W.lane = lane;
    W.cb = lane % LPT;
    W.tg = lane / LPT;
  }
  const int cb = W.cb, tg = W.tg;
  const int myh = perm_head<LPT, G>(cb);
  const int dup = lane & (D - 1);
  float *ews = a.ews + int64_t(gu) * G * cap;
  uint8_t *ewsh = a.ewsh + int64_t(gu) * G * cap;
  double *subM = a.subM + int64_t(gu) * a.nsub_cap * G;

  // queries: one 16-byte load per head (slot i holding head i ^ myh), issued before the
  // first row loads and converted after them, so waiting for them leaves the rows in flight
  u32x4 qv[G];
  {
    const char *qp = a.q + int64_t(gu) * G * HD * int(sizeof(T));
#pragma unroll
    for (int i = 0; i < G; ++i) qv[i] = ld16g(qp + ((i ^ myh) * HD + cb * EPV) * int(sizeof(T)));
  }
  __builtin_amdgcn_sched_barrier(0);
  float oacc[G][EPV];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < EPV; ++j) oacc[g][j] = 0.f;
  double Mrun = -INFINITY, Zrun = 0.0;

  // this split's sub-chunks [c0, c1)
  const int nsub = L > 0 ? (L + CHW - 1) / CHW : 0;
  const int per = (nsub + a.n_splits - 1) / a.n_splits;
  const int c0 = min(nsub, int(blockIdx.x) * per), c1 = min(nsub, c0 + per);
  u32x4 kr[PF][UNR], vr[PF][UNR];
  float mv[PF];
  int vv[PF];
  // (every slot is issued once per sub-chunk it serves, clamped to the split's
  // last sub-chunk, so the loads past the range re-read lines already in L2)
  // (issued whether or not the split has sub-chunks -- an empty one loads the unit's first
  // row -- so no path reaches the loop with fewer loads outstanding than another)
#pragma unroll
  for (int s = 0; s < PF; ++s)
    W.issue(kr[s], vr[s], mv[s], vv[s], c0 < c1 ? min(c0 + wave + NW * s, c1 - 1) : 0, c0 < c1);
  __builtin_amdgcn_sched_barrier(0);
  // scaled by tau (exact in float64)
  double qf[G][EPV];
#pragma unroll
  for (int i = 0; i < G; ++i)
#pragma unroll
    for (int j = 0; j < EPV; ++j) qf[i][j] = double(TR::get(qv[i], j)) * a.scale;
  for (int base = c0 + wave; base < c1; base += NW * PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int c = base + NW * s;
      if (c < c1) {
        const bool tail = (c + 1) * CHW > L;
        if (VOTES && lane < CHW) sh.st.vt[wave][lane] = vv[s];
        double lg[UNR];
#pragma unroll
        for (int it = 0; it < UNR; ++it) {
          double acc[G];
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g] = 0.0;
#pragma unroll
          for (int j = 0; j < EPV; ++j) {
            const double kj = double(TR::get(kr[s][it], j));
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = fma(qf[g][j], kj, acc[g]);
          }
          lg[it] = preduce<LPT, G, 0>(acc);
          if (tail && c * CHW + it * TPI + tg >= L) lg[it] = -INFINITY;
        }
        double mx = lg[0];
#pragma unroll
        for (int it = 1; it < UNR; ++it) mx = fmax(mx, lg[it]);
#pragma unroll
        for (int o = LPT; o < 64; o <<= 1) mx = fmax(mx, __shfl_xor(mx, o));
        if (__ballot(mx > Mrun)) {
          const double Mnew = fmax(Mrun, mx);
          const double f = Mrun > -INFINITY ? exp(Mrun - Mnew) : 0.0;
          Zrun *= f;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float fg = float(readlane_f64(f, perm_rep_lane<LPT, G>(g)));
#pragma unroll
            for (int j = 0; j < EPV; ++j) oacc[g][j] *= fg;
          }
          Mrun = Mnew;
        }
        if (tg == 0 && dup == 0) subM[int64_t(c) * G + myh] = Mrun;
        __builtin_amdgcn_wave_barrier();
        // one weight per (token, head): lane `dup` takes iterations dup, dup + D, ...
#pragma unroll
        for (int r = 0; r < ITL; ++r) {
          const int it = dup + D * r;
          if (it < UNR) {
            double x = lg[0];
#pragma unroll
            for (int i2 = 1; i2 < UNR; ++i2) x = it == i2 ? lg[i2] : x;
            const int tok = c * CHW + it * TPI + tg;
            int shc;
            const float e = exp_shifted(x - Mrun, shc);
            float p = 1.f;
            if (VOTES) p = (a.append && tok == L - 1) ? 1.f : float(sh.st.vt[wave][min(tok, L - 1) - c * CHW]);
            const float w = shc ? 0.f : p * e;   // below exp(-SHIFT_STEP) of the maximum
            Zrun += double(w);
            sh.st.w[wave][it][tg][myh] = w;
            if (tok < L) {
              ews[int64_t(myh) * cap + tok] = e;
              ewsh[int64_t(myh) * cap + tok] = uint8_t(shc);
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int it = 0; it < UNR; ++it) {
          float wv[G];
#pragma unroll
          for (int g = 0; g < G; ++g) wv[g] = sh.st.w[wave][it][tg][g];
#pragma unroll
          for (int j = 0; j < EPV; ++j) {
            const float vj = TR::get(vr[s][it], j);
#pragma unroll
            for (int g = 0; g < G; ++g) oacc[g][j] = fmaf(wv[g], vj, oacc[g][j]);
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
      W.issue(kr[s], vr[s], mv[s], vv[s], min(c + NW * PF, c1 - 1));
    }
  }

  // ---- this wave's partials, then the workgroup's split partial
  double zt = Zrun;
#pragma unroll
  for (int o = 1; o < D; o <<= 1) zt += __shfl_xor(zt, o);
#pragma unroll
  for (int o = LPT; o < 64; o <<= 1) zt += __shfl_xor(zt, o);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < EPV; ++j) {
      float x = oacc[g][j];
#pragma unroll
      for (int o = LPT; o < 64; o <<= 1) x += __shfl_xor(x, o);
      oacc[g][j] = x;
    }
  __syncthreads();   // streaming scratch becomes the combine's space
  if (lane < LPT) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < EPV; ++j) sh.ep.pO[wave][g][cb * EPV + j] = oacc[g][j];
  }
  if (tg == 0 && dup == 0) {
    sh.ep.pM[wave][myh] = Mrun;
    sh.ep.pZ[wave][myh] = zt;
  }
  __syncthreads();
  const int64_t pbase = int64_t(gu) * a.n_splits + blockIdx.x;
  if (wave == 0) {
    constexpr int NC = NW * G;
    const int w = lane / G, g = lane % G;
    const bool act = lane < NC;
    const double pm = act ? sh.ep.pM[w][g] : -INFINITY;
    double M = pm;
#pragma unroll
    for (int o = G; o < NC; o <<= 1) M = fmax(M, __shfl_xor(M, o));
    const double ew = pm > -INFINITY ? exp(pm - M) : 0.0;
    double Z = act ? sh.ep.pZ[w][g] * ew : 0.0;
#pragma unroll
    for (int o = G; o < NC; o <<= 1) Z += __shfl_xor(Z, o);
    if (act) sh.ep.fac[w][g] = float(ew);
    if (lane < G) {
      a.partM[pbase * G + g] = M;
      a.partZ[pbase * G + g] = Z;
    }
  }
  __syncthreads();
  float *po = a.partO + pbase * G * HD;
  for (int idx = tid; idx < G * HD; idx += NT) {
    const int g = idx / HD, e = idx - (idx / HD) * HD;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) acc = fmaf(sh.ep.pO[w][g][e], sh.ep.fac[w][g], acc);
    po[idx] = acc;
  }
}

// ---------------------------------------------------------------- epilogue launches
// The per-head score and finish kernels (one attention unit and one unit per scope,
// chosen on the host from the same launch arguments) are separate kernels, so they
// carry none of the general kernels' code for several units.
template <int G, int CH>
__global__ __launch_bounds__(WG) void k_epi_score(const StepArgs a) {
  __shared__ ScoreLds sh;
  epi_score<G, CH>(a, sh);
}

template <int G, int CH>
__global__ __launch_bounds__(WG) void k_epi_score_head(const StepArgs a) {
  __shared__ ScoreLds sh;
  epi_score_head<G, CH>(a, sh);
}

template <typename T, int G>
__global__ __launch_bounds__(WG) void k_epi_finish(const StepArgs a) {
  __shared__ EpiLds sh;
  epi_finish<T, G>(a, sh);
}

template <typename T, int G>
__global__ __launch_bounds__(WG) void k_epi_finish_head(const StepArgs a) {
  __shared__ EpiLds sh;
  epi_finish_head<T, G>(a, sh);
}

template <typename T, int G>
static hipError_t launch_split_tg(const StepArgs &a, hipStream_t st) {
  using Geo = UnitGeometry<T, G>;
  const dim3 grid(a.n_splits, a.n_scopes * a.attn_units);
  if (a.bulk) {
    if (a.votes) hipLaunchKernelGGL((k_decode_split<T, G, true, true>), grid, dim3(Geo::NT), 0, st, a);
    else hipLaunchKernelGGL((k_decode_split<T, G, false, true>), grid, dim3(Geo::NT), 0, st, a);
  } else {
    if (a.votes) hipLaunchKernelGGL((k_decode_split<T, G, true>), grid, dim3(Geo::NT), 0, st, a);
    else hipLaunchKernelGGL((k_decode_split<T, G, false>), grid, dim3(Geo::NT), 0, st, a);
  }
  const int chunks = std::max(1, std::min(a.n_score_chunks, (a.max_len + a.score_chunk - 1) / a.score_chunk));
  if (a.attn_units == 1 && a.units == 1 && a.score_chunk <= (8 / G) * WG)
    hipLaunchKernelGGL((k_epi_score_head<G, Geo::CHW>), dim3(chunks, a.n_scopes), dim3(WG), 0, st, a);
  else
    hipLaunchKernelGGL((k_epi_score<G, Geo::CHW>), dim3(chunks, a.n_scopes), dim3(WG), 0, st, a);
  // the finish kernel selects, folds and moves; a call that cannot evict (budget >= capacity),
  // appends nothing and reports no flags has nothing for it to do
  const bool finish = !a.merge_select &&
                      (a.append || a.mode == 2 || a.evict_out || a.bulk || (a.mode != 0 && a.budget < a.capacity));
  // (several finish workgroups per scope only with the score kernel's length copy)
  const int fin_blocks = a.steplen ? std::max(1, a.fin_blocks) : 1;
  if (finish) {
    if (a.units == 1 && a.mode == 1)
      hipLaunchKernelGGL((k_epi_finish_head<T, G>), dim3(a.n_scopes), dim3(WG), 0, st, a);
    else
      hipLaunchKernelGGL((k_epi_finish<T, G>), dim3(a.n_scopes, fin_blocks), dim3(WG), 0, st, a);
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_split_g(const StepArgs &a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_split_tg<T, 1>(a, st);
    case 2: return launch_split_tg<T, 2>(a, st);
    case 4: return launch_split_tg<T, 4>(a, st);
    case 8: return launch_split_tg<T, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const StepArgs &a, int dtype, int G, hipStream_t st) {
  return dtype == 0 ? launch_split_g<bf16_t>(a, G, st) : launch_split_g<float>(a, G, st);
}

template <typename T, int G>
static hipError_t launch_attention_tg(const StepArgs &a, hipStream_t st) {
  using Geo = UnitGeometry<T, G>;
  const dim3 grid(a.n_splits, a.n_scopes * a.attn_units);
  if (a.votes) hipLaunchKernelGGL((k_decode_split<T, G, true>), grid, dim3(Geo::NT), 0, st, a);
  else hipLaunchKernelGGL((k_decode_split<T, G, false>), grid, dim3(Geo::NT), 0, st, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_attention_g(const StepArgs &a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_attention_tg<T, 1>(a, st);
    case 2: return launch_attention_tg<T, 2>(a, st);
    case 4: return launch_attention_tg<T, 4>(a, st);
    case 8: return launch_attention_tg<T, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_attention(const StepArgs &a, int dtype, int G, hipStream_t st) {
  return dtype == 0 ? launch_attention_g<bf16_t>(a, G, st) : launch_attention_g<float>(a, G, st);
}

}  // namespace kvc
