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

#include "kvc_decode.h"
#include "kvc_ops.h"

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

__device__ __forceinline__ double apply_rule(int rule, double alpha, double m_old, double s) {
  if (rule == 0) return s;                                  // single
  if (rule == 1) return m_old + s;                          // cumulative
  return alpha * m_old + (1.0 - alpha) * s;                 // EMA
}

template <typename T, int G>
struct SplitLds {
  double lgt[G][Geometry<T>::CH];
  float w[Geometry<T>::CH][G];
  double red[4][G];
  double Mrun[G], Zrun[G];
  float ofac[G];
  float ored[4][G][HD];
};

struct EpiLds {
  union {
    SelectLds sel;
    FoldLds fold;
  };
  double M[64], Z[64];
  int red[8];
  int best_slot;
};

// ---------------------------------------------------------------- epilogue
// CH: tokens per sub-chunk, the granularity at which the streaming phase
// recorded its running maxima (subM) for the per-token weights.
// ew: per-token weights exp(l - M_sub) of the scope's first attention unit,
// [ua][g][ew_ld]; fm: sub-chunk maxima [ua][fm_ld][g], replaced in place by the
// score factors.
template <typename T, int G, int CH>
__device__ void decode_epilogue(const StepArgs &a, const int scope, const int L, EpiLds &sh,
                                const float *ew, int64_t ew_ld, double *fm, int64_t fm_ld) {
  const int tid = threadIdx.x;
  const int Ua = a.attn_units, cap = a.capacity, ns = a.n_splits;
  const int gu0 = scope * Ua;
  const int64_t sc = int64_t(scope) * cap;
  const int row_bytes = HD * int(sizeof(T));

  // (1) combine split partials: per attention head M, Z, lse, o.
  if (tid < Ua * G) {
    const int gu = gu0 + tid / G, g = tid % G;
    double M = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) M = fmax(M, a.partM[(int64_t(gu) * ns + sp) * G + g]);
    double Z = 0.0;
    for (int sp = 0; sp < ns; ++sp) {
      const double pm = a.partM[(int64_t(gu) * ns + sp) * G + g];
      if (pm > -INFINITY) Z += a.partZ[(int64_t(gu) * ns + sp) * G + g] * exp(pm - M);
    }
    for (int sp = 0; sp < ns; ++sp) {
      const double pm = a.partM[(int64_t(gu) * ns + sp) * G + g];
      a.fac[(int64_t(gu) * ns + sp) * G + g] = (Z > 0.0 && pm > -INFINITY) ? float(exp(pm - M) / Z) : 0.f;
    }
    sh.M[tid] = M;
    sh.Z[tid] = Z;
    a.lse[int64_t(gu) * G + g] = Z > 0.0 ? float(M + log(Z)) : -INFINITY;
  }
  __syncthreads();
  for (int idx = tid; idx < Ua * G * HD; idx += WG) {
    const int pair = idx / HD, e = idx - (idx / HD) * HD;
    const int gu = gu0 + pair / G, g = pair % G;
    float acc = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
      const int64_t pi = (int64_t(gu) * ns + sp) * G + g;
      acc = fmaf(a.partO[pi * HD + e], a.fac[pi], acc);
    }
    a.out[(int64_t(gu) * G + g) * HD + e] = acc;
  }

  // (2) score factors F = exp(M_sub - M) / Z, in place of the sub-chunk maxima.
  const bool score = a.refresh && (a.mode != 0 || a.s != nullptr);
  const int nsubL = (L + CH - 1) / CH;
  if (score) {
    for (int idx = tid; idx < Ua * nsubL * G; idx += WG) {
      const int ua = idx / (nsubL * G), rem = idx - ua * (nsubL * G);
      const int c = rem / G, g = rem - (rem / G) * G;
      double *p = fm + (int64_t(ua) * fm_ld + c) * G + g;
      const double Z = sh.Z[ua * G + g];
      *p = Z > 0.0 ? exp(*p - sh.M[ua * G + g]) / Z : 0.0;
    }
  }
  __syncthreads();

  // (3) score s(i), utility m(i) and, for a single eviction, the argmin key.
  const bool step = a.mode != 0;
  const int k = step ? max(0, L - a.budget) : 0;
  const double inv_heads = 1.0 / double(Ua * G);
  const double alpha = double(a.alpha);
  uint64_t best = ~0ull;
  int best_slot = 0x7fffffff;
  for (int i = tid; i < L; i += WG) {
    const bool isnew = a.append && i == L - 1;
    float mval = 0.f;
    if (score) {
      const int pv = isnew ? 1 : (a.votes ? a.votes[sc + i] : 1);
      const int c = i / CH;
      double acc = 0.0;
      for (int ua = 0; ua < Ua; ++ua) {
#pragma unroll
        for (int g = 0; g < G; ++g)
          acc += double(ew[(int64_t(ua) * G + g) * ew_ld + i]) * fm[(int64_t(ua) * fm_ld + c) * G + g];
      }
      const double sv = double(pv) * acc * inv_heads;
      if (a.s) a.s[sc + i] = float(sv);
      if (step) {
        const double mo = isnew ? 0.0 : double(a.m[sc + i]);
        mval = float(apply_rule(a.rule, alpha, mo, sv));
        a.m[sc + i] = mval;
      }
    } else if (step) {
      mval = isnew ? 0.f : a.m[sc + i];
    }
    if (isnew && !(score && step)) a.m[sc + i] = 0.f;
    if (k == 1) {
      const uint32_t pi = uint32_t(isnew ? a.t : a.pos[sc + i]);
      const uint64_t key = order_key(mval, pi);
      if (key < best) {
        best = key;
        best_slot = i;
      }
    }
  }

  // (4) the appended token's rows and slot arrays.
  if (a.append) {
    const int nv = row_bytes / 16;
    for (int idx = tid; idx < a.units * nv; idx += WG) {
      const int u = idx / nv, c = idx - (idx / nv) * nv;
      const int64_t row = (int64_t(scope) * a.scope_stride + int64_t(u) * a.unit_stride + (L - 1)) * row_bytes;
      const int64_t src = (int64_t(scope) * a.units + u) * row_bytes;
      st16(a.k + row + 16 * c, ld16(a.k_new + src + 16 * c));
      st16(a.v + row + 16 * c, ld16(a.v_new + src + 16 * c));
    }
    if (tid == 0) {
      if (a.votes) a.votes[sc + L - 1] = 1;
      a.pos[sc + L - 1] = a.t;
    }
  }
  if (k == 1) best_slot = wg_argmin_finish(best, best_slot, sh.sel);
  __threadfence_block();
  __syncthreads();

  if (!step) {
    if (tid == 0) a.len[scope] = L;
    return;
  }
  if (k <= 0) {
    for (int i = tid; i < L; i += WG) {
      if (a.evict_out) a.evict_out[sc + i] = 0;
      if (a.mode == 2) a.flags[sc + i] = 0;
    }
    if (tid == 0) a.len[scope] = L;
    return;
  }
  if (a.mode == 2 && k > 1) {     // a merge handles one eviction per step
    if (tid == 0) {
      a.status[0] = -3;
      a.len[scope] = L;
    }
    for (int i = tid; i < L; i += WG) a.flags[sc + i] = 0;
    return;
  }

  // (5) selection of the k lowest (m, pos).
  uint8_t *flags = a.flags + sc;
  int32_t *list = a.list + sc;
  int e1 = -1;
  if (k == 1) {
    e1 = best_slot;
    for (int i = tid; i < L; i += WG) {
      if (a.evict_out) a.evict_out[sc + i] = (i == e1);
      if (a.mode == 2) flags[i] = (i == e1);
    }
    if (tid == 0) list[0] = e1;
  } else {
    const float *mm = a.m + sc;
    const int32_t *pp = a.pos + sc;
    auto key = [&](int i) -> uint64_t { return order_key(mm[i], uint32_t(pp[i])); };
    const SelectCut cut = wg_select_cut(key, L, k, sh.sel);
    wg_apply_cut(key, L, cut, flags, a.evict_out ? a.evict_out + sc : nullptr, list, sh.sel);
  }
  __threadfence_block();
  __syncthreads();

  // (6) moment fold of the evicted rows, before they are overwritten.
  if (a.mom_S) {
    for (int u = 0; u < a.units; ++u) {
      const int64_t row0 = int64_t(scope) * a.scope_stride + int64_t(u) * a.unit_stride;
      const T *Kb = reinterpret_cast<const T *>(a.k) + row0 * HD;
      const T *Vb = reinterpret_cast<const T *>(a.v) + row0 * HD;
      const int64_t mu = int64_t(scope) * a.units + u;
      if (k == 1) {
        FoldAcc f;
        fold_zero(f);
        if (tid == 0) sh.fold.slots[0] = e1;
        __syncthreads();
        fold_slots<T>(f, Kb, Vb, 1, sh.fold);
        fold_commit(f, 1, a.mom_n + mu, a.mom_sk + mu * HD, a.mom_sv + mu * HD, a.mom_S + mu * HD * HD);
      } else {
        fold_flagged<T>(Kb, Vb, flags, L, a.mom_n + mu, a.mom_sk + mu * HD, a.mom_sv + mu * HD,
                        a.mom_S + mu * HD * HD, sh.fold);
      }
      __syncthreads();
    }
  }

  if (a.mode == 2) {       // selection only: a merge pass compacts afterwards
    if (tid == 0) a.len[scope] = L;
    return;
  }

  // (7) hole-filling compaction.
  ScopeRows rows{a.k, a.v, int64_t(scope) * a.scope_stride, a.unit_stride, a.units, row_bytes,
                 a.votes ? a.votes + sc : nullptr, a.pos + sc, a.m + sc};
  if (k == 1) {
    if (e1 < L - 1) move_slot_wg(rows, L - 1, e1);
  } else {
    wg_compact_flags(rows, flags, L, k, a.list2 + sc, sh.red);
  }
  if (tid == 0) a.len[scope] = L - k;
}

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
        kr[it] = u32x4{0, 0, 0, 0};
        vr[it] = u32x4{0, 0, 0, 0};
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
    }
    return;
  }
  decode_epilogue<T, G, CH>(a, scope, L, lds.ep, a.ews + int64_t(scope) * a.attn_units * G * cap, cap,
                            a.subM + int64_t(scope) * a.attn_units * a.nsub_cap * G, a.nsub_cap);
  if (tid == 0) a.counters[scope] = 0;
}

// ---------------------------------------------------------------- one workgroup per scope
// For launches with one attention unit per scope and enough scopes to fill
// the device. The workgroup streams its unit's whole cache: each of the four
// waves takes every fourth sub-chunk of CHW tokens and keeps PF sub-chunks of
// 16-byte loads in flight, so waves never wait on each other while streaming.
// A wave forms float64 logits, reduces them so each lane holds one head's
// logit (transposed reduction), keeps a running per-head maximum (rescaling
// its value sums only when the maximum moves) and records the maximum of
// every sub-chunk for the per-token weights. The four waves' partials then
// feed the same epilogue as the split kernel, inside this workgroup: no
// counters, no device-scope fences.
template <typename T>
struct UnitGeometry {
  static constexpr int EPV = ElemTraits<T>::EPV;
  static constexpr int LPT = HD / EPV;
  static constexpr int TPI = 64 / LPT;
  static constexpr int UNR = 4;            // iterations per sub-chunk
  static constexpr int CHW = TPI * UNR;    // tokens per sub-chunk
  static constexpr int PF = 4;             // sub-chunks of loads in flight per wave
  static constexpr int NW = WG / 64;       // waves
};

int decode_unit_chunk_tokens(int dtype) {
  return dtype == 0 ? UnitGeometry<bf16_t>::CHW : UnitGeometry<float>::CHW;
}

template <typename T, int G>
struct UnitWave {
  using Geo = UnitGeometry<T>;
  static constexpr int UNR = Geo::UNR, TPI = Geo::TPI, LPT = Geo::LPT, EPV = Geo::EPV, CHW = Geo::CHW;

  const char *Kb, *Vb, *Kn, *Vn;
  const int32_t *vrow;    // the scope's votes, or any valid int row when votes are absent
  int L, append, cb, tg, lane;

  // Loads of sub-chunk c (token index clamped into the live range, so every
  // call issues the same loads and the wait counts stay exact).
  __device__ __forceinline__ void issue(u32x4 (&kr)[UNR], u32x4 (&vr)[UNR], int (&vt)[UNR], int c) const {
#pragma unroll
    for (int it = 0; it < UNR; ++it) {
      const int tok = min(c * CHW + it * TPI + tg, L - 1);
      const bool isnew = append && tok == L - 1;
      const char *ks = isnew ? Kn : Kb + int64_t(tok) * (HD * int64_t(sizeof(T)));
      const char *vs = isnew ? Vn : Vb + int64_t(tok) * (HD * int64_t(sizeof(T)));
      kr[it] = ld16(ks + 16 * cb);
      vr[it] = ld16(vs + 16 * cb);
      const int vote = vrow[tok];          // slot L-1 holds no vote yet when it is the appended token
      vt[it] = isnew ? 1 : vote;
    }
  }
};

template <typename T, int G>
__global__ __launch_bounds__(WG, 1) void k_decode_unit(const StepArgs a) {
  using TR = ElemTraits<T>;
  using Geo = UnitGeometry<T>;
  constexpr int EPV = Geo::EPV, LPT = Geo::LPT, TPI = Geo::TPI, UNR = Geo::UNR;
  constexpr int CHW = Geo::CHW, PF = Geo::PF, NW = Geo::NW;

  __shared__ union {
    float w[NW][UNR][TPI][G];
    EpiLds ep;
  } lds;
  // dynamic LDS: weights e[G][lds_len] (float), then sub-chunk maxima [nsub][G] (double)
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int lds_len = a.lds_len;
  float *e_lds = reinterpret_cast<float *>(dyn);
  double *m_lds = reinterpret_cast<double *>(dyn + size_t(G) * lds_len * 4);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int scope = blockIdx.x, gu = scope;
  const int unit = a.attn_unit0;
  const int cap = a.capacity;
  int L = a.len[scope] + a.append;
  const bool overflow = L > cap || L > lds_len;
  if (overflow) L = 0;

  UnitWave<T, G> W;
  {
    const int64_t row0 = int64_t(scope) * a.scope_stride + int64_t(unit) * a.unit_stride;
    W.Kb = a.k + row0 * (HD * int64_t(sizeof(T)));
    W.Vb = a.v + row0 * (HD * int64_t(sizeof(T)));
    W.Kn = a.k_new + (int64_t(scope) * a.units + unit) * (HD * int64_t(sizeof(T)));
    W.Vn = a.v_new + (int64_t(scope) * a.units + unit) * (HD * int64_t(sizeof(T)));
    W.vrow = (a.votes ? a.votes : a.pos) + int64_t(scope) * cap;
    W.L = L;
    W.append = a.append;
    W.cb = lane % LPT;
    W.tg = lane / LPT;
    W.lane = lane;
  }
  const int cb = W.cb, tg = W.tg;
  const int myh = lane_head<LPT, G>(lane);
  const bool leader = head_leader<LPT, G>(lane);

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
  double Mrun = -INFINITY, Zrun = 0.0;

  const int nsub = L > 0 ? (L + CHW - 1) / CHW : 0;
  u32x4 kr[PF][UNR], vr[PF][UNR];
  int vt[PF][UNR];
  if (nsub > 0) {
#pragma unroll
    for (int s = 0; s < PF; ++s) W.issue(kr[s], vr[s], vt[s], wave + NW * s);
  }
  const bool has_votes = a.votes != nullptr;
  for (int base = wave; base < nsub; base += NW * PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int c = base + NW * s;
      if (c < nsub) {
        // logits: lane ends with head myh of token (c*CHW + it*TPI + tg)
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
          const double l = treduce<LPT, G, 0>(acc, lane) * a.scale;
          lg[it] = (c * CHW + it * TPI + tg < L) ? l : -INFINITY;
        }
        double mx = lg[0];
#pragma unroll
        for (int it = 1; it < UNR; ++it) mx = fmax(mx, lg[it]);
#pragma unroll
        for (int o = LPT; o < 64; o <<= 1) mx = fmax(mx, __shfl_xor(mx, o));
        const double Mnew = fmax(Mrun, mx);
        if (__ballot(Mnew > Mrun)) {
          const double f = Mrun > -INFINITY ? exp(Mrun - Mnew) : 0.0;
          Zrun *= f;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float fg = float(readlane_f64(f, head_rep_lane<LPT, G>(g)));
#pragma unroll
            for (int j = 0; j < EPV; ++j) oacc[g][j] *= fg;
          }
          Mrun = Mnew;
        }
        if (tg == 0 && leader) m_lds[c * G + myh] = Mrun;
        // weights p_i exp(l - M): one lane per (token, head) publishes
#pragma unroll
        for (int it = 0; it < UNR; ++it) {
          const int tok = c * CHW + it * TPI + tg;
          const float e = exp_split(lg[it] - Mrun);
          const float w = (has_votes ? float(vt[s][it]) : 1.f) * e;
          Zrun += double(w);
          if (leader) {
            lds.w[wave][it][tg][myh] = w;
            if (tok < L) e_lds[myh * lds_len + tok] = e;
          }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int it = 0; it < UNR; ++it) {
          float wv[G];
#pragma unroll
          for (int g = 0; g < G; ++g) wv[g] = lds.w[wave][it][tg][g];
#pragma unroll
          for (int j = 0; j < EPV; ++j) {
            const float vj = TR::get(vr[s][it], j);
#pragma unroll
            for (int g = 0; g < G; ++g) oacc[g][j] = fmaf(wv[g], vj, oacc[g][j]);
          }
        }
        __builtin_amdgcn_wave_barrier();
      }
      W.issue(kr[s], vr[s], vt[s], c + NW * PF);
    }
  }

  // this wave's partials: (M, Z) per head and the value sums
  double zt = Zrun;
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
  const int64_t pbase = int64_t(gu) * a.n_splits + wave;
  if (lane < LPT) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < EPV; ++j) a.partO[(pbase * G + g) * HD + cb * EPV + j] = oacc[g][j];
  }
  if (tg == 0 && leader) {
    a.partM[pbase * G + myh] = Mrun;
    a.partZ[pbase * G + myh] = zt;
  }
  __threadfence_block();
  __syncthreads();
  if (overflow) {
    if (tid == 0) a.status[0] = -4;
    return;
  }
  decode_epilogue<T, G, CHW>(a, scope, L, lds.ep, e_lds, lds_len, m_lds, 0);
}

// Dynamic LDS of the per-scope kernel for caches of up to lds_len live tokens.
size_t decode_unit_lds_bytes(int dtype, int G, int lds_len) {
  const int chw = decode_unit_chunk_tokens(dtype);
  return size_t(G) * lds_len * 4 + size_t((lds_len + chw - 1) / chw) * G * 8;
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

template <typename T, int G>
static hipError_t launch_unit_tg(const StepArgs &a, hipStream_t st) {
  const size_t dyn = decode_unit_lds_bytes(std::is_same<T, float>::value ? 1 : 0, G, a.lds_len);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_decode_unit<T, G>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(dyn));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode_unit<T, G>), dim3(a.n_scopes), dim3(WG), dyn, st, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_unit_g(const StepArgs &a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_unit_tg<T, 1>(a, st);
    case 2: return launch_unit_tg<T, 2>(a, st);
    case 4: return launch_unit_tg<T, 4>(a, st);
    case 8: return launch_unit_tg<T, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const StepArgs &a, int dtype, int G, hipStream_t st) {
  dim3 grid(a.n_splits, a.n_scopes * a.attn_units);
  return dtype == 0 ? launch_g<bf16_t>(a, G, grid, st) : launch_g<float>(a, G, grid, st);
}

hipError_t launch_decode_unit(const StepArgs &a, int dtype, int G, hipStream_t st) {
  return dtype == 0 ? launch_unit_g<bf16_t>(a, G, st) : launch_unit_g<float>(a, G, st);
}

}  // namespace kvc
