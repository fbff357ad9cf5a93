// Scope epilogue of the decode step (combine split partials, score, utility,
// select, moment fold, compaction), shared by the decode kernels.
#pragma once

#include "kvc_decode.h"
#include "kvc_ops.h"

namespace kvc {

__device__ __forceinline__ double apply_rule(int rule, double alpha, double m_old, double s) {
  if (rule == 0) return s;                                  // single
  if (rule == 1) return m_old + s;                          // cumulative
  return alpha * m_old + (1.0 - alpha) * s;                 // EMA
}

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

  const bool step = a.mode != 0;
  const int k = step ? max(0, L - a.budget) : 0;
  if (a.bulk && k > 1) {   // the grid-wide kernels launched after this one take over from (3)
    if (tid == 0) {
      BulkScope &b = a.bulk[scope];
      b.prefix = 0;
      b.mask = 0;
      b.krem = k;
      b.done = 0;
      b.L = L;
      b.k = k;
      b.n_pairs = 0;
    }
    return;
  }

  // (3) score s(i), utility m(i) and, for a single eviction, the argmin key.
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

  if (a.bulk && tid == 0) a.bulk[scope].k = 0;   // finished here: the bulk kernels skip this scope

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

}  // namespace kvc
