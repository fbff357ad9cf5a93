// Scope epilogue of the split-K decode step, as two grid launches after the
// attention kernel:
//   score  (workgroups x scopes): per-token score s(i) and utility m(i) over
//          token chunks of every scope, the lowest (m, pos) key of each chunk,
//          the appended token's rows;
//   finish (one workgroup per scope): combine the split partials into o and
//          lse, then select -> fold -> compact, or hand a scope that evicts
//          more than one entry to the grid-wide bulk kernels.
#pragma once

#include "kvc_decode.h"
#include "kvc_ops.h"

namespace kvc {

__device__ __forceinline__ double apply_rule(int rule, double alpha, double m_old, double s) {
  if (rule == 0) return s;                                  // single
  if (rule == 1) return m_old + s;                          // cumulative
  return alpha * m_old + (1.0 - alpha) * s;                 // EMA
}

// Largest (sub-chunks touched by one score chunk) x (attention heads of a
// scope): the host sizes score chunks so a chunk's factors fit.
constexpr int SCORE_FAC_MAX = 1280;
// Split partials (heads x splits) the score kernel stages in LDS at once.
constexpr int SCORE_PAIR_MAX = 1024;

struct ScoreLds {
  double M[64], iZ[64];
  double fac[SCORE_FAC_MAX];
  double pm[SCORE_PAIR_MAX];   // split maxima; then the splits' output weights exp(pm - M) / Z
  double pz[SCORE_PAIR_MAX];
  double red[WG];              // per-(part, token) head sums when a chunk has fewer tokens than threads
  uint64_t wkey[WG / 64];
  int wslot[WG / 64], wpos[WG / 64];
};

struct EpiLds {
  union {
    SelectLds sel;
    FoldLds fold;
  };
  uint64_t ckey[WG / 64];
  int cslot[WG / 64], cpos[WG / 64];
};

// Wave argmin of (key, position) carrying the slot.
__device__ __forceinline__ void wave_min_key_pos(uint64_t &key, uint32_t &pos, int &slot) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t k2 = shfl_xor_u64(key, o);
    const uint32_t p2 = __shfl_xor(pos, o);
    const int s2 = __shfl_xor(slot, o);
    if (key_pos_less(k2, p2, key, pos)) {
      key = k2;
      pos = p2;
      slot = s2;
    }
  }
}

// M and Z of attention head (gu, g) over the split partials.
template <int G>
__device__ __forceinline__ void combine_head(const StepArgs &a, int gu, int g, double &M, double &Z) {
  const int ns = a.n_splits;
  M = -INFINITY;
  for (int sp = 0; sp < ns; ++sp) M = fmax(M, a.partM[(int64_t(gu) * ns + sp) * G + g]);
  Z = 0.0;
  for (int sp = 0; sp < ns; ++sp) {
    const double pm = a.partM[(int64_t(gu) * ns + sp) * G + g];
    if (pm > -INFINITY) Z += a.partZ[(int64_t(gu) * ns + sp) * G + g] * exp(pm - M);
  }
}

// The new token's K and V rows of units y, y + ny, ... of the scope into slot L - 1.
__device__ __forceinline__ void append_rows_wg(const StepArgs &a, int scope, int L, int y = 0, int ny = 1) {
  const int64_t rb = a.row_bytes;
  copy_rows_wg(
      (a.units - y + ny - 1) / ny, a.row_bytes / 16,
      [&](int i, const char *&ks, const char *&vs) {
        const int64_t off = (int64_t(scope) * a.units + y + i * ny) * rb;
        ks = a.k_new + off;
        vs = a.v_new + off;
      },
      [&](int i, char *&kd, char *&vd) {
        const int64_t off = (int64_t(scope) * a.scope_stride + int64_t(y + i * ny) * a.unit_stride + (L - 1)) * rb;
        kd = a.k + off;
        vd = a.v + off;
      });
}

// ---------------------------------------------------------------- score
// InertiaKV §3.1 eq. (1): s(i) = mean over the scope's Ua*G attention heads of
// a_{h,i} = p_i e_{h,i} F_{h,c(i)}, where e = exp(l - M_sub) is the weight the
// attention kernel stored (times exp(-SHIFT_STEP * sh) for a shifted one) and
// F = exp(M_sub - M) / Z the factor of its CH-token sub-chunk; then eqs.
// (2)-(4) for m(i), in float64, stored as float32. For a step that evicts one
// entry, each chunk also reports its lowest (float64 m, pos); a scope that
// evicts more than one keeps the float64 utilities (m64) for the selection.
// Workgroups stride over the scope's chunks, so any live length is covered.
template <int G, int CH>
__device__ void epi_score(const StepArgs &a, ScoreLds &sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int scope = blockIdx.y;
  const int Ua = a.attn_units, cap = a.capacity, H = Ua * G;
  const int L = a.len[scope] + a.append;
  if (a.steplen && blockIdx.x == 0 && tid == 0) a.steplen[scope] = L;   // for a split finish
  if (L > cap) return;   // reported by the finish kernel
  const int64_t sc = int64_t(scope) * cap;
  const int gu0 = scope * Ua;
  const bool step = a.mode != 0;
  const bool score = a.refresh && (step || a.s != nullptr);
  const int k = step ? max(0, L - a.budget) : 0;
  const double inv_heads = 1.0 / double(H);
  const double alpha = double(a.alpha);
  const float *ews = a.ews + int64_t(gu0) * G * cap;
  const uint8_t *ewsh = a.ewsh + int64_t(gu0) * G * cap;
  double *m64 = (step && k > 1 && a.m64) ? a.m64 + sc : nullptr;
  const int chunk = a.score_chunk;
  // threads per token (a power of two): the units of a token are split over them when the
  // chunk has fewer tokens than threads and there are units to split
  int parts = 1;
  while (parts < Ua && chunk * parts * 2 <= WG) parts *= 2;

  // per attention head M and Z over the split partials (staged in LDS when they fit)
  const int ns = a.n_splits, P = H * ns;
  const bool staged = P <= SCORE_PAIR_MAX;
  if (staged) {
    for (int idx = tid; idx < P; idx += WG) {
      const int h = idx / ns, sp = idx - (idx / ns) * ns;
      const int64_t pi = (int64_t(gu0 + h / G) * ns + sp) * G + h % G;
      sh.pm[idx] = a.partM[pi];
      sh.pz[idx] = a.partZ[pi];
    }
    __syncthreads();
  }
  if (tid < H) {
    double M, Z;
    if (staged) {
      M = -INFINITY;
      for (int sp = 0; sp < ns; ++sp) M = fmax(M, sh.pm[tid * ns + sp]);
      Z = 0.0;
      for (int sp = 0; sp < ns; ++sp) {
        const double pm = sh.pm[tid * ns + sp];
        if (pm > -INFINITY) Z += sh.pz[tid * ns + sp] * exp(pm - M);
      }
    } else {
      combine_head<G>(a, gu0 + tid / G, tid % G, M, Z);
    }
    sh.M[tid] = M;
    sh.iZ[tid] = Z > 0.0 ? 1.0 / Z : 0.0;
    if (blockIdx.x == tid % gridDim.x) a.lse[int64_t(gu0) * G + tid] = Z > 0.0 ? float(M + log(Z)) : -INFINITY;
  }
  __syncthreads();
  // the attention output of the heads h = blockIdx.x (mod gridDim.x): o = sum over
  // splits of the split's value sums times exp(M_split - M) / Z
  if (staged) {
    for (int idx = tid; idx < P; idx += WG) {
      const int h = idx / ns;
      const double pm = sh.pm[idx];
      sh.pm[idx] = (sh.iZ[h] > 0.0 && pm > -INFINITY) ? exp(pm - sh.M[h]) * sh.iZ[h] : 0.0;
    }
    __syncthreads();
  }
  for (int idx = tid; idx < H * HD; idx += WG) {
    const int h = idx / HD, e = idx - (idx / HD) * HD;
    if (h % gridDim.x != blockIdx.x) continue;
    const int64_t gh = int64_t(gu0) * G + h;   // (gu0 + h / G) * G + h % G
    float acc = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
      const int64_t pi = (int64_t(gu0 + h / G) * ns + sp) * G + h % G;
      double wgt;
      if (staged) {
        wgt = sh.pm[h * ns + sp];
      } else {
        const double pm = a.partM[pi];
        wgt = (sh.iZ[h] > 0.0 && pm > -INFINITY) ? exp(pm - sh.M[h]) * sh.iZ[h] : 0.0;
      }
      acc = fmaf(a.partO[pi * HD + e], float(wgt), acc);
    }
    a.out[gh * HD + e] = acc;
  }
  for (int i0 = blockIdx.x * chunk; i0 < L; i0 += gridDim.x * chunk) {
    const int i1 = min(L, i0 + chunk);
    const int c0 = i0 / CH, nsc = (i1 - 1) / CH - c0 + 1;
    __syncthreads();
    if (score) {
      for (int idx = tid; idx < nsc * H; idx += WG) {
        const int c = c0 + idx / H, h = idx - (idx / H) * H;
        const double m = a.subM[(int64_t(gu0 + h / G) * a.nsub_cap + c) * G + h % G];
        sh.fac[idx] = sh.iZ[h] > 0.0 ? exp(m - sh.M[h]) * sh.iZ[h] : 0.0;
      }
    }
    __syncthreads();
    // a chunk of fewer tokens than threads: thread (token t, part p) sums the units p,
    // p + parts, ... of token i0 + t; the parts are added in order below
    if (score && parts > 1) {
      const int span = WG / parts, i = i0 + tid % span, p = tid / span;
      double acc = 0.0;
      if (i < i1) {
        const double *f = sh.fac + (i / CH - c0) * H;
        for (int ua = p; ua < Ua; ua += parts) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const int64_t wi = (int64_t(ua) * G + g) * cap + i;
            const int shv = ewsh[wi];
            const double x = double(ews[wi]) * f[ua * G + g];
            acc += shv ? x * shift_scale(shv) : x;
          }
        }
      }
      sh.red[tid] = acc;
      __syncthreads();
    }
    uint64_t best = ~0ull;
    uint32_t bpos = 0xffffffffu;
    int bslot = 0x7fffffff;
    for (int i = i0 + tid; i < i1; i += WG) {
      const bool isnew = a.append && i == L - 1;
      double mval = 0.0;
      if (score) {
        const int pv = isnew ? 1 : (a.votes ? a.votes[sc + i] : 1);
        double acc = 0.0;
        if (parts > 1) {
          for (int p = 0; p < parts; ++p) acc += sh.red[p * (WG / parts) + tid];
        } else {
          const double *f = sh.fac + (i / CH - c0) * H;
          for (int ua = 0; ua < Ua; ++ua) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const int64_t wi = (int64_t(ua) * G + g) * cap + i;
              const int shv = ewsh[wi];
              const double x = double(ews[wi]) * f[ua * G + g];
              acc += shv ? x * shift_scale(shv) : x;
            }
          }
        }
        const double sv = double(pv) * acc * inv_heads;
        if (a.s) a.s[sc + i] = float(sv);
        if (step) {
          const double mo = isnew ? 0.0 : double(a.m[sc + i]);
          mval = apply_rule(a.rule, alpha, mo, sv);
          a.m[sc + i] = float(mval);
        }
      } else if (step) {
        mval = isnew ? 0.0 : double(a.m[sc + i]);
      }
      if (isnew && !(score && step)) a.m[sc + i] = 0.f;
      if (m64) m64[i] = mval;
      if (k == 1) {
        const uint64_t key = orderable_f64(mval);
        const uint32_t p = uint32_t(isnew ? a.t : a.pos[sc + i]);
        if (key_pos_less(key, p, best, bpos)) {
          best = key;
          bpos = p;
          bslot = i;
        }
      }
    }
    if (k == 1) {   // (utility, position) pairs are distinct: the minimum names one slot
      wave_min_key_pos(best, bpos, bslot);
      if (lane == 0) {
        sh.wkey[wave] = best;
        sh.wslot[wave] = bslot;
        sh.wpos[wave] = int(bpos);
      }
      __syncthreads();
      if (tid == 0) {
#pragma unroll
        for (int w = 1; w < WG / 64; ++w) {
          if (key_pos_less(sh.wkey[w], uint32_t(sh.wpos[w]), best, bpos)) {
            best = sh.wkey[w];
            bpos = uint32_t(sh.wpos[w]);
            bslot = sh.wslot[w];
          }
        }
        const int64_t ci = int64_t(scope) * a.n_score_chunks + i0 / chunk;
        a.cand_key[ci] = best;
        a.cand_pos[ci] = int(bpos);
        a.cand_slot[ci] = bslot;
      }
    }
    // the appended token's vote and position, by the chunk that holds it
    if (a.append && i0 <= L - 1 && L - 1 < i1 && tid == 0) {
      if (a.votes) a.votes[sc + L - 1] = 1;
      a.pos[sc + L - 1] = a.t;
    }
  }
  // its rows: every workgroup of the scope copies units blockIdx.x, blockIdx.x + gridDim.x, ...
  if (a.append && int(blockIdx.x) < a.units) append_rows_wg(a, scope, L, blockIdx.x, gridDim.x);
}

// epi_score for scopes of one attention unit (per-KV-head caches), whose chunks
// hold 2048 / G tokens, TPT = 8 / G per thread. Everything the workgroup's
// first chunk reads -- the split partials, this workgroup's share of the output
// partials, the chunk's sub-chunk maxima, each thread's tokens (weights, shift
// counts, vote, utility, position) and the new token's rows -- is requested at
// entry, beside the live length (bounded by the chunk's end within the capacity
// and masked once the length is known), so the chunk waits on memory once. The
// split terms exp(M_split - M) are formed one per thread and summed per head in
// split order, so the arithmetic, its order and its results are epi_score's.
// Chunks past the launch's first (a device length beyond the sized bound) load
// as they go.
template <int G, int CH>
__device__ void epi_score_head(const StepArgs &a, ScoreLds &sh) {
  constexpr int TPT = 8 / G;
  constexpr int PPT = SCORE_PAIR_MAX / WG;                 // staged partials per thread
  constexpr int SPT = (8 * WG / CH + G + WG - 1) / WG;     // sub-chunk maxima per thread
  constexpr int OPT = 16;                                  // output partials per thread, prefetched
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int scope = blockIdx.y;
  const int cap = a.capacity;
  const int64_t sc = int64_t(scope) * cap;
  const bool step = a.mode != 0;
  const bool score = a.refresh && (step || a.s != nullptr);
  const double inv_heads = 1.0 / double(G);
  const double alpha = double(a.alpha);
  const float *ews = a.ews + int64_t(scope) * G * cap;
  const uint8_t *ewsh = a.ewsh + int64_t(scope) * G * cap;
  const int chunk = a.score_chunk;
  const int ns = a.n_splits, P = G * ns;
  const bool staged = P <= SCORE_PAIR_MAX;

  // ---- requests at entry (none waits for the length)
  const int Lraw = a.len[scope] + a.append;
  double lpm[PPT], lpz[PPT];
#pragma unroll
  for (int r = 0; r < PPT; ++r) {
    const int idx = tid + r * WG;
    lpm[r] = -INFINITY;
    lpz[r] = 0.0;
    if (staged && idx < P) {
      const int h = idx / ns, sp = idx - (idx / ns) * ns;
      const int64_t pi = (int64_t(scope) * ns + sp) * G + h;
      lpm[r] = a.partM[pi];
      lpz[r] = a.partZ[pi];
    }
  }
  // the output element (head blockIdx.x, element tid) when each workgroup has at most one head
  const bool pre_out = staged && ns <= OPT && int(gridDim.x) >= G;
  float po[OPT];
  if (pre_out && int(blockIdx.x) < G && tid < HD) {
#pragma unroll
    for (int sp = 0; sp < OPT; ++sp)
      po[sp] = sp < ns ? a.partO[((int64_t(scope) * ns + sp) * G + blockIdx.x) * HD + tid] : 0.f;
  }
  int i0 = blockIdx.x * chunk;
  const int iend = min(cap, i0 + chunk);   // the chunk's end before the length is known
  double lsm[SPT];
  {
    const int c0 = i0 / CH, nsc = i0 < iend ? (iend - 1) / CH - c0 + 1 : 0;
#pragma unroll
    for (int r = 0; r < SPT; ++r) {
      const int idx = tid + r * WG;
      lsm[r] = -INFINITY;
      if (score && idx < nsc * G) lsm[r] = a.subM[(int64_t(scope) * a.nsub_cap + c0 + idx / G) * G + idx % G];
    }
  }
  float ev[TPT][G];
  int evs[TPT][G], pv[TPT], pp[TPT];
  float mo[TPT];
  auto load_tokens = [&](int j0, int j1) {
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      const int i = j0 + tid + r * WG;
      const bool ok = i < j1;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        ev[r][g] = (score && ok) ? ews[int64_t(g) * cap + i] : 0.f;
        evs[r][g] = (score && ok) ? int(ewsh[int64_t(g) * cap + i]) : 0;
      }
      pv[r] = (score && ok && a.votes) ? a.votes[sc + i] : 1;
      mo[r] = (step && ok) ? a.m[sc + i] : 0.f;
      pp[r] = ok ? a.pos[sc + i] : 0;
    }
  };
  load_tokens(i0, iend);
  // the new token's rows (stored by the chunk that holds slot L - 1)
  const int nv = a.row_bytes / 16;
  const int64_t asrc = int64_t(scope) * a.units * a.row_bytes;
  u32x4 ak = u32x4(0u), av = u32x4(0u);
  if (a.append && a.units == 1 && tid < nv) {
    ak = ld16(a.k_new + asrc + 16 * tid);
    av = ld16(a.v_new + asrc + 16 * tid);
  }
  const int L = Lraw;
  if (a.steplen && blockIdx.x == 0 && tid == 0) a.steplen[scope] = L;   // for a split finish
  if (L > cap) return;   // reported by the finish kernel
  const int k = step ? max(0, L - a.budget) : 0;
  double *m64 = (step && k > 1 && a.m64) ? a.m64 + sc : nullptr;
  int i1 = min(L, i0 + chunk);
  int c0 = i0 / CH;
  int nsc = i0 < L ? (i1 - 1) / CH - c0 + 1 : 0;

  // ---- M per head; the split terms; Z, lse; the output weights and the chunk's factors
  if (staged) {
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int idx = tid + r * WG;
      if (idx < P) {
        sh.pm[idx] = lpm[r];
        sh.pz[idx] = lpz[r];
      }
    }
    __syncthreads();
    if (tid < G) {
      double M = -INFINITY;
      for (int sp = 0; sp < ns; ++sp) M = fmax(M, sh.pm[tid * ns + sp]);
      sh.M[tid] = M;
    }
    __syncthreads();
    // exp(M_split - M) per split, and its term of Z
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int idx = tid + r * WG;
      if (idx < P) {
        const double pm = lpm[r];
        const double e = pm > -INFINITY ? exp(pm - sh.M[idx / ns]) : 0.0;
        sh.pm[idx] = e;
        sh.pz[idx] = pm > -INFINITY ? lpz[r] * e : 0.0;
      }
    }
    __syncthreads();
    if (tid < G) {
      double Z = 0.0;
      for (int sp = 0; sp < ns; ++sp) Z += sh.pz[tid * ns + sp];
      sh.iZ[tid] = Z > 0.0 ? 1.0 / Z : 0.0;
      if (blockIdx.x == tid % gridDim.x) a.lse[int64_t(scope) * G + tid] = Z > 0.0 ? float(sh.M[tid] + log(Z)) : -INFINITY;
    }
  } else {
    if (tid < G) {
      double M, Z;
      combine_head<G>(a, scope, tid, M, Z);
      sh.M[tid] = M;
      sh.iZ[tid] = Z > 0.0 ? 1.0 / Z : 0.0;
      if (blockIdx.x == tid % gridDim.x) a.lse[int64_t(scope) * G + tid] = Z > 0.0 ? float(M + log(Z)) : -INFINITY;
    }
  }
  __syncthreads();
  if (staged) {
#pragma unroll
    for (int r = 0; r < PPT; ++r) {
      const int idx = tid + r * WG;
      if (idx < P) {
        const int h = idx / ns;
        sh.pm[idx] = (sh.iZ[h] > 0.0 && lpm[r] > -INFINITY) ? sh.pm[idx] * sh.iZ[h] : 0.0;
      }
    }
  }
  if (score) {
#pragma unroll
    for (int r = 0; r < SPT; ++r) {
      const int idx = tid + r * WG;
      if (idx < nsc * G) {
        const int h = idx % G;
        sh.fac[idx] = sh.iZ[h] > 0.0 ? exp(lsm[r] - sh.M[h]) * sh.iZ[h] : 0.0;
      }
    }
  }
  __syncthreads();
  if (pre_out) {
    if (int(blockIdx.x) < G && tid < HD) {
      const int h = blockIdx.x;
      float acc = 0.f;
#pragma unroll
      for (int sp = 0; sp < OPT; ++sp)
        if (sp < ns) acc = fmaf(po[sp], float(sh.pm[h * ns + sp]), acc);
      a.out[(int64_t(scope) * G + h) * HD + tid] = acc;
    }
  } else {
    for (int idx = tid; idx < G * HD; idx += WG) {
      const int h = idx / HD, e = idx - (idx / HD) * HD;
      if (h % gridDim.x != blockIdx.x) continue;
      float acc = 0.f;
      for (int sp = 0; sp < ns; ++sp) {
        const int64_t pi = (int64_t(scope) * ns + sp) * G + h;
        double wgt;
        if (staged) {
          wgt = sh.pm[h * ns + sp];
        } else {
          const double pm = a.partM[pi];
          wgt = (sh.iZ[h] > 0.0 && pm > -INFINITY) ? exp(pm - sh.M[h]) * sh.iZ[h] : 0.0;
        }
        acc = fmaf(a.partO[pi * HD + e], float(wgt), acc);
      }
      a.out[(int64_t(scope) * G + h) * HD + e] = acc;
    }
  }

  // ---- chunks: the first from the values requested at entry, later ones load as they go
  for (bool first = true; i0 < L; first = false) {
    if (!first) {
      __syncthreads();
      if (score)
        for (int idx = tid; idx < nsc * G; idx += WG) {
          const int h = idx % G;
          const double m = a.subM[(int64_t(scope) * a.nsub_cap + c0 + idx / G) * G + h];
          sh.fac[idx] = sh.iZ[h] > 0.0 ? exp(m - sh.M[h]) * sh.iZ[h] : 0.0;
        }
      load_tokens(i0, i1);
      __syncthreads();
    }
    uint64_t best = ~0ull;
    uint32_t bpos = 0xffffffffu;
    int bslot = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < TPT; ++r) {
      const int i = i0 + tid + r * WG;
      if (i >= i1) continue;
      const bool isnew = a.append && i == L - 1;
      double mval = 0.0;
      if (score) {
        const int p = isnew ? 1 : pv[r];
        const double *f = sh.fac + (i / CH - c0) * G;
        double acc = 0.0;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const double x = double(ev[r][g]) * f[g];
          acc += evs[r][g] ? x * shift_scale(evs[r][g]) : x;
        }
        const double sv = double(p) * acc * inv_heads;
        if (a.s) a.s[sc + i] = float(sv);
        if (step) {
          const double m_old = isnew ? 0.0 : double(mo[r]);
          mval = apply_rule(a.rule, alpha, m_old, sv);
          a.m[sc + i] = float(mval);
        }
      } else if (step) {
        mval = isnew ? 0.0 : double(mo[r]);
      }
      if (isnew && !(score && step)) a.m[sc + i] = 0.f;
      if (m64) m64[i] = mval;
      if (k == 1) {
        const uint64_t key = orderable_f64(mval);
        const uint32_t p = uint32_t(isnew ? a.t : pp[r]);
        if (key_pos_less(key, p, best, bpos)) {
          best = key;
          bpos = p;
          bslot = i;
        }
      }
    }
    if (k == 1) {   // (utility, position) pairs are distinct: the minimum names one slot
      wave_min_key_pos(best, bpos, bslot);
      if (lane == 0) {
        sh.wkey[wave] = best;
        sh.wslot[wave] = bslot;
        sh.wpos[wave] = int(bpos);
      }
      __syncthreads();
      if (tid == 0) {
#pragma unroll
        for (int w = 1; w < WG / 64; ++w) {
          if (key_pos_less(sh.wkey[w], uint32_t(sh.wpos[w]), best, bpos)) {
            best = sh.wkey[w];
            bpos = uint32_t(sh.wpos[w]);
            bslot = sh.wslot[w];
          }
        }
        const int64_t ci = int64_t(scope) * a.n_score_chunks + i0 / chunk;
        a.cand_key[ci] = best;
        a.cand_pos[ci] = int(bpos);
        a.cand_slot[ci] = bslot;
      }
    }
    if (a.append && i0 <= L - 1 && L - 1 < i1) {
      const int64_t arow = (int64_t(scope) * a.scope_stride + (L - 1)) * a.row_bytes;
      if (first && a.units == 1) {
        if (tid < nv) {
          st16(a.k + arow + 16 * tid, ak);
          st16(a.v + arow + 16 * tid, av);
        }
      } else {
        // one vector at a time: the batched copy's registers would be allocated for the
        // whole kernel, and this path (a later chunk, or several units) is rare here
        for (int idx = tid; idx < a.units * nv; idx += WG) {
          const int u = idx / nv, c = idx - (idx / nv) * nv;
          const int64_t row = (int64_t(scope) * a.scope_stride + int64_t(u) * a.unit_stride + (L - 1)) * a.row_bytes;
          const int64_t src = (int64_t(scope) * a.units + u) * a.row_bytes;
          st16(a.k + row + 16 * c, ld16(a.k_new + src + 16 * c));
          st16(a.v + row + 16 * c, ld16(a.v_new + src + 16 * c));
        }
      }
      if (tid == 0) {
        if (a.votes) a.votes[sc + L - 1] = 1;
        a.pos[sc + L - 1] = a.t;
      }
    }
    i0 += gridDim.x * chunk;
    i1 = min(L, i0 + chunk);
    c0 = i0 / CH;
    nsc = i0 < L ? (i1 - 1) / CH - c0 + 1 : 0;
  }
}

// ---------------------------------------------------------------- finish
// The evicted entry of a one-entry eviction: the lowest (utility, position) key
// over the score chunks' candidates (the whole workgroup; every thread returns it).
__device__ int finish_pick(const StepArgs &a, EpiLds &sh, int scope, int L) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nch = (L + a.score_chunk - 1) / a.score_chunk;
  uint64_t best = ~0ull;
  uint32_t bpos = 0xffffffffu;
  int bslot = 0x7fffffff;
  for (int c = tid; c < nch; c += WG) {
    const int64_t ci = int64_t(scope) * a.n_score_chunks + c;
    const uint64_t key = a.cand_key[ci];
    const uint32_t p = uint32_t(a.cand_pos[ci]);
    if (key_pos_less(key, p, best, bpos)) {
      best = key;
      bpos = p;
      bslot = a.cand_slot[ci];
    }
  }
  wave_min_key_pos(best, bpos, bslot);
  if (lane == 0) {
    sh.ckey[wave] = best;
    sh.cslot[wave] = bslot;
    sh.cpos[wave] = int(bpos);
  }
  __syncthreads();
  best = sh.ckey[0];
  bpos = uint32_t(sh.cpos[0]);
  int e1 = sh.cslot[0];
#pragma unroll
  for (int w = 1; w < WG / 64; ++w) {
    if (key_pos_less(sh.ckey[w], uint32_t(sh.cpos[w]), best, bpos)) {
      best = sh.ckey[w];
      bpos = uint32_t(sh.cpos[w]);
      e1 = sh.cslot[w];
    }
  }
  return e1;
}

// The rows of units y, y + ny, y + 2 ny, ... of the scope: slot src -> dst.
__device__ __forceinline__ void move_unit_rows_wg(const ScopeRows &r, int src, int dst, int y, int ny) {
  copy_rows_wg(
      (r.units - y + ny - 1) / ny, r.row_bytes / 16,
      [&](int i, const char *&ks, const char *&vs) {
        const int64_t off = ((r.row0 + int64_t(y + i * ny) * r.unit_stride) + src) * r.row_bytes;
        ks = r.k + off;
        vs = r.v + off;
      },
      [&](int i, char *&kd, char *&vd) {
        const int64_t off = ((r.row0 + int64_t(y + i * ny) * r.unit_stride) + dst) * r.row_bytes;
        kd = r.k + off;
        vd = r.v + off;
      });
}

// One workgroup per scope, or (gridDim.y > 1: a full step on multi-unit scopes
// without moments) gridDim.y of them: workgroup y moves the rows of units y,
// y + gridDim.y, ... into the evicted slot, and workgroup 0 does everything
// else. The live length then comes from the score kernel's copy (steplen),
// since workgroup 0 rewrites len while the others may still read it.
// MULTI false: one workgroup per scope and one unit per scope (the per-head
// finish kernel's fallback), without the code for several units.
template <typename T, int G, bool MULTI = true>
__device__ void epi_finish(const StepArgs &a, EpiLds &sh) {
  const int tid = threadIdx.x;
  const int scope = blockIdx.x;
  const int cap = a.capacity;
  const int64_t sc = int64_t(scope) * cap;
  const int row_bytes = HD * int(sizeof(T));
  const int ny = MULTI ? int(gridDim.y) : 1, y = MULTI ? int(blockIdx.y) : 0;
  const int L = ny > 1 ? a.steplen[scope] : a.len[scope] + a.append;
  if (y > 0) {   // the move of this workgroup's units, when one entry is evicted
    if (L > cap || a.mode != 1 || L - a.budget != 1) return;
    const int e = finish_pick(a, sh, scope, L);
    if (e < L - 1) {
      ScopeRows rows{a.k, a.v, int64_t(scope) * a.scope_stride, a.unit_stride, a.units, row_bytes,
                     nullptr, a.pos + sc, nullptr};
      move_unit_rows_wg(rows, L - 1, e, y, ny);
    }
    return;
  }
  if (L > cap) {
    if (tid == 0) {
      a.status[0] = -4;
      if (a.bulk) a.bulk[scope].run = 0;
      if (a.mode == 2) a.list[sc] = -1;   // nothing for the merge kernels
    }
    return;
  }

  const bool step = a.mode != 0;
  const int k = step ? max(0, L - a.budget) : 0;
  if (a.bulk) {
    if (k > 1) {   // the grid-wide kernels launched after this one take over
      if (tid == 0) {
        BulkScope &b = a.bulk[scope];
        b.prefix = 0;
        b.mask = 0;
        b.lprefix = 0;
        b.lmask = 0;
        b.krem = k;
        b.done = 0;
        b.L = L;
        b.k = k;
        b.B = L - k;
        b.n_pairs = 0;
        b.run = 1;
      }
      return;
    }
    if (tid == 0) a.bulk[scope].run = 0;
  }
  if (!step) {
    if (tid == 0) a.len[scope] = L;
    return;
  }
  // merge mode: list[0] of the scope names the entry the merge kernels take (-1: none)
  if (k <= 0) {
    if (a.evict_out)
      for (int i = tid; i < L; i += WG) a.evict_out[sc + i] = 0;
    if (tid == 0) {
      if (a.mode == 2) a.list[sc] = -1;
      a.len[scope] = L;
    }
    return;
  }
  if (a.mode == 2 && k > 1) {     // a merge handles one eviction per step
    if (tid == 0) {
      a.status[0] = -3;
      a.list[sc] = -1;
      a.len[scope] = L;
    }
    return;
  }

  // selection of the k lowest (m, pos)
  uint8_t *flags = a.flags + sc;
  int32_t *list = a.list + sc;
  int e1 = -1;
  if (k == 1) {
    e1 = finish_pick(a, sh, scope, L);
    if (a.evict_out)
      for (int i = tid; i < L; i += WG) a.evict_out[sc + i] = (i == e1);
    if (tid == 0) list[0] = e1;
  } else {
    // more than one eviction without the bulk kernels (a launch sized for at most
    // one, on a longer device length): one workgroup selects, folds and compacts,
    // ranking the float64 utilities the score kernel kept
    const double *mm = a.m64 + sc;
    const int32_t *pp = a.pos + sc;
    wg_select_f64_pos([&](int i) { return mm[i]; }, [&](int i) { return pp[i]; }, L, k, flags,
                      a.evict_out ? a.evict_out + sc : nullptr, list, sh.sel);
  }
  __threadfence_block();
  __syncthreads();

  // moment fold of the evicted rows, before they are overwritten
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

  // hole-filling compaction
  ScopeRows rows{a.k, a.v, int64_t(scope) * a.scope_stride, a.unit_stride, a.units, row_bytes,
                 a.votes ? a.votes + sc : nullptr, a.pos + sc, a.m + sc};
  if (k == 1) {
    if (e1 < L - 1) {
      if (ny > 1) {
        move_unit_rows_wg(rows, L - 1, e1, 0, ny);
        if (tid == 0) {
          if (rows.votes) rows.votes[e1] = rows.votes[L - 1];
          rows.pos[e1] = rows.pos[L - 1];
          if (rows.m) rows.m[e1] = rows.m[L - 1];
        }
      } else if (MULTI) {
        move_slot_wg(rows, L - 1, e1);
      } else {
        move_slot_wg<1>(rows, L - 1, e1);
      }
    }
  } else {
    wg_compact_flags(rows, flags, L, k, a.list2 + sc, sh.fold.red);
  }
  if (tid == 0) a.len[scope] = L - k;
}

// epi_finish for a full step (mode 1) on per-head scopes (one unit per scope):
// the loads that do not depend on the evicted slot -- the score chunks'
// candidates of the launch's length bound, the unit's moment sums, and (once
// the length is known) the last slot's row, vote, position and utility, which
// fill the hole -- are requested at entry, so a one-entry eviction waits on
// memory for the candidates and then for the evicted rows only. The fold adds
// fmaf(v_r, k_c, 0) to S and k, v to the sums as fold_slots / fold_commit do.
// Any other case (no eviction, several, a length over the capacity) is
// epi_finish's.
template <typename T, int G>
__device__ void epi_finish_head(const StepArgs &a, EpiLds &sh) {
  constexpr int RB = HD * int(sizeof(T)), NV = RB / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int scope = blockIdx.x;
  const int cap = a.capacity;
  const int64_t sc = int64_t(scope) * cap;
  // ---- requests at entry
  const int ncmax = min(a.n_score_chunks, (a.max_len + a.score_chunk - 1) / a.score_chunk);
  uint64_t pkey = ~0ull;
  uint32_t ppos = 0xffffffffu;
  int pslot = 0x7fffffff;
  if (tid < ncmax) {
    const int64_t ci = int64_t(scope) * a.n_score_chunks + tid;
    pkey = a.cand_key[ci];
    ppos = uint32_t(a.cand_pos[ci]);
    pslot = a.cand_slot[ci];
  }
  const int col = 4 * (tid & 31), row0 = tid >> 5;
  float *S = a.mom_S ? a.mom_S + int64_t(scope) * HD * HD : nullptr;
  float4 s4[16];
  float ssum = 0.f;
  if (S) {
#pragma unroll
    for (int j = 0; j < 16; ++j) s4[j] = *reinterpret_cast<const float4 *>(S + (row0 + 8 * j) * HD + col);
    ssum = tid < HD ? a.mom_sk[int64_t(scope) * HD + tid] : a.mom_sv[int64_t(scope) * HD + tid - HD];
  }
  const int L = a.len[scope] + a.append;
  if (L > cap || L - a.budget != 1 || a.mode != 1 || (a.bulk && L - a.budget > 1)) {
    epi_finish<T, G, false>(a, sh);
    return;
  }
  const char *Kb = a.k + int64_t(scope) * a.scope_stride * RB;
  const char *Vb = a.v + int64_t(scope) * a.scope_stride * RB;
  u32x4 lk = u32x4(0u), lv = u32x4(0u);
  if (tid < NV) {
    lk = ld16(Kb + int64_t(L - 1) * RB + 16 * tid);
    lv = ld16(Vb + int64_t(L - 1) * RB + 16 * tid);
  }
  int lvote = 0, lpos = 0;
  float lm = 0.f;
  if (tid == 0) {
    if (a.votes) lvote = a.votes[sc + L - 1];
    lpos = a.pos[sc + L - 1];
    lm = a.m[sc + L - 1];
  }
  if (a.bulk && tid == 0) a.bulk[scope].run = 0;

  // ---- the evicted entry: the lowest (utility, position) key over the chunks
  const int nch = (L + a.score_chunk - 1) / a.score_chunk;
  uint64_t best = ~0ull;
  uint32_t bpos = 0xffffffffu;
  int bslot = 0x7fffffff;
  if (tid < nch && tid < ncmax) {
    best = pkey;
    bpos = ppos;
    bslot = pslot;
  }
  for (int c = tid < ncmax ? tid + WG : tid; c < nch; c += WG) {
    const int64_t ci = int64_t(scope) * a.n_score_chunks + c;
    const uint64_t key = a.cand_key[ci];
    const uint32_t p = uint32_t(a.cand_pos[ci]);
    const int sl = a.cand_slot[ci];
    if (key_pos_less(key, p, best, bpos)) {
      best = key;
      bpos = p;
      bslot = sl;
    }
  }
  wave_min_key_pos(best, bpos, bslot);
  if (lane == 0) {
    sh.ckey[wave] = best;
    sh.cslot[wave] = bslot;
    sh.cpos[wave] = int(bpos);
  }
  __syncthreads();
  best = sh.ckey[0];
  bpos = uint32_t(sh.cpos[0]);
  int e1 = sh.cslot[0];
#pragma unroll
  for (int w = 1; w < WG / 64; ++w) {
    if (key_pos_less(sh.ckey[w], uint32_t(sh.cpos[w]), best, bpos)) {
      best = sh.ckey[w];
      bpos = uint32_t(sh.cpos[w]);
      e1 = sh.cslot[w];
    }
  }
  if (a.evict_out)
    for (int i = tid; i < L; i += WG) a.evict_out[sc + i] = (i == e1);

  // ---- fold of the evicted rows (read before the hole is filled)
  if (S) {
    const T *Kt = reinterpret_cast<const T *>(Kb), *Vt = reinterpret_cast<const T *>(Vb);
    if (tid < HD) sh.fold.kb[0][tid] = load_elem<T>(Kt, int64_t(e1) * HD + tid);
    else sh.fold.vb[0][tid - HD] = load_elem<T>(Vt, int64_t(e1) * HD + tid - HD);
    __syncthreads();
    const float4 k4 = *reinterpret_cast<const float4 *>(&sh.fold.kb[0][col]);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float va = sh.fold.vb[0][row0 + 8 * j];
      float4 x = s4[j];
      x.x += fmaf(va, k4.x, 0.f);
      x.y += fmaf(va, k4.y, 0.f);
      x.z += fmaf(va, k4.z, 0.f);
      x.w += fmaf(va, k4.w, 0.f);
      *reinterpret_cast<float4 *>(S + (row0 + 8 * j) * HD + col) = x;
    }
    const float add = 0.f + (tid < HD ? sh.fold.kb[0][tid] : sh.fold.vb[0][tid - HD]);
    if (tid < HD) a.mom_sk[int64_t(scope) * HD + tid] = ssum + add;
    else a.mom_sv[int64_t(scope) * HD + tid - HD] = ssum + add;
    if (tid == 0) a.mom_n[scope] += 1;
  }

  // ---- the last slot fills the hole
  if (e1 < L - 1) {
    if (tid < NV) {
      st16(const_cast<char *>(Kb) + int64_t(e1) * RB + 16 * tid, lk);
      st16(const_cast<char *>(Vb) + int64_t(e1) * RB + 16 * tid, lv);
    }
    if (tid == 0) {
      if (a.votes) a.votes[sc + e1] = lvote;
      a.pos[sc + e1] = lpos;
      a.m[sc + e1] = lm;
    }
  }
  if (tid == 0) a.len[scope] = L - 1;
}

}  // namespace kvc
