// Consecutive attention groups of a scope that cannot evict: the layers after
// the first of a model-scope decode step (InertiaKV §3.1: one slot set per
// sequence shared by every layer, the utility updated after every compressed
// layer; the first layer has already evicted to the budget, so the later ones
// only attend, score and update). Three launches cover all the groups:
//
//   k_decode_split (decode_split.hip) over every unit of every group: split-K
//     attention, per-token weights and sub-chunk maxima to the workspace;
//   k_groups_combine, one workgroup per unit: each head's M, Z, lse and output
//     over the split partials;
//   k_groups_score, (token chunk, scope) workgroups: each group's score
//     s_j(i) = mean over the group's heads of p_i e F, and the group-by-group
//     utility chain in closed form, m <- rule_j(... rule_0(m, s_0) ..., s_j):
//       single      m = s_{n-1}
//       cumulative  m = m + sum_j s_j
//       EMA         m = alpha^n m + sum_j (1 - alpha) alpha^(n-1-j) s_j
//     in float64, stored once as float32.
#include <algorithm>

#include "kvc_device.h"
#include "kvc_groups.h"

namespace kvc {

namespace {

constexpr int GROUPS_CT = 32;               // tokens per score workgroup
constexpr int GROUPS_PARTS = WG / GROUPS_CT;  // threads per token (each takes every PARTS-th group)
constexpr int GROUPS_NS_MAX = 64;           // split partials per head the combine stages

template <int G>
__global__ __launch_bounds__(HD) void k_groups_combine(const GroupsArgs a) {
  __shared__ double wgt[G][GROUPS_NS_MAX];
  __shared__ double sM[G], sIZ[G];
  const int gu = blockIdx.x, tid = threadIdx.x, ns = a.n_splits;
  const int64_t pb = int64_t(gu) * ns;
  if (tid < G) {
    const int g = tid;
    double M = -INFINITY;
    for (int sp = 0; sp < ns; ++sp) M = fmax(M, a.partM[(pb + sp) * G + g]);
    double Z = 0.0;
    for (int sp = 0; sp < ns; ++sp) {
      const double pm = a.partM[(pb + sp) * G + g];
      if (pm > -INFINITY) Z += a.partZ[(pb + sp) * G + g] * exp(pm - M);
    }
    const double iZ = Z > 0.0 ? 1.0 / Z : 0.0;
    for (int sp = 0; sp < ns; ++sp) {
      const double pm = a.partM[(pb + sp) * G + g];
      wgt[g][sp] = (iZ > 0.0 && pm > -INFINITY) ? exp(pm - M) * iZ : 0.0;
    }
    sM[g] = M;
    sIZ[g] = iZ;
    a.lse[int64_t(gu) * G + g] = Z > 0.0 ? float(M + log(Z)) : -INFINITY;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float acc = 0.f;
    for (int sp = 0; sp < ns; ++sp) acc = fmaf(a.partO[((pb + sp) * G + g) * HD + tid], float(wgt[g][sp]), acc);
    st_nt(&a.out[(int64_t(gu) * G + g) * HD + tid], acc);
  }
  // M and 1/Z for the score kernel, over split 0's partials (every read of them is above the barrier)
  if (tid < G) {
    a.partM[pb * G + tid] = sM[tid];
    a.partZ[pb * G + tid] = sIZ[tid];
  }
}

// Thread (token t, part p) of a workgroup sums the groups p, p + PARTS, ... for
// token i0 + t; the parts are then added in order, so the result does not
// depend on scheduling.
template <int G, int CH>
__global__ __launch_bounds__(WG) void k_groups_score(const GroupsArgs a) {
  extern __shared__ double fac[];   // [units * G][NSC]: exp(m_c - M) / Z per head and sub-chunk
  constexpr int CT = GROUPS_CT, PARTS = GROUPS_PARTS, NSC = CT / CH;
  static_assert(CT % CH == 0, "score chunks are whole sub-chunks");
  __shared__ double red_t[PARTS][CT], red_l[PARTS][CT];
  const int tid = threadIdx.x, scope = blockIdx.y;
  const int cap = a.capacity, H = a.units * G, ns = a.n_splits;
  int L = a.len[scope];
  if (L > cap) L = 0;
  const int64_t sc = int64_t(scope) * cap;
  const int gu0 = scope * a.units;
  const int tok = tid % CT, part = tid / CT;
  const int n = a.n_groups, gsz = a.group_units;
  const double alpha = a.alpha;
  const double inv_heads = 1.0 / double(gsz * G);
  for (int i0 = blockIdx.x * CT; i0 < L; i0 += gridDim.x * CT) {
    const int c0 = i0 / CH;
    __syncthreads();   // the previous chunk's reads of fac and red are done
    for (int idx = tid; idx < H * NSC; idx += WG) {
      const int h = idx / NSC, cl = idx - (idx / NSC) * NSC;
      const int64_t gu = gu0 + h / G;
      const int g = h % G, c = c0 + cl;
      double f = 0.0;
      if (c * CH < L) {
        const double M = a.partM[gu * ns * G + g], iZ = a.partZ[gu * ns * G + g];
        const double sm = a.subM[(gu * a.nsub_cap + c) * G + g];
        f = iZ > 0.0 ? exp(sm - M) * iZ : 0.0;
      }
      fac[idx] = f;
    }
    __syncthreads();
    const int i = i0 + tok;
    double tot = 0.0, last = 0.0;
    if (i < L) {
      const int cl = tok / CH;
      for (int j = part; j < n; j += PARTS) {
        double acc = 0.0;
        // UB units' weights loaded before any is used (their loads overlap), then summed in order
        constexpr int UB = G >= 4 ? 4 : 8 / G;
        for (int u0 = j * gsz; u0 < (j + 1) * gsz; u0 += UB) {
          float ev[UB][G];
          int sv[UB][G];
#pragma unroll
          for (int uu = 0; uu < UB; ++uu)
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const int u = min(u0 + uu, (j + 1) * gsz - 1);
              const int64_t wi = ((int64_t(gu0) + u) * G + g) * cap + i;
              ev[uu][g] = a.ews[wi];
              sv[uu][g] = a.ewsh[wi];
            }
#pragma unroll
          for (int uu = 0; uu < UB; ++uu) {
            if (u0 + uu >= (j + 1) * gsz) break;
#pragma unroll
            for (int g = 0; g < G; ++g) {
              const double x = double(ev[uu][g]) * fac[((u0 + uu) * G + g) * NSC + cl];
              acc += sv[uu][g] ? x * shift_scale(sv[uu][g]) : x;
            }
          }
        }
        const double sj = acc * inv_heads;
        if (j == n - 1) last = sj;
        tot += (a.rule == 2 ? (1.0 - alpha) * pow(alpha, double(n - 1 - j)) : 1.0) * sj;
      }
    }
    red_t[part][tok] = tot;
    red_l[part][tok] = last;
    __syncthreads();
    if (part == 0 && i < L) {
      double t = 0.0, l = 0.0;
#pragma unroll
      for (int p = 0; p < PARTS; ++p) {
        t += red_t[p][tok];
        l += red_l[p][tok];
      }
      const double pv = a.votes ? double(a.votes[sc + i]) : 1.0;
      t *= pv;
      l *= pv;
      const double mo = double(ld_nt(&a.m[sc + i]));
      const double mv = a.rule == 0 ? l : a.rule == 1 ? mo + t : pow(alpha, double(n)) * mo + t;
      st_nt(&a.m[sc + i], float(mv));
      if (a.s) st_nt(&a.s[sc + i], float(l));
    }
  }
}

// The same chain over the per-unit kernel's weight sums: s_j(i) = sum over the
// group's units of wsum[unit][i] / (group_units * G) (votes already applied).
__global__ __launch_bounds__(WG) void k_groups_wscore(const GroupsArgs a, int G) {
  constexpr int CT = GROUPS_CT, PARTS = GROUPS_PARTS;
  __shared__ double red_t[PARTS][CT], red_l[PARTS][CT];
  const int tid = threadIdx.x, scope = blockIdx.y;
  const int cap = a.capacity;
  int L = a.len[scope];
  if (L > cap || L > a.max_len) L = 0;   // the per-unit kernel wrote nothing (status reported there)
  const int64_t sc = int64_t(scope) * cap;
  const int64_t gu0 = int64_t(scope) * a.units;
  const int tok = tid % CT, part = tid / CT;
  const int n = a.n_groups, gsz = a.group_units;
  const double alpha = a.alpha;
  const double inv_heads = 1.0 / double(gsz * G);
  for (int i0 = blockIdx.x * CT; i0 < L; i0 += gridDim.x * CT) {
    __syncthreads();   // the previous chunk's reads of red are done
    const int i = i0 + tok;
    double tot = 0.0, last = 0.0;
    if (i < L) {
      for (int j = part; j < n; j += PARTS) {
        const double *w = a.wsum + (gu0 + int64_t(j) * gsz) * a.wsum_stride + i;
        double acc = 0.0;
        constexpr int UB = 8;
        for (int u0 = 0; u0 < gsz; u0 += UB) {
          double x[UB];
#pragma unroll
          for (int uu = 0; uu < UB; ++uu) x[uu] = w[int64_t(min(u0 + uu, gsz - 1)) * a.wsum_stride];
#pragma unroll
          for (int uu = 0; uu < UB; ++uu)
            if (u0 + uu < gsz) acc += x[uu];
        }
        const double sj = acc * inv_heads;
        if (j == n - 1) last = sj;
        tot += (a.rule == 2 ? (1.0 - alpha) * pow(alpha, double(n - 1 - j)) : 1.0) * sj;
      }
    }
    red_t[part][tok] = tot;
    red_l[part][tok] = last;
    __syncthreads();
    if (part == 0 && i < L) {
      double t = 0.0, l = 0.0;
#pragma unroll
      for (int p = 0; p < PARTS; ++p) {
        t += red_t[p][tok];
        l += red_l[p][tok];
      }
      const double mo = double(ld_nt(&a.m[sc + i]));
      const double mv = a.rule == 0 ? l : a.rule == 1 ? mo + t : pow(alpha, double(n)) * mo + t;
      st_nt(&a.m[sc + i], float(mv));
      if (a.s) st_nt(&a.s[sc + i], float(l));
    }
  }
}

template <int G, int CH>
hipError_t launch_groups_tg(const GroupsArgs &g, bool score, int n_chunks, size_t lds, hipStream_t st) {
  hipLaunchKernelGGL((k_groups_combine<G>), dim3(g.n_scopes * g.units), dim3(HD), 0, st, g);
  if (score) hipLaunchKernelGGL((k_groups_score<G, CH>), dim3(n_chunks, g.n_scopes), dim3(WG), lds, st, g);
  return hipGetLastError();
}

template <int CH>
hipError_t launch_groups_t(const GroupsArgs &g, int G, bool score, int n_chunks, size_t lds, hipStream_t st) {
  switch (G) {
    case 1: return launch_groups_tg<1, CH>(g, score, n_chunks, lds, st);
    case 2: return launch_groups_tg<2, CH>(g, score, n_chunks, lds, st);
    case 4: return launch_groups_tg<4, CH>(g, score, n_chunks, lds, st);
    case 8: return launch_groups_tg<8, CH>(g, score, n_chunks, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int groups_score_chunk(int) { return GROUPS_CT; }

size_t groups_score_lds_bytes(int dtype, int G, int units) {
  return size_t(units) * G * (GROUPS_CT / decode_chunk_tokens(dtype)) * sizeof(double);
}

hipError_t launch_groups_wscore(const GroupsArgs &g, int G, hipStream_t st) {
  const int n_chunks = std::max(1, (g.max_len + GROUPS_CT - 1) / GROUPS_CT);
  hipLaunchKernelGGL(k_groups_wscore, dim3(n_chunks, g.n_scopes), dim3(WG), 0, st, g, G);
  return hipGetLastError();
}

hipError_t launch_groups_epilogue(const GroupsArgs &g, int dtype, int G, bool score, hipStream_t st) {
  if (g.n_splits > GROUPS_NS_MAX) return hipErrorInvalidValue;
  const int n_chunks = std::max(1, (g.max_len + GROUPS_CT - 1) / GROUPS_CT);
  const size_t lds = groups_score_lds_bytes(dtype, G, g.units);
  const int CH = decode_chunk_tokens(dtype);
  if (CH == 16) return launch_groups_t<16>(g, G, score, n_chunks, lds, st);
  if (CH == 8) return launch_groups_t<8>(g, G, score, n_chunks, lds, st);
  return hipErrorInvalidValue;
}

}  // namespace kvc
