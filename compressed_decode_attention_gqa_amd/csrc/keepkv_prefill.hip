// KeepKV prefill compression by greedy all-pairs ZIP merging (reading notes on
// KeepKV: the inference algorithm's prefill steps 2-5 and the paragraphs on
// candidate choice): while a per-head scope holds more than B live entries,
// the pair of candidate entries (position < protect_from) whose keys have the
// largest cosine is ZIP-merged (eqs. (7), (10), (12) with the guard) under the
// group-mean reference logits, and the merged entry replaces the pair in the
// slot of the older one. Ties: cosine descending, then the pair's lower
// position, then its higher position.
//
// Kernels, in launch order:
//   k_pm_prep    key norms (float64) and the candidate flags of every slot.
//   k_pm_rows    each candidate's best partner: the block's 128 candidate keys
//                are the float64 MFMA operator of kvc_f64mfma.h (transposed
//                use), 16 keys per tile are the A operand, so a lane holds the
//                dot products of 8 rows x 4 tokens; cos = dot / (|k_i| |k_j|).
//   k_pm_loop    one workgroup per scope runs the greedy loop: the pair is the
//                row of largest best-cosine (ties to the lower position) and its
//                partner; after the merge only the merged row and the rows whose
//                best partner was one of the pair are recomputed, and every other
//                row takes the merged entry as partner when it beats its best.
// Products of the cache's bf16 (or fp32) keys are exact in float64, so the
// cosines equal the ones of the float64 oracle up to the rounding of the sums.
#include "kvc_f64mfma.h"
#include "kvc_kernels.h"

namespace kvc {
namespace {

constexpr int PM_NT = 512;       // k_pm_rows: 8 waves, two per SIMD
constexpr int PM_LOOP = 1024;    // k_pm_loop: 16 waves
constexpr int PM_ORPH = 1024;    // orphan rows recomputed per batch

// (cos, pos) order: higher cosine first, then the lower position.
__device__ __forceinline__ bool pm_better(double c1, int p1, double c2, int p2) {
  return c1 > c2 || (c1 == c2 && p1 < p2);
}

template <typename T>
__global__ __launch_bounds__(256) void k_pm_prep(PrefillMergeArgs p) {
  const int sc = blockIdx.y, i = blockIdx.x * 256 + threadIdx.x;
  if (i >= p.capacity) return;
  const int L = min(p.len[sc], p.capacity);
  const int64_t slot = int64_t(sc) * p.capacity + i;
  const T *kr = reinterpret_cast<const T *>(p.k) + (int64_t(sc) * p.scope_stride + i) * HD;
  double n = 0.0;
  if (i < L) {
#pragma unroll 8
    for (int b = 0; b < HD; ++b) {
      const double x = double(load_elem<T>(kr, b));
      n = fma(x, x, n);
    }
  }
  p.norm[slot] = sqrt(n);
  p.cand[slot] = (i < L && p.pos[slot] < p.protect_from) ? 1 : 0;
  p.rowarg[slot] = -1;
  p.rowmax[slot] = -INFINITY;
  if (i < L) p.evict[slot] = 0;
}

// grid (row blocks of 128, scopes), 512 threads; every token of the scope.
template <typename T>
__global__ __launch_bounds__(PM_NT, 1) void k_pm_rows(PrefillMergeArgs p) {
  __shared__ FmOperator op;
  __shared__ double bcos[PM_NT / 64][128];
  __shared__ int bpos[PM_NT / 64][128], bslot[PM_NT / 64][128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = blockIdx.x * 128, sc = blockIdx.y;
  const int L = min(p.len[sc], p.capacity);
  const int t0 = 0, t1 = L;
  if (rb >= L) return;
  const int64_t so = int64_t(sc) * p.capacity;
  const T *Kb = reinterpret_cast<const T *>(p.k) + int64_t(sc) * p.scope_stride * HD;
  for (int e = tid; e < HD * HD; e += PM_NT) {
    const int r = e >> 7, b = e & 127, row = rb + r;
    const double v = (row < L && p.cand[so + row]) ? double(load_elem<T>(Kb, int64_t(row) * HD + b)) : 0.0;
    fm_put_t(op, r, b, v);
  }
  const int jl = lane & 15, tq = lane >> 4;
  double nrow[FM_RT], best[FM_RT];
  int bp[FM_RT], bs[FM_RT];
  bool rc[FM_RT];
#pragma unroll
  for (int ct = 0; ct < FM_RT; ++ct) {
    const int row = rb + 16 * ct + jl;
    rc[ct] = row < L && p.cand[so + row];
    nrow[ct] = rc[ct] ? p.norm[so + row] : 0.0;
    best[ct] = -INFINITY;
    bp[ct] = 0x7fffffff;
    bs[ct] = -1;
  }
  __syncthreads();
  constexpr int ES = sizeof(T);
  const char *Kc = reinterpret_cast<const char *>(Kb);
  const int n16 = (t1 - t0 + FM_TILE - 1) / FM_TILE;
  for (int t = wave; t < n16; t += PM_NT / 64) {
    const int tb = t0 + t * FM_TILE;
    FmRow<T> kr;
    kr.load(Kc + (int64_t(min(tb + jl, t1 - 1)) * HD + 32 * tq) * ES);
    double x[32];
#pragma unroll
    for (int s = 0; s < 32; ++s) x[s] = kr.get(s);
    fm_d4 acc[FM_RT];
#pragma unroll
    for (int ct = 0; ct < FM_RT; ++ct) acc[ct] = fm_d4{0.0, 0.0, 0.0, 0.0};
    fm_apply_t(op, lane, x, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = tb + tq + 4 * r;
      const int jc = min(j, t1 - 1);
      const bool cj = j < t1 && p.cand[so + jc];
      const double nj = p.norm[so + jc];
      const int pj = p.pos[so + jc];
#pragma unroll
      for (int ct = 0; ct < FM_RT; ++ct) {
        const int row = rb + 16 * ct + jl;
        if (rc[ct] && cj && j != row) {
          const double den = nrow[ct] * nj;
          const double c = den > 0.0 ? acc[ct][r] / den : 0.0;
          if (pm_better(c, pj, best[ct], bp[ct])) {
            best[ct] = c;
            bp[ct] = pj;
            bs[ct] = j;
          }
        }
      }
    }
  }
  // rows 16 ct + jl: combine the four token groups of the wave, then the waves
#pragma unroll
  for (int ct = 0; ct < FM_RT; ++ct) {
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const double c2 = __shfl_xor(best[ct], o);
      const int p2 = __shfl_xor(bp[ct], o), s2 = __shfl_xor(bs[ct], o);
      if (s2 >= 0 && (bs[ct] < 0 || pm_better(c2, p2, best[ct], bp[ct]))) {
        best[ct] = c2;
        bp[ct] = p2;
        bs[ct] = s2;
      }
    }
    if (tq == 0) {
      bcos[wave][16 * ct + jl] = best[ct];
      bpos[wave][16 * ct + jl] = bp[ct];
      bslot[wave][16 * ct + jl] = bs[ct];
    }
  }
  __syncthreads();
  if (tid < 128 && rb + tid < L && p.cand[so + rb + tid]) {
    double c = -INFINITY;
    int pp = 0x7fffffff, ss = -1;
    for (int wv = 0; wv < PM_NT / 64; ++wv) {
      const int s2 = bslot[wv][tid];
      if (s2 >= 0 && (ss < 0 || pm_better(bcos[wv][tid], bpos[wv][tid], c, pp))) {
        c = bcos[wv][tid];
        pp = bpos[wv][tid];
        ss = s2;
      }
    }
    p.rowmax[so + rb + tid] = c;
    p.rowarg[so + rb + tid] = ss;
  }
}

struct LoopLds {
  double kn[HD];            // the key whose row is being computed (float64)
  double red_c[PM_LOOP / 64];
  int red_p[PM_LOOP / 64], red_s[PM_LOOP / 64];
  double lbar[2];
  double wgt[4];
  int orph[PM_ORPH];
  int n_orph, more, pick_i, pick_j;
  double nk;
};

// Workgroup-wide best (c, p, s) by pm_better over the threads' candidates; result in sh.
__device__ __forceinline__ void loop_argmax(LoopLds &sh, double c, int pp, int ss, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double c2 = __shfl_xor(c, o);
    const int p2 = __shfl_xor(pp, o), s2 = __shfl_xor(ss, o);
    if (s2 >= 0 && (ss < 0 || pm_better(c2, p2, c, pp))) {
      c = c2;
      pp = p2;
      ss = s2;
    }
  }
  if (lane == 0) {
    sh.red_c[wave] = c;
    sh.red_p[wave] = pp;
    sh.red_s[wave] = ss;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < PM_LOOP / 64; ++w)
      if (sh.red_s[w] >= 0 && (sh.red_s[0] < 0 || pm_better(sh.red_c[w], sh.red_p[w], sh.red_c[0], sh.red_p[0]))) {
        sh.red_c[0] = sh.red_c[w];
        sh.red_p[0] = sh.red_p[w];
        sh.red_s[0] = sh.red_s[w];
      }
  }
  __syncthreads();
}

// Best partner of row `row` (its key in sh.kn, norm sh.nk) over the candidates.
template <typename T>
__device__ __forceinline__ void loop_row(const PrefillMergeArgs &p, LoopLds &sh, const T *Kb, int64_t so, int L,
                                         int row, int tid) {
  double c = -INFINITY;
  int pp = 0x7fffffff, ss = -1;
  for (int j = tid; j < L; j += PM_LOOP) {
    if (j == row || !p.cand[so + j]) continue;
    double dot = 0.0;
    for (int b = 0; b < HD; ++b) dot = fma(sh.kn[b], double(load_elem<T>(Kb, int64_t(j) * HD + b)), dot);
    const double den = sh.nk * p.norm[so + j];
    const double cs = den > 0.0 ? dot / den : 0.0;
    const int pj = p.pos[so + j];
    if (pm_better(cs, pj, c, pp)) {
      c = cs;
      pp = pj;
      ss = j;
    }
  }
  loop_argmax(sh, c, pp, ss, tid);
  if (tid == 0) {
    p.rowmax[so + row] = sh.red_s[0] >= 0 ? sh.red_c[0] : -INFINITY;
    p.rowarg[so + row] = sh.red_s[0];
  }
}

template <typename T>
__global__ __launch_bounds__(PM_LOOP) void k_pm_loop(PrefillMergeArgs p) {
  __shared__ LoopLds sh;
  const int sc = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = min(p.len[sc], p.capacity);
  const int64_t so = int64_t(sc) * p.capacity;
  T *Kw = reinterpret_cast<T *>(p.k) + int64_t(sc) * p.scope_stride * HD;
  T *Vw = reinterpret_cast<T *>(p.v) + int64_t(sc) * p.scope_stride * HD;
  const T *Kb = Kw;
  int live = L, merged = 0;
  while (live > p.budget) {
    // ---- the pair: the row of largest best-cosine (ties to the lower position) and its partner
    {
      double c = -INFINITY;
      int pp = 0x7fffffff, ss = -1;
      for (int i = tid; i < L; i += PM_LOOP) {
        if (!p.cand[so + i] || p.rowarg[so + i] < 0) continue;
        const double ci = p.rowmax[so + i];
        const int pi = p.pos[so + i];
        if (pm_better(ci, pi, c, pp)) {
          c = ci;
          pp = pi;
          ss = i;
        }
      }
      loop_argmax(sh, c, pp, ss, tid);
    }
    const int si = sh.red_s[0];
    if (si < 0) {   // fewer than two entries may merge: the budget cannot be reached
      if (tid == 0) p.status[0] = -4;
      break;
    }
    const int sj = p.rowarg[so + si];
    // the older entry of the pair survives; the other is removed
    const bool older = p.pos[so + si] < p.pos[so + sj];
    const int surv = older ? si : sj, gone = older ? sj : si;
    // ---- reference logits of the two entries (group-mean query)
    if (wave < 2) {
      const int x = wave == 0 ? gone : surv;
      const T *q = reinterpret_cast<const T *>(p.q) + int64_t(sc) * p.G * HD;
      double acc = 0.0;
      for (int j = lane; j < HD; j += 64) {
        const double kx = double(load_elem<T>(Kb, int64_t(x) * HD + j));
        double qs = 0.0;
        for (int g = 0; g < p.G; ++g) qs += double(load_elem<T>(q, g * HD + j)) * kx;
        acc += qs;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) acc += __shfl_xor(acc, o);
      if (lane == 0) sh.lbar[wave] = acc * p.scale / double(p.G);
    }
    __syncthreads();
    if (tid == 0) {
      const double le = sh.lbar[0], lc = sh.lbar[1];
      const double mu = fmax(le, lc);
      const double pe = double(p.votes[so + gone]), pc = double(p.votes[so + surv]);
      const double we = pe * exp(le - mu), wc = pc * exp(lc - mu);
      const double num = mu + log(we + wc) - log(pe + pc);
      const double den = we * le + wc * lc;
      const bool guarded = fabs(den) < double(p.eps) * exp(-mu);
      sh.wgt[0] = we / (we + wc);
      sh.wgt[1] = wc / (we + wc);
      sh.wgt[2] = guarded ? 0.5 : we * num / den;
      sh.wgt[3] = guarded ? 0.5 : wc * num / den;
    }
    __syncthreads();
    if (tid < HD) {   // element tid of the two rows; the merged row rounded to the cache dtype
      const double kek = double(load_elem<T>(Kb, int64_t(gone) * HD + tid));
      const double kck = double(load_elem<T>(Kb, int64_t(surv) * HD + tid));
      const double vek = double(load_elem<T>(Vw, int64_t(gone) * HD + tid));
      const double vck = double(load_elem<T>(Vw, int64_t(surv) * HD + tid));
      store_elem<T>(Kw, int64_t(surv) * HD + tid, float(sh.wgt[2] * kek + sh.wgt[3] * kck));
      store_elem<T>(Vw, int64_t(surv) * HD + tid, float(sh.wgt[0] * vek + sh.wgt[1] * vck));
      sh.kn[tid] = double(load_elem<T>(Kw, int64_t(surv) * HD + tid));
    }
    if (tid == 0) {
      p.votes[so + surv] += p.votes[so + gone];
      if (p.m) p.m[so + surv] += p.m[so + gone];
      p.cand[so + gone] = 0;
      p.evict[so + gone] = 1;
      if (p.pairs) {
        p.pairs[(so + merged) * 2] = surv;
        p.pairs[(so + merged) * 2 + 1] = gone;
      }
      sh.n_orph = 0;
      sh.more = 0;
    }
    __threadfence_block();
    __syncthreads();
    if (wave == 0) {
      double n = 0.0;
      for (int b = lane; b < HD; b += 64) n = fma(sh.kn[b], sh.kn[b], n);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) n += __shfl_xor(n, o);
      if (lane == 0) {
        sh.nk = sqrt(n);
        p.norm[so + surv] = sh.nk;
      }
    }
    __syncthreads();
    // ---- the merged row against every candidate; others adopt it when it beats their best,
    // rows whose best partner was one of the pair become orphans
    {
      const int ps = p.pos[so + surv];
      double c = -INFINITY;
      int pp = 0x7fffffff, ss = -1;
      for (int j = tid; j < L; j += PM_LOOP) {
        if (j == surv || !p.cand[so + j]) continue;
        double dot = 0.0;
        for (int b = 0; b < HD; ++b) dot = fma(sh.kn[b], double(load_elem<T>(Kb, int64_t(j) * HD + b)), dot);
        const double den = sh.nk * p.norm[so + j];
        const double cs = den > 0.0 ? dot / den : 0.0;
        const int pj = p.pos[so + j];
        if (pm_better(cs, pj, c, pp)) {
          c = cs;
          pp = pj;
          ss = j;
        }
        const int ra = p.rowarg[so + j];
        if (ra == surv || ra == gone) {
          const int k = atomicAdd(&sh.n_orph, 1);
          if (k < PM_ORPH) sh.orph[k] = j;
          else p.rowarg[so + j] = -2;      // recomputed in a later batch
        } else if (ra < 0 || pm_better(cs, ps, p.rowmax[so + j], p.pos[so + ra])) {
          p.rowmax[so + j] = cs;
          p.rowarg[so + j] = surv;
        }
      }
      loop_argmax(sh, c, pp, ss, tid);
      if (tid == 0) {
        p.rowmax[so + surv] = sh.red_s[0] >= 0 ? sh.red_c[0] : -INFINITY;
        p.rowarg[so + surv] = sh.red_s[0];
      }
    }
    __threadfence_block();
    __syncthreads();
    // ---- orphans, in batches of PM_ORPH
    for (;;) {
      const int n = min(sh.n_orph, PM_ORPH);
      for (int k = 0; k < n; ++k) {
        const int o = sh.orph[k];
        if (tid < HD) sh.kn[tid] = double(load_elem<T>(Kb, int64_t(o) * HD + tid));
        if (tid == 0) sh.nk = p.norm[so + o];
        __syncthreads();
        loop_row<T>(p, sh, Kb, so, L, o, tid);
        __threadfence_block();
        __syncthreads();
      }
      const bool overflow = sh.n_orph > PM_ORPH;
      __syncthreads();
      if (!overflow) break;
      if (tid == 0) sh.n_orph = 0;
      __syncthreads();
      for (int j = tid; j < L; j += PM_LOOP)
        if (p.cand[so + j] && p.rowarg[so + j] == -2) {
          const int k = atomicAdd(&sh.n_orph, 1);
          if (k < PM_ORPH) {
            sh.orph[k] = j;
            p.rowarg[so + j] = -1;
          }
        }
      __syncthreads();
    }
    --live;
    ++merged;
  }
  if (tid == 0 && p.n_merged) p.n_merged[sc] = merged;
}

}  // namespace

hipError_t launch_prefill_merge(const PrefillMergeArgs &p, int dtype, hipStream_t st) {
  const dim3 g1((p.capacity + 255) / 256, p.n_scopes), g2((p.capacity + 127) / 128, p.n_scopes);
  if (dtype == 0) {
    hipLaunchKernelGGL(k_pm_prep<bf16_t>, g1, dim3(256), 0, st, p);
    hipLaunchKernelGGL(k_pm_rows<bf16_t>, g2, dim3(PM_NT), 0, st, p);
  } else {
    hipLaunchKernelGGL(k_pm_prep<float>, g1, dim3(256), 0, st, p);
    hipLaunchKernelGGL(k_pm_rows<float>, g2, dim3(PM_NT), 0, st, p);
  }
  if (dtype == 0) hipLaunchKernelGGL(k_pm_loop<bf16_t>, dim3(p.n_scopes), dim3(PM_LOOP), 0, st, p);
  else hipLaunchKernelGGL(k_pm_loop<float>, dim3(p.n_scopes), dim3(PM_LOOP), 0, st, p);
  return hipGetLastError();
}

}  // namespace kvc
