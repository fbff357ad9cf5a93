// KeepKV prefill compression by greedy all-pairs ZIP merging (reading notes on
// KeepKV: the inference algorithm's prefill steps 2-5 and the paragraphs on
// candidate choice): while a per-head scope holds more than B live entries,
// the pair of candidate entries (position < protect_from) whose keys have the
// largest cosine is ZIP-merged (eqs. (7), (10), (12) with the guard) under the
// group-mean reference logits, and the merged entry replaces the pair in the
// slot of the older one. Ties: cosine descending, then the pair's lower
// position, then its higher position.
//
// Every candidate row keeps its PK best partners (cosine, then position),
// sorted; every candidate outside a row's list ranks no higher than the list's
// last entry. Kernels, in launch order:
//   k_pm_prep    key norms (float64) and the candidate flags of every slot.
//   k_pm_rows    the initial lists: the block's 64 candidate keys are the
//                float64 MFMA operator of kvc_f64mfma.h (transposed use), 16 keys
//                per tile are the A operand, so a lane holds the dot products of
//                4 rows x 4 tokens and keeps its own top PK per row; the lanes'
//                lists are merged (their union holds every row's top PK).
//   k_pm_loop    one workgroup per scope runs the greedy loop: the pair is the
//                row whose list head is largest (ties to the lower position) and
//                that head. After the merge the merged entry's cosine with every
//                candidate is computed once: it gives the merged row its new list,
//                every other row drops the two merged entries from its list and
//                takes the merged one when it beats the list's last entry, and
//                only a row whose list runs empty is recomputed in full.
// Products of the cache's bf16 (or fp32) keys are exact in float64, so the
// cosines equal the ones of the float64 oracle up to the rounding of the sums.
#include "kvc_f64mfma.h"
#include "kvc_kernels.h"

namespace kvc {
namespace {

constexpr int PK = 4;            // partners kept per row
constexpr int PM_NT = 256;       // k_pm_rows: 4 waves
constexpr int PM_CT = 4;         // k_pm_rows: 16-row column tiles of the operator in use
constexpr int PM_ROWS = 16 * PM_CT;
constexpr int PM_LOOP = 1024;    // k_pm_loop: 16 waves
constexpr int PM_ORPH = 1024;    // rows recomputed per batch

// (cos, pos) order: higher cosine first, then the lower position.
__device__ __forceinline__ bool pm_better(double c1, int p1, double c2, int p2) {
  return c1 > c2 || (c1 == c2 && p1 < p2);
}

// Sorted insertion (best first) of (c, pp, ss) into a list of PK entries; empty entries
// (slot -1) sort last. An entry that would rank past the end is dropped. Branch-free:
// the new entry's rank is the number of entries that stay ahead of it (a prefix).
__device__ __forceinline__ void pk_insert(double (&lc)[PK], int (&lp)[PK], int (&ls)[PK], double c, int pp, int ss) {
  int rank = 0;
#pragma unroll
  for (int k = 0; k < PK; ++k) rank += (ls[k] >= 0 && !pm_better(c, pp, lc[k], lp[k])) ? 1 : 0;
#pragma unroll
  for (int k = PK - 1; k > 0; --k) {
    const bool take_new = k == rank, take_prev = k > rank;
    lc[k] = take_new ? c : (take_prev ? lc[k - 1] : lc[k]);
    lp[k] = take_new ? pp : (take_prev ? lp[k - 1] : lp[k]);
    ls[k] = take_new ? ss : (take_prev ? ls[k - 1] : ls[k]);
  }
  if (rank == 0) {
    lc[0] = c;
    lp[0] = pp;
    ls[0] = ss;
  }
}

// A row's partner list: 64 bytes, read and written as four 16-byte vectors. Empty
// entries have slot -1; slot[0] == -2 marks a row whose recomputation is pending.
struct PmRec {
  double c[PK];
  int s[PK];
  int p[PK];
};
static_assert(sizeof(PmRec) == 64, "partner record is 64 bytes");

__device__ __forceinline__ void rec_load(const PrefillMergeArgs &a, int64_t row, double (&c)[PK], int (&pp)[PK],
                                         int (&ss)[PK]) {
  const PmRec *r = reinterpret_cast<const PmRec *>(a.rec) + row;
  const u32x4 w0 = ld16(&r->c[0]), w1 = ld16(&r->c[2]), w2 = ld16(&r->s[0]), w3 = ld16(&r->p[0]);
  c[0] = __hiloint2double(int(w0.y), int(w0.x));
  c[1] = __hiloint2double(int(w0.w), int(w0.z));
  c[2] = __hiloint2double(int(w1.y), int(w1.x));
  c[3] = __hiloint2double(int(w1.w), int(w1.z));
  ss[0] = int(w2.x); ss[1] = int(w2.y); ss[2] = int(w2.z); ss[3] = int(w2.w);
  pp[0] = int(w3.x); pp[1] = int(w3.y); pp[2] = int(w3.z); pp[3] = int(w3.w);
}

__device__ __forceinline__ void rec_store(const PrefillMergeArgs &a, int64_t row, const double (&c)[PK],
                                          const int (&pp)[PK], const int (&ss)[PK]) {
  PmRec *r = reinterpret_cast<PmRec *>(a.rec) + row;
  st16(&r->c[0], u32x4{uint32_t(__double2loint(c[0])), uint32_t(__double2hiint(c[0])),
                       uint32_t(__double2loint(c[1])), uint32_t(__double2hiint(c[1]))});
  st16(&r->c[2], u32x4{uint32_t(__double2loint(c[2])), uint32_t(__double2hiint(c[2])),
                       uint32_t(__double2loint(c[3])), uint32_t(__double2hiint(c[3]))});
  st16(&r->s[0], u32x4{uint32_t(ss[0]), uint32_t(ss[1]), uint32_t(ss[2]), uint32_t(ss[3])});
  st16(&r->p[0], u32x4{uint32_t(pp[0]), uint32_t(pp[1]), uint32_t(pp[2]), uint32_t(pp[3])});
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
  const double nc[PK] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
  const int np[PK] = {0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7fffffff}, ns[PK] = {-1, -1, -1, -1};
  rec_store(p, slot, nc, np, ns);
  if (i < L) p.evict[slot] = 0;
}

struct RowsMerge {
  double c[PM_NT / 64][PM_ROWS][PK];
  int p[PM_NT / 64][PM_ROWS][PK], s[PM_NT / 64][PM_ROWS][PK];
};
union RowsLds {
  FmOperator op;
  RowsMerge m;
};

// grid (row blocks of 64, scopes), 256 threads; every token of the scope.
template <typename T>
__global__ __launch_bounds__(PM_NT, 1) void k_pm_rows(PrefillMergeArgs p) {
  __shared__ RowsLds sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rb = blockIdx.x * PM_ROWS, sc = blockIdx.y;
  const int L = min(p.len[sc], p.capacity);
  if (rb >= L) return;
  const int64_t so = int64_t(sc) * p.capacity;
  const T *Kb = reinterpret_cast<const T *>(p.k) + int64_t(sc) * p.scope_stride * HD;
  for (int e = tid; e < PM_ROWS * HD; e += PM_NT) {
    const int r = e >> 7, b = e & 127, row = rb + r;
    const double v = (row < L && p.cand[so + row]) ? double(load_elem<T>(Kb, int64_t(row) * HD + b)) : 0.0;
    fm_put_t(sh.op, r, b, v);
  }
  const int jl = lane & 15, tq = lane >> 4;
  double nrow[PM_CT];
  bool rc[PM_CT];
  double lc[PM_CT][PK];
  int lp[PM_CT][PK], ls[PM_CT][PK];
#pragma unroll
  for (int ct = 0; ct < PM_CT; ++ct) {
    const int row = rb + 16 * ct + jl;
    rc[ct] = row < L && p.cand[so + row];
    nrow[ct] = rc[ct] ? p.norm[so + row] : 0.0;
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      lc[ct][k] = -INFINITY;
      lp[ct][k] = 0x7fffffff;
      ls[ct][k] = -1;
    }
  }
  __syncthreads();
  constexpr int ES = sizeof(T);
  const char *Kc = reinterpret_cast<const char *>(Kb);
  const int n16 = (L + FM_TILE - 1) / FM_TILE;
  for (int t = wave; t < n16; t += PM_NT / 64) {
    const int tb = t * FM_TILE;
    FmRow<T> kr;
    kr.load(Kc + (int64_t(min(tb + jl, L - 1)) * HD + 32 * tq) * ES);
    double x[32];
#pragma unroll
    for (int s = 0; s < 32; ++s) x[s] = kr.get(s);
    fm_d4 acc[PM_CT];
#pragma unroll
    for (int ct = 0; ct < PM_CT; ++ct) acc[ct] = fm_d4{0.0, 0.0, 0.0, 0.0};
    fm_apply_t<PM_CT>(sh.op, lane, x, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = tb + tq + 4 * r;
      const int jc = min(j, L - 1);
      const bool cj = j < L && p.cand[so + jc];
      const double nj = p.norm[so + jc];
      const int pj = p.pos[so + jc];
#pragma unroll
      for (int ct = 0; ct < PM_CT; ++ct) {
        const int row = rb + 16 * ct + jl;
        if (rc[ct] && cj && j != row) {
          const double den = nrow[ct] * nj;
          const double c = den > 0.0 ? acc[ct][r] / den : 0.0;
          pk_insert(lc[ct], lp[ct], ls[ct], c, pj, j);
        }
      }
    }
  }
  // merge the lists of the four token groups of the wave (rows 16 ct + jl)
#pragma unroll
  for (int ct = 0; ct < PM_CT; ++ct) {
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      double oc[PK];
      int op_[PK], os[PK];
#pragma unroll
      for (int k = 0; k < PK; ++k) {
        oc[k] = __shfl_xor(lc[ct][k], o);
        op_[k] = __shfl_xor(lp[ct][k], o);
        os[k] = __shfl_xor(ls[ct][k], o);
      }
#pragma unroll
      for (int k = 0; k < PK; ++k)
        if (os[k] >= 0) pk_insert(lc[ct], lp[ct], ls[ct], oc[k], op_[k], os[k]);
    }
  }
  __syncthreads();   // the operator is no longer read: its LDS holds the waves' lists
  if (tq == 0) {
#pragma unroll
    for (int ct = 0; ct < PM_CT; ++ct)
#pragma unroll
      for (int k = 0; k < PK; ++k) {
        sh.m.c[wave][16 * ct + jl][k] = lc[ct][k];
        sh.m.p[wave][16 * ct + jl][k] = lp[ct][k];
        sh.m.s[wave][16 * ct + jl][k] = ls[ct][k];
      }
  }
  __syncthreads();
  if (tid < PM_ROWS && rb + tid < L && p.cand[so + rb + tid]) {
    double c[PK];
    int pp[PK], ss[PK];
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      c[k] = sh.m.c[0][tid][k];
      pp[k] = sh.m.p[0][tid][k];
      ss[k] = sh.m.s[0][tid][k];
    }
    for (int wv = 1; wv < PM_NT / 64; ++wv)
#pragma unroll
      for (int k = 0; k < PK; ++k)
        if (sh.m.s[wv][tid][k] >= 0) pk_insert(c, pp, ss, sh.m.c[wv][tid][k], sh.m.p[wv][tid][k], sh.m.s[wv][tid][k]);
    rec_store(p, so + rb + tid, c, pp, ss);
  }
}

struct LoopLds {
  double kn[HD];            // the key whose row is being computed (float64)
  double red_c[PM_LOOP / 64];
  int red_p[PM_LOOP / 64], red_s[PM_LOOP / 64], red_t[PM_LOOP / 64];
  double lbar[2];
  double wgt[4];
  int orph[PM_ORPH];
  int n_orph;
  double nk;
  double top_c[PK];
  int top_s[PK], top_p[PK];
};

// Workgroup-wide best (c, p) by pm_better over the threads' offers; winner's slot in
// red_s[0] and thread in red_t[0].
__device__ __forceinline__ void loop_argmax(LoopLds &sh, double c, int pp, int ss, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  int tt = tid;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double c2 = __shfl_xor(c, o);
    const int p2 = __shfl_xor(pp, o), s2 = __shfl_xor(ss, o), t2 = __shfl_xor(tt, o);
    if (s2 >= 0 && (ss < 0 || pm_better(c2, p2, c, pp))) {
      c = c2;
      pp = p2;
      ss = s2;
      tt = t2;
    }
  }
  if (lane == 0) {
    sh.red_c[wave] = c;
    sh.red_p[wave] = pp;
    sh.red_s[wave] = ss;
    sh.red_t[wave] = tt;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < PM_LOOP / 64; ++w)
      if (sh.red_s[w] >= 0 && (sh.red_s[0] < 0 || pm_better(sh.red_c[w], sh.red_p[w], sh.red_c[0], sh.red_p[0]))) {
        sh.red_c[0] = sh.red_c[w];
        sh.red_p[0] = sh.red_p[w];
        sh.red_s[0] = sh.red_s[w];
        sh.red_t[0] = sh.red_t[w];
      }
  }
  __syncthreads();
}

// The PK best of the threads' sorted local lists, by PK rounds of a workgroup argmax over the
// lists' heads; written to row `row`'s list.
__device__ __forceinline__ void loop_topk(const PrefillMergeArgs &p, LoopLds &sh, int64_t so, int row,
                                          const double (&lc)[PK], const int (&lp)[PK], const int (&ls)[PK],
                                          int tid) {
  int h = 0;
  for (int k = 0; k < PK; ++k) {
    double c = -INFINITY;
    int pp = 0x7fffffff, ss = -1;
#pragma unroll
    for (int q = 0; q < PK; ++q)
      if (q == h) {
        c = lc[q];
        pp = lp[q];
        ss = ls[q];
      }
    loop_argmax(sh, c, pp, ss, tid);
    if (tid == 0) {
      sh.top_c[k] = sh.red_c[0];
      sh.top_s[k] = sh.red_s[0];
      sh.top_p[k] = sh.red_p[0];
    }
    if (sh.red_s[0] >= 0 && sh.red_t[0] == tid) ++h;
    __syncthreads();
  }
  if (tid == 0) {
    double c[PK];
    int pp[PK], ss[PK];
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      c[k] = sh.top_c[k];
      ss[k] = sh.top_s[k];
      pp[k] = sh.top_s[k] >= 0 ? sh.top_p[k] : 0x7fffffff;
    }
    rec_store(p, so + row, c, pp, ss);
  }
}

// cos(kn, k_j) for a candidate j (kn in LDS, norm sh.nk).
template <typename T>
__device__ __forceinline__ double loop_cos(const PrefillMergeArgs &p, const LoopLds &sh, const T *Kb, int64_t so,
                                           int j) {
  constexpr int EPV = ElemTraits<T>::EPV;
  const char *row = reinterpret_cast<const char *>(Kb + int64_t(j) * HD);
  double dot = 0.0;
#pragma unroll 4
  for (int v = 0; v < HD / EPV; ++v) {
    const u32x4 w = ld16(row + 16 * v);
#pragma unroll
    for (int e = 0; e < EPV; ++e) dot = fma(sh.kn[v * EPV + e], double(ElemTraits<T>::get(w, e)), dot);
  }
  const double den = sh.nk * p.norm[so + j];
  return den > 0.0 ? dot / den : 0.0;
}

// Full list of row `row` (its key in sh.kn, norm sh.nk) over the candidates.
template <typename T>
__device__ __forceinline__ void loop_row(const PrefillMergeArgs &p, LoopLds &sh, const T *Kb, int64_t so, int L,
                                         int row, int tid) {
  double lc[PK];
  int lp[PK], ls[PK];
#pragma unroll
  for (int k = 0; k < PK; ++k) {
    lc[k] = -INFINITY;
    lp[k] = 0x7fffffff;
    ls[k] = -1;
  }
  for (int j = tid; j < L; j += PM_LOOP) {
    if (j == row || !p.cand[so + j]) continue;
    pk_insert(lc, lp, ls, loop_cos<T>(p, sh, Kb, so, j), p.pos[so + j], j);
  }
  loop_topk(p, sh, so, row, lc, lp, ls, tid);
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
    // ---- the pair: the row whose list head is largest (ties to the lower position) and that head
    {
      double c = -INFINITY;
      int pp = 0x7fffffff, ss = -1;
      for (int i = tid; i < L; i += PM_LOOP) {
        if (!p.cand[so + i]) continue;
        const PmRec *r = reinterpret_cast<const PmRec *>(p.rec) + so + i;
        if (r->s[0] < 0) continue;
        const double ci = r->c[0];
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
    const int sj = (reinterpret_cast<const PmRec *>(p.rec) + so + si)->s[0];
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
    // ---- the merged entry against every candidate: its own list, and every other row drops the
    // two merged entries and takes the merged one when it beats its last entry; rows left
    // with an empty list are recomputed in full
    {
      const int ps = p.pos[so + surv];
      double lc[PK];
      int lp[PK], ls[PK];
#pragma unroll
      for (int k = 0; k < PK; ++k) {
        lc[k] = -INFINITY;
        lp[k] = 0x7fffffff;
        ls[k] = -1;
      }
      for (int j = tid; j < L; j += PM_LOOP) {
        if (j == surv || !p.cand[so + j]) continue;
        const double cs = loop_cos<T>(p, sh, Kb, so, j);
        const int pj = p.pos[so + j];
        pk_insert(lc, lp, ls, cs, pj, j);
        // row j's list without the two merged entries (the kept entries stay in order)
        double oc[PK];
        int opp[PK], os[PK];
        rec_load(p, so + j, oc, opp, os);
        double jc[PK];
        int jp[PK], js[PK];
#pragma unroll
        for (int k = 0; k < PK; ++k) {
          jc[k] = -INFINITY;
          jp[k] = 0x7fffffff;
          js[k] = -1;
        }
        int n = 0;
        bool dropped = false;
        double last_c = -INFINITY;
        int last_p = 0x7fffffff;
#pragma unroll
        for (int k = 0; k < PK; ++k) {
          if (os[k] < 0) continue;
          if (os[k] == surv || os[k] == gone) {
            dropped = true;
            continue;
          }
          pk_insert(jc, jp, js, oc[k], opp[k], os[k]);
          last_c = oc[k];
          last_p = opp[k];
          ++n;
        }
        if (n == 0) {
          const int k = atomicAdd(&sh.n_orph, 1);
          if (k < PM_ORPH) sh.orph[k] = j;
          js[0] = -2;                      // recomputed below (in a later batch past PM_ORPH)
          rec_store(p, so + j, jc, jp, js);
          continue;
        }
        // the merged entry joins the list when it ranks above the list's last entry
        const bool joins = pm_better(cs, ps, last_c, last_p);
        if (joins) pk_insert(jc, jp, js, cs, ps, surv);
        if (joins || dropped) rec_store(p, so + j, jc, jp, js);
      }
      loop_topk(p, sh, so, surv, lc, lp, ls, tid);
    }
    __threadfence_block();
    __syncthreads();
    // ---- rows whose lists ran empty, in batches of PM_ORPH
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
      for (int j = tid; j < L; j += PM_LOOP) {
        PmRec *r = reinterpret_cast<PmRec *>(p.rec) + so + j;
        if (p.cand[so + j] && r->s[0] == -2) {
          const int k = atomicAdd(&sh.n_orph, 1);
          if (k < PM_ORPH) {
            sh.orph[k] = j;
            r->s[0] = -1;
          }
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
  const dim3 g1((p.capacity + 255) / 256, p.n_scopes), g2((p.capacity + PM_ROWS - 1) / PM_ROWS, p.n_scopes);
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
