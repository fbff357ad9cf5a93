// KeepKV prefill compression by greedy all-pairs ZIP merging (reading notes on
// KeepKV: the inference algorithm's prefill steps 2-5 and the paragraphs on
// candidate choice): while a per-head scope holds more than B live entries,
// the pair of candidate entries (position < protect_from) whose keys have the
// largest cosine is ZIP-merged (eqs. (7), (10), (12) with the guard) under the
// group-mean reference logits, and the merged entry replaces the pair in the
// slot of the older one. Ties: cosine descending, then the pair's lower
// position, then its higher position.
//
// Every candidate row keeps a list of its PK best partners (cosine, then
// position), sorted, such that every candidate outside the list ranks no
// higher than the list's last entry; a row's best pair is its list head. A row
// whose list runs empty becomes stale and keeps a bound instead: the cosine of
// its old last entry, which no partner outside the old list exceeds. Every pair
// with a listed row in it is covered by that row's list, so the only pairs no
// list covers join two stale rows, and their cosine is at most the second
// largest stale bound: while that bound stays below the best list head, the
// greedy choice from the heads is exact; otherwise the stale rows that could
// reach the head are recomputed first, in batches.
//
// Kernels, in launch order:
//   k_pm_prep   key norms (float64), positions and candidate flags of every
//               slot; empty lists.
//   k_pm_rows   the initial lists: the block's 64 candidate keys are the float64
//               MFMA operator of kvc_f64mfma.h (transposed use), 16 keys per tile
//               are the A operand, so a lane holds the dot products of 4 rows x 4
//               tokens and keeps its own top PK per row; the lanes' lists are
//               merged (their union holds every row's top PK).
//   k_pm_loop   one workgroup per scope runs the greedy loop over the scope's
//               candidates, listed in LDS. Per merge: the merge itself (one wave,
//               float64 weights); then one pass of the merged key against every
//               candidate, 16 lanes per key row (16 bytes each, 8 row steps of
//               loads in flight; the 8 steps' partial dot products reduced over
//               the 16 lanes by the lane-permuted transposed reduction), after
//               which one lane per step owns that row with its list in
//               registers: the merged row's
//               list is collected, every other row drops the merged pair or takes
//               the merged entry when it beats an entry of its list (or goes
//               stale), and the heads and stale bounds for the next pair choice
//               are reduced on the way. When two stale bounds could reach the
//               best head, the stale rows that could are recomputed on the
//               float64 MFMA, 16 per pass (their keys as a 16-row operator tile),
//               and only their new heads join the pair choice.
// Products of the cache's bf16 (or fp32) keys are exact in float64, so the
// cosines equal the ones of the float64 oracle up to the rounding of the sums.
#include "kvc_f64mfma.h"
#include "kvc_kernels.h"

namespace kvc {
namespace {

constexpr int PK = 4;            // partners kept per row
constexpr int PM_NT = 512;       // k_pm_rows: 8 waves, two per SIMD
constexpr int PM_CT = 4;         // k_pm_rows: 16-row column tiles of the operator in use
constexpr int PM_ROWS = 16 * PM_CT;
constexpr int PL_NT = 512;       // k_pm_loop: 8 waves
constexpr int PL_W = PL_NT / 64;
constexpr int PL_NS = 8;         // row steps per batch of the merge pass (a power of 2, <= 16)
constexpr int PL_NQ = 16;        // stale rows recomputed per pass: one 16-row MFMA operator tile
constexpr int PL_TODO = 256;     // stale rows collected per recomputation round
constexpr int PL_SCAN = 8;       // rows per thread per load batch of the head scan
constexpr int PL_CAND = 1024;    // rows whose list may change, queued per merge pass (more: handled in place)
constexpr int STALE = -2;        // slot value of a stale row's entries (entry 0 holds the bound)
constexpr int NOPOS = 0x7fffffff;

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

// pk_insert only when the entry ranks above the list's last entry (or the list has room): in a
// stream of candidates most are rejected by this one comparison.
__device__ __forceinline__ void pk_offer(double (&lc)[PK], int (&lp)[PK], int (&ls)[PK], double c, int pp, int ss) {
  if (ls[PK - 1] < 0 || pm_better(c, pp, lc[PK - 1], lp[PK - 1])) pk_insert(lc, lp, ls, c, pp, ss);
}

__device__ __forceinline__ void list_clear(double (&lc)[PK], int (&lp)[PK], int (&ls)[PK]) {
#pragma unroll
  for (int k = 0; k < PK; ++k) {
    lc[k] = -INFINITY;
    lp[k] = NOPOS;
    ls[k] = -1;
  }
}

// Each lane takes the union's best PK of its list and the list of lane ^ o (disjoint rows).
__device__ __forceinline__ void list_merge_xor(double (&lc)[PK], int (&lp)[PK], int (&ls)[PK], int o) {
  double oc[PK];
  int op[PK], os[PK];
#pragma unroll
  for (int k = 0; k < PK; ++k) {
    oc[k] = __shfl_xor(lc[k], o);
    op[k] = __shfl_xor(lp[k], o);
    os[k] = __shfl_xor(ls[k], o);
  }
#pragma unroll
  for (int k = 0; k < PK; ++k)
    if (os[k] >= 0) pk_insert(lc, lp, ls, oc[k], op[k], os[k]);
}

// 16-byte entries {float64 value, int, int}: a list entry (cosine, slot, position) and a
// row's metadata (key norm, position, candidate flag).
__device__ __forceinline__ u32x4 ent_pack(double c, int a, int b) {
  return u32x4{uint32_t(__double2loint(c)), uint32_t(__double2hiint(c)), uint32_t(a), uint32_t(b)};
}
__device__ __forceinline__ double ent_c(const u32x4 &w) { return __hiloint2double(int(w.y), int(w.x)); }

__device__ __forceinline__ char *rec_at(const PrefillMergeArgs &a, int64_t row) {
  return static_cast<char *>(a.rec) + row * 64;
}
__device__ __forceinline__ char *meta_at(const PrefillMergeArgs &a, int64_t row) {
  return static_cast<char *>(a.meta) + row * 16;
}
__device__ __forceinline__ bool pm_cand(const PrefillMergeArgs &a, int64_t row) {
  return reinterpret_cast<const int *>(meta_at(a, row))[3] != 0;
}
__device__ __forceinline__ double pm_norm(const PrefillMergeArgs &a, int64_t row) {
  return *reinterpret_cast<const double *>(meta_at(a, row));
}

__device__ __forceinline__ void rec_store(const PrefillMergeArgs &a, int64_t row, const double (&c)[PK],
                                          const int (&pp)[PK], const int (&ss)[PK]) {
#pragma unroll
  for (int k = 0; k < PK; ++k) st16(rec_at(a, row) + 16 * k, ent_pack(c[k], ss[k], pp[k]));
}

__device__ __forceinline__ void rec_store_stale(const PrefillMergeArgs &a, int64_t row, double bound) {
#pragma unroll
  for (int k = 0; k < PK; ++k) st16(rec_at(a, row) + 16 * k, ent_pack(bound, STALE, NOPOS));
}

// 32-byte row summaries, what the merge loop reads of a row in every pass (the list itself
// only when it may change): [0, 8) the key norm (float64), [8, 12) the position, [12, 16) the
// cosine of the list's last entry rounded down to a float (-inf: no entry), [16, 24) the
// head's cosine or a stale row's bound, [24, 32) the entries' partner slots (16 bits each;
// SUM_NONE: no entry, SUM_STALE: a stale row). Slots fit 16 bits: at most
// PREFILL_MAX_ROWS = 32768 of them.
constexpr uint32_t SUM_NONE = 0xffffu, SUM_STALE = 0xfffeu;
static_assert(PREFILL_MAX_ROWS <= 0xfffe, "slots of a scope fit 16 bits below the markers");

__device__ __forceinline__ char *sum_at(const PrefillMergeArgs &a, int64_t row) {
  return static_cast<char *>(a.sum) + row * 32;
}

// The largest float not above c.
__device__ __forceinline__ float float_below(double c) {
  const float f = float(c);
  return double(f) > c ? nextafterf(f, -INFINITY) : f;
}

// The list-dependent half of a summary (and the last entry's bound) after a list is stored.
__device__ __forceinline__ void sum_store_list(const PrefillMergeArgs &a, int64_t row, const double (&c)[PK],
                                               const int (&ss)[PK]) {
  double last = -INFINITY;
  uint32_t part[PK];
#pragma unroll
  for (int k = 0; k < PK; ++k) {
    if (ss[k] >= 0) last = c[k];
    part[k] = ss[k] >= 0 ? uint32_t(ss[k]) : SUM_NONE;
  }
  const double hd = ss[0] >= 0 ? c[0] : -INFINITY;
  reinterpret_cast<float *>(sum_at(a, row))[3] = float_below(last);
  st16(sum_at(a, row) + 16, u32x4{uint32_t(__double2loint(hd)), uint32_t(__double2hiint(hd)),
                                  part[0] | (part[1] << 16), part[2] | (part[3] << 16)});
}

__device__ __forceinline__ void sum_store_stale(const PrefillMergeArgs &a, int64_t row, double bound) {
  reinterpret_cast<float *>(sum_at(a, row))[3] = -INFINITY;
  st16(sum_at(a, row) + 16, u32x4{uint32_t(__double2loint(bound)), uint32_t(__double2hiint(bound)),
                                  SUM_STALE | (SUM_STALE << 16), SUM_STALE | (SUM_STALE << 16)});
}

// Does a summary's partner field (two words) hold slot s?
__device__ __forceinline__ bool sum_has(uint32_t pa, uint32_t pb, int s) {
  const uint32_t u = uint32_t(s);
  return (pa & 0xffffu) == u || (pa >> 16) == u || (pb & 0xffffu) == u || (pb >> 16) == u;
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
  const int pos = p.pos[slot];
  st16(meta_at(p, slot), ent_pack(sqrt(n), pos, (i < L && pos < p.protect_from) ? 1 : 0));
  double c[PK];
  int pp[PK], ss[PK];
  list_clear(c, pp, ss);
  rec_store(p, slot, c, pp, ss);
  // the summary: norm, position, an empty list
  const u32x4 m0 = ent_pack(sqrt(n), pos, 0);
  st16(sum_at(p, slot), u32x4{m0.x, m0.y, m0.z, uint32_t(__float_as_int(-INFINITY))});
  sum_store_list(p, slot, c, ss);
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
    const double v = (row < L && pm_cand(p, so + row)) ? double(load_elem<T>(Kb, int64_t(row) * HD + b)) : 0.0;
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
    rc[ct] = row < L && pm_cand(p, so + row);
    nrow[ct] = rc[ct] ? pm_norm(p, so + row) : 0.0;
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
      const bool cj = j < L && pm_cand(p, so + jc);
      const double nj = pm_norm(p, so + jc);
      const int pj = p.pos[so + jc];
#pragma unroll
      for (int ct = 0; ct < PM_CT; ++ct) {
        const int row = rb + 16 * ct + jl;
        if (rc[ct] && cj && j != row) {
          const double den = nrow[ct] * nj;
          const double c = den > 0.0 ? acc[ct][r] / den : 0.0;
          pk_offer(lc[ct], lp[ct], ls[ct], c, pj, j);
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
  if (tid < PM_ROWS && rb + tid < L && pm_cand(p, so + rb + tid)) {
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
    sum_store_list(p, so + rb + tid, c, ss);
  }
}

// The 8 elements [8 e, 8 e + 8) of a key row (16 lanes per row).
template <typename T>
struct Chunk8;
template <>
struct Chunk8<bf16_t> {
  u32x4 w;
  __device__ __forceinline__ void load(const char *row, int e) { w = ld16(row + 16 * e); }
  __device__ __forceinline__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ double get(int u) const { return double(ElemTraits<bf16_t>::get(w, u)); }
};
template <>
struct Chunk8<float> {
  u32x4 w0, w1;
  __device__ __forceinline__ void load(const char *row, int e) {
    w0 = ld16(row + 32 * e);
    w1 = ld16(row + 32 * e + 16);
  }
  __device__ __forceinline__ void zero() { w0 = w1 = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ double get(int u) const { return double(ElemTraits<float>::get(u < 4 ? w0 : w1, u & 3)); }
};

// The keys of up to 16 rows as the B operand of v_mfma_f64_16x16x4 (the transposed use of
// kvc_f64mfma.h restricted to its first column tile): 16 KB.
struct FmOp16 {
  fm_d2 a[FM_S2][64];
};
__device__ __forceinline__ void op16_put(FmOp16 &op, int j, int b, double v) {   // row j < 16, element b
  const int g = b >> 5, s = b & 31;
  op.a[s >> 1][fm_swz(s >> 1, j + 16 * g)][s & 1] = v;
}
// acc[r] += X[l % 16] . y_{l / 16 + 4 r}: lane l holds elements [32 g, 32 g + 32) of token
// l % 16's row (kr, g = l / 16) as A values and ends with row l % 16 of X against tokens
// l / 16 + 4 r. The A values are converted to float64 step by step.
template <typename T>
__device__ __forceinline__ void op16_apply(const FmOp16 &op, int lane, const FmRow<T> &kr, fm_d4 &acc) {
#pragma unroll
  for (int s2 = 0; s2 < FM_S2; ++s2) {
    const fm_d2 bf = op.a[s2][fm_swz(s2, lane)];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(kr.get(2 * s2), bf.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(kr.get(2 * s2 + 1), bf.y, acc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct LoopLds {
  uint16_t live[PREFILL_MAX_ROWS];  // the scope's candidate slots (any order)
  FmOp16 rop;                     // keys of the rows being recomputed
  double qk[1][HD];               // float64 merged key of the merge pass
  double qn[PL_NQ];
  int qrow[PL_NQ], qpos[PL_NQ];
  double hc[PL_W], hu1[PL_W], hu2[PL_W];              // per-wave head and stale-bound reductions
  int hp[PL_W], hs[PL_W], hsj[PL_W], hpj[PL_W];
  double lc[PL_NQ][PL_W][PK];                         // per-wave best partners of the query rows
  int lp[PL_NQ][PL_W][PK], ls[PL_NQ][PL_W][PK];
  int todo[PL_TODO];
  double th_c[PL_TODO];           // the recomputed rows' new heads (cosine, partner slot and position)
  int th_s[PL_TODO], th_p[PL_TODO], th_pos[PL_TODO];
  double cand_c[PL_CAND];         // rows of a merge pass whose list may change: the merged key's cosine,
  int cand_row[PL_CAND], cand_pos[PL_CAND];   // the row's slot and position
  double xb[PL_NT];               // each thread's largest stale bound below the head, and its row
  int xr[PL_NT];                  // (-1 once it is taken into the recomputation)
  int n_todo, n_live, gidx, n_cand;
};

// The best list head (largest cosine, ties to the lower row position) and the two largest
// stale bounds seen so far.
struct Heads {
  double c, u1, u2;
  int p, s, sj, pj;   // row position, row slot, partner slot, partner position
  __device__ __forceinline__ void clear() {
    c = u1 = u2 = -INFINITY;
    p = pj = NOPOS;
    s = sj = -1;
  }
  __device__ __forceinline__ void offer(double c0, int pi, int row, int s0, int p0) {
    if (s >= 0 && !pm_better(c0, pi, c, p)) return;
    c = c0;
    p = pi;
    s = row;
    sj = s0;
    pj = p0;
  }
  __device__ __forceinline__ void bound(double b) {
    const double n1 = fmax(u1, b), n2 = fmax(u2, fmin(u1, b));
    u1 = n1;
    u2 = n2;
  }
  // a row's list as loaded or rewritten: entry 0 is its head, or its stale bound
  __device__ __forceinline__ void row(double c0, int s0, int p0, int pi, int r) {
    if (s0 >= 0) offer(c0, pi, r, s0, p0);
    else if (s0 == STALE) bound(c0);
  }
  // the same from a row's summary (halves s0, s1); the head partner's position is not
  // in it (the chosen head's is looked up afterwards)
  __device__ __forceinline__ void sum_row(const u32x4 &s0, const u32x4 &s1, int r) {
    const uint32_t h0 = s1.z & 0xffffu;
    if (h0 == SUM_STALE) bound(ent_c(s1));
    else if (h0 != SUM_NONE) offer(ent_c(s1), int(s0.z), r, int(h0), NOPOS);
  }
  __device__ __forceinline__ void take(const Heads &o) {
    if (o.s >= 0) offer(o.c, o.p, o.s, o.sj, o.pj);
    const double n1 = fmax(u1, o.u1), n2 = fmax(fmin(u1, o.u1), fmax(u2, o.u2));
    u1 = n1;
    u2 = n2;
  }
  __device__ __forceinline__ Heads xor_lane(int o) const {
    Heads h;
    h.c = __shfl_xor(c, o);
    h.u1 = __shfl_xor(u1, o);
    h.u2 = __shfl_xor(u2, o);
    h.p = __shfl_xor(p, o);
    h.s = __shfl_xor(s, o);
    h.sj = __shfl_xor(sj, o);
    h.pj = __shfl_xor(pj, o);
    return h;
  }
};

// Wave reduction of the lanes' Heads, written to the LDS slot of the wave.
__device__ __forceinline__ void heads_to_lds(LoopLds &sh, Heads h, int lane, int wave) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) h.take(h.xor_lane(o));
  if (lane == 0) {
    sh.hc[wave] = h.c;
    sh.hu1[wave] = h.u1;
    sh.hu2[wave] = h.u2;
    sh.hp[wave] = h.p;
    sh.hs[wave] = h.s;
    sh.hsj[wave] = h.sj;
    sh.hpj[wave] = h.pj;
  }
}

// The waves' Heads from LDS, combined in wave order (every thread gets the same result).
__device__ __forceinline__ void heads_from_lds(const LoopLds &sh, Heads &h) {
#pragma unroll
  for (int w = 0; w < PL_W; ++w) {
    Heads o;
    o.c = sh.hc[w];
    o.u1 = sh.hu1[w];
    o.u2 = sh.hu2[w];
    o.p = sh.hp[w];
    o.s = sh.hs[w];
    o.sj = sh.hsj[w];
    o.pj = sh.hpj[w];
    h.take(o);
  }
}

// The PK best entries of the union of the lanes' sorted lists (distinct rows), by PK
// rounds of a wave argmax over the lists' heads; the winning lane drops its head. Every
// lane receives the result.
__device__ __forceinline__ void wave_topk(double (&lc)[PK], int (&lp)[PK], int (&ls)[PK], int lane,
                                          double (&oc)[PK], int (&op)[PK], int (&os)[PK]) {
#pragma unroll
  for (int k = 0; k < PK; ++k) {
    double c = lc[0];
    int pp = lp[0], ss = ls[0], who = lane;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double c2 = __shfl_xor(c, o);
      const int p2 = __shfl_xor(pp, o), s2 = __shfl_xor(ss, o), w2 = __shfl_xor(who, o);
      if (s2 >= 0 && (ss < 0 || pm_better(c2, p2, c, pp))) {
        c = c2;
        pp = p2;
        ss = s2;
        who = w2;
      }
    }
    oc[k] = c;
    op[k] = pp;
    os[k] = ss;
    const bool pop = ss >= 0 && who == lane;
#pragma unroll
    for (int x = 0; x < PK - 1; ++x) {
      lc[x] = pop ? lc[x + 1] : lc[x];
      lp[x] = pop ? lp[x + 1] : lp[x];
      ls[x] = pop ? ls[x + 1] : ls[x];
    }
    lc[PK - 1] = pop ? -INFINITY : lc[PK - 1];
    lp[PK - 1] = pop ? NOPOS : lp[PK - 1];
    ls[PK - 1] = pop ? -1 : ls[PK - 1];
  }
}

// The final list of query row q from the waves' lists in LDS (every lane of the calling
// wave receives it).
__device__ __forceinline__ void final_list(const LoopLds &sh, int q, int lane, double (&c)[PK], int (&pp)[PK],
                                           int (&ss)[PK]) {
  double lc[PK];
  int lp[PK], ls[PK];
  list_clear(lc, lp, ls);
  if (lane < PL_W * PK) {   // lane 4 w + k holds entry k of wave w's list
    lc[0] = sh.lc[q][lane / PK][lane % PK];
    lp[0] = sh.lp[q][lane / PK][lane % PK];
    ls[0] = sh.ls[q][lane / PK][lane % PK];
  }
  wave_topk(lc, lp, ls, lane, c, pp, ss);
}

// Full scan of the candidates' records: heads and stale bounds (ends with a barrier; every
// thread receives the result).
__device__ __forceinline__ void scan_heads(const PrefillMergeArgs &p, LoopLds &sh, int64_t so, int n_live, int tid,
                                           Heads &h) {
  const int lane = tid & 63, wave = tid >> 6;
  Heads m;
  m.clear();
  for (int k0 = 0; k0 < n_live; k0 += PL_NT * PL_SCAN) {
    int jr[PL_SCAN];
    u32x4 s0[PL_SCAN], s1[PL_SCAN];
#pragma unroll
    for (int u = 0; u < PL_SCAN; ++u) {
      const int k = k0 + u * PL_NT + tid;
      jr[u] = k < n_live ? sh.live[k] : -1;
      if (jr[u] >= 0) {
        s0[u] = ld16(sum_at(p, so + jr[u]));
        s1[u] = ld16(sum_at(p, so + jr[u]) + 16);
      } else {
        s0[u] = s1[u] = u32x4{0u, 0u, SUM_NONE, SUM_NONE};
      }
    }
#pragma unroll
    for (int u = 0; u < PL_SCAN; ++u)
      if (jr[u] >= 0) m.sum_row(s0[u], s1[u], jr[u]);
  }
  heads_to_lds(sh, m, lane, wave);
  __syncthreads();
  h.clear();
  heads_from_lds(sh, h);
  if (h.s >= 0) h.pj = p.pos[so + h.sj];   // the head partner's position (not in the summaries)
}

// Stale rows recomputed in full against every candidate, on the float64 MFMA: the keys of
// nq (<= 16) rows are the operator sh.rop (rows nq.. zero), 16 candidates per tile are the A
// operand, so lane l holds row l % 16 against candidates l / 16 + 4 r and keeps that row's
// best PK; the lanes' and waves' lists are merged into each row's record. sh.qn / qrow hold
// the rows' norms and slots.
template <typename T>
__device__ __forceinline__ void pass_recompute(const PrefillMergeArgs &p, LoopLds &sh, const char *Kc, int64_t so,
                                               int n_live, int nq, int b, int tid) {
  constexpr int ES = sizeof(T);
  const int lane = tid & 63, wave = tid >> 6, jl = lane & 15, tq = lane >> 4;
  const bool mine = jl < nq;
  const double qnj = mine ? sh.qn[jl] : 0.0;
  const int qrj = mine ? sh.qrow[jl] : -1;
  double lc[PK];
  int lp[PK], ls[PK];
  list_clear(lc, lp, ls);
  const int n16 = (n_live + FM_TILE - 1) / FM_TILE;
  for (int t = wave; t < n16; t += PL_W) {
    const int tb = t * FM_TILE;
    FmRow<T> kr;
    kr.load(Kc + (int64_t(sh.live[min(tb + jl, n_live - 1)]) * HD + 32 * tq) * ES);
    int jr[4];
    u32x4 mr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k = tb + tq + 4 * r;
      jr[r] = k < n_live ? int(sh.live[k]) : -1;
      // the summary's first half: norm and position
      mr[r] = jr[r] >= 0 ? ld16(sum_at(p, so + jr[r])) : u32x4{0u, 0u, 0u, 0u};
    }
    fm_d4 acc = fm_d4{0.0, 0.0, 0.0, 0.0};
    op16_apply<T>(sh.rop, lane, kr, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (!mine || jr[r] < 0 || jr[r] == qrj) continue;
      const double den = qnj * ent_c(mr[r]);
      pk_offer(lc, lp, ls, den > 0.0 ? acc[r] / den : 0.0, int(mr[r].z), jr[r]);
    }
  }
  // lanes of equal row (the four token groups), then the waves
  list_merge_xor(lc, lp, ls, 16);
  list_merge_xor(lc, lp, ls, 32);
  if (tq == 0 && mine) {
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      sh.lc[jl][wave][k] = lc[k];
      sh.lp[jl][wave][k] = lp[k];
      sh.ls[jl][wave][k] = ls[k];
    }
  }
  __syncthreads();
  if (tid < nq) {
    double c[PK];
    int pp[PK], ss[PK];
#pragma unroll
    for (int k = 0; k < PK; ++k) {
      c[k] = sh.lc[tid][0][k];
      pp[k] = sh.lp[tid][0][k];
      ss[k] = sh.ls[tid][0][k];
    }
    for (int w = 1; w < PL_W; ++w)
#pragma unroll
      for (int k = 0; k < PK; ++k)
        if (sh.ls[tid][w][k] >= 0) pk_insert(c, pp, ss, sh.lc[tid][w][k], sh.lp[tid][w][k], sh.ls[tid][w][k]);
    rec_store(p, so + sh.qrow[tid], c, pp, ss);
    sum_store_list(p, so + sh.qrow[tid], c, ss);
    sh.th_c[b + tid] = c[0];
    sh.th_s[b + tid] = ss[0];
    sh.th_p[b + tid] = pp[0];
    sh.th_pos[b + tid] = sh.qpos[tid];
  }
  __syncthreads();
}

template <typename T>
__global__ __launch_bounds__(PL_NT, 1) void k_pm_loop(PrefillMergeArgs p) {
  __shared__ LoopLds sh;
  constexpr int ES = sizeof(T), NS = PL_NS;
  const int sc = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int e = lane & 15, gi = lane >> 4;
  const int L = min(p.len[sc], p.capacity);
  const int64_t so = int64_t(sc) * p.capacity;
  T *Kw = reinterpret_cast<T *>(p.k) + int64_t(sc) * p.scope_stride * HD;
  T *Vw = reinterpret_cast<T *>(p.v) + int64_t(sc) * p.scope_stride * HD;
  const T *Kb = Kw;
  const char *Kc = reinterpret_cast<const char *>(Kb);
  int live = L, merged = 0;
  if (live <= p.budget) {
    if (tid == 0 && p.n_merged) p.n_merged[sc] = 0;
    return;
  }
  // ---- the candidate list, then the heads of the initial lists
  if (tid == 0) sh.n_live = 0;
  __syncthreads();
  for (int i = tid; i < L; i += PL_NT)
    if (pm_cand(p, so + i)) {
      const int k = atomicAdd(&sh.n_live, 1);
      if (k < PREFILL_MAX_ROWS) sh.live[k] = uint16_t(i);
    }
  __syncthreads();
  int n_live = min(sh.n_live, PREFILL_MAX_ROWS);
  Heads h;
  scan_heads(p, sh, so, n_live, tid, h);
  int rounds = 0;   // recomputation rounds since the last merge (each one clears >= 2 stale rows)
  while (live > p.budget) {
    // ---- two stale rows might form a pair at least as good as the best head: recompute the
    // stale rows whose bound reaches it, then scan again
    if (h.u2 > -INFINITY && h.u2 >= h.c) {
      if (++rounds > n_live) {   // cannot happen: stop rather than loop
        if (tid == 0) p.status[0] = -7;
        break;
      }
      if (tid == 0) sh.n_todo = 0;
      __syncthreads();
      // stale rows whose bound reaches the best head are recomputed; the others' bounds are kept
      // (each thread's three largest: its largest row may fill a spare row of the recomputation)
      Heads rest;
      rest.clear();
      double xb1 = -INFINITY, xb2 = -INFINITY, xb3 = -INFINITY;
      int xr1 = -1;
      for (int k0 = 0; k0 < n_live; k0 += PL_NT * PL_SCAN) {
        int jr[PL_SCAN];
        u32x4 er[PL_SCAN];
#pragma unroll
        for (int u = 0; u < PL_SCAN; ++u) {
          const int k = k0 + u * PL_NT + tid;
          jr[u] = k < n_live ? int(sh.live[k]) : -1;
          // the summary's second half: head (a stale row's bound) and partner slots
          er[u] = jr[u] >= 0 ? ld16(sum_at(p, so + jr[u]) + 16) : u32x4{0u, 0u, SUM_NONE, SUM_NONE};
        }
#pragma unroll
        for (int u = 0; u < PL_SCAN; ++u) {
          if (jr[u] < 0 || (er[u].z & 0xffffu) != SUM_STALE) continue;
          const double b = ent_c(er[u]);
          if (b >= h.c) {
            const int t = atomicAdd(&sh.n_todo, 1);
            if (t < PL_TODO) sh.todo[t] = jr[u];
          } else if (b > xb1) {
            xb3 = xb2;
            xb2 = xb1;
            xb1 = b;
            xr1 = jr[u];
          } else if (b > xb2) {
            xb3 = xb2;
            xb2 = b;
          } else {
            xb3 = fmax(xb3, b);
          }
        }
      }
      // A recomputation pass streams every key for up to PL_NQ rows: when fewer rows must be
      // recomputed, the stale rows with the largest bounds below the head (each thread's
      // largest) fill the pass, since they are the next ones the choice may need.
      sh.xb[tid] = xb1;
      sh.xr[tid] = xr1;
      __syncthreads();
      if (wave == 0) {
        const int nt0 = min(sh.n_todo, PL_TODO);
        if (nt0 < PL_NQ) {
          constexpr int PER = PL_NT / 64;
          double v[PER];
#pragma unroll
          for (int i = 0; i < PER; ++i) v[i] = sh.xr[lane + 64 * i] >= 0 ? sh.xb[lane + 64 * i] : -INFINITY;
          int added = 0;
          for (int r = nt0; r < PL_NQ; ++r) {
            double bv = -INFINITY;
            int bi = -1;
#pragma unroll
            for (int i = 0; i < PER; ++i)
              if (v[i] > bv) {
                bv = v[i];
                bi = lane + 64 * i;
              }
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
              const double v2 = __shfl_xor(bv, o);
              const int i2 = __shfl_xor(bi, o);
              if (v2 > bv || (v2 == bv && i2 >= 0 && (bi < 0 || i2 < bi))) {
                bv = v2;
                bi = i2;
              }
            }
            if (bi < 0) break;   // no stale row left
#pragma unroll
            for (int i = 0; i < PER; ++i)
              if (bi == lane + 64 * i) v[i] = -INFINITY;
            if (lane == 0) {
              sh.todo[r] = sh.xr[bi];
              sh.xr[bi] = -1;
            }
            ++added;
          }
          if (lane == 0) sh.n_todo = nt0 + added;
        }
      }
      __syncthreads();
      {
        const bool taken = xr1 >= 0 && sh.xr[tid] < 0;
        rest.bound(taken ? xb2 : xb1);
        rest.bound(taken ? xb3 : xb2);
      }
      heads_to_lds(sh, rest, lane, wave);
      __syncthreads();
      rest.clear();
      heads_from_lds(sh, rest);
      const int nt = min(sh.n_todo, PL_TODO);
      for (int b = 0; b < nt; b += PL_NQ) {
        const int nq = min(PL_NQ, nt - b);
        for (int e = tid; e < PL_NQ * HD; e += PL_NT) {
          const int q = e / HD, x = e % HD;
          const int row = q < nq ? sh.todo[b + q] : -1;
          op16_put(sh.rop, q, x, row >= 0 ? double(load_elem<T>(Kb, int64_t(row) * HD + x)) : 0.0);
          if (x == 0 && row >= 0) {
            const u32x4 m = ld16(sum_at(p, so + row));
            sh.qn[q] = ent_c(m);
            sh.qrow[q] = row;
            sh.qpos[q] = int(m.z);
          }
        }
        __syncthreads();
        pass_recompute<T>(p, sh, Kc, so, n_live, nq, b, tid);
      }
      if (sh.n_todo > PL_TODO) {   // some reaching rows are still stale: rescan everything
        __syncthreads();
        scan_heads(p, sh, so, n_live, tid, h);
      } else {
        // only the recomputed rows changed: the best head so far or one of theirs; the stale
        // bounds left are the rest's
        h.u1 = rest.u1;
        h.u2 = rest.u2;
        for (int q = 0; q < nt; ++q) h.row(sh.th_c[q], sh.th_s[q], sh.th_p[q], sh.th_pos[q], sh.todo[q]);
      }
      continue;
    }
    if (h.s < 0) {   // fewer than two entries may merge: the budget cannot be reached
      if (tid == 0) p.status[0] = -4;
      break;
    }
    if (h.sj >= L) {   // cannot happen: every list entry is a live candidate
      if (tid == 0) p.status[0] = -7;
      break;
    }
    rounds = 0;
    // the older entry of the pair survives; the other is removed
    const bool older = h.p < h.pj;
    const int surv = older ? h.s : h.sj, gone = older ? h.sj : h.s, ps = older ? h.p : h.pj;
    // ---- the merge (wave 0; two elements per lane)
    if (wave == 0) {
      const int e0 = lane, e1 = lane + 64;
      const T *q = reinterpret_cast<const T *>(p.q) + int64_t(sc) * p.G * HD;
      const double kg0 = double(load_elem<T>(Kb, int64_t(gone) * HD + e0));
      const double kg1 = double(load_elem<T>(Kb, int64_t(gone) * HD + e1));
      const double kc0 = double(load_elem<T>(Kb, int64_t(surv) * HD + e0));
      const double kc1 = double(load_elem<T>(Kb, int64_t(surv) * HD + e1));
      const double vg0 = double(load_elem<T>(Vw, int64_t(gone) * HD + e0));
      const double vg1 = double(load_elem<T>(Vw, int64_t(gone) * HD + e1));
      const double vc0 = double(load_elem<T>(Vw, int64_t(surv) * HD + e0));
      const double vc1 = double(load_elem<T>(Vw, int64_t(surv) * HD + e1));
      const int vote_e = p.votes[so + gone], vote_c = p.votes[so + surv];
      const float m_e = p.m ? p.m[so + gone] : 0.0f, m_c = p.m ? p.m[so + surv] : 0.0f;
      double ae = 0.0, ac = 0.0;
      for (int g = 0; g < p.G; ++g) {
        const double q0 = double(load_elem<T>(q, g * HD + e0)), q1 = double(load_elem<T>(q, g * HD + e1));
        ae += q0 * kg0 + q1 * kg1;
        ac += q0 * kc0 + q1 * kc1;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        ae += __shfl_xor(ae, o);
        ac += __shfl_xor(ac, o);
      }
      // reference logits of the two entries (group-mean query) and the ZIP weights
      const double le = ae * p.scale / double(p.G), lc = ac * p.scale / double(p.G);
      const double mu = fmax(le, lc);
      const double pe = double(vote_e), pc = double(vote_c);
      const double we = pe * exp(le - mu), wc = pc * exp(lc - mu);
      const double num = mu + log(we + wc) - log(pe + pc);
      const double den = we * le + wc * lc;
      const bool guarded = fabs(den) < double(p.eps) * exp(-mu);
      const double wv0 = we / (we + wc), wv1 = wc / (we + wc);
      const double wk0 = guarded ? 0.5 : we * num / den, wk1 = guarded ? 0.5 : wc * num / den;
      // the merged rows, rounded to the cache dtype
      const float k0 = round_once<T>(wk0 * kg0 + wk1 * kc0), k1 = round_once<T>(wk0 * kg1 + wk1 * kc1);
      store_elem<T>(Kw, int64_t(surv) * HD + e0, k0);
      store_elem<T>(Kw, int64_t(surv) * HD + e1, k1);
      store_elem<T>(Vw, int64_t(surv) * HD + e0, round_once<T>(wv0 * vg0 + wv1 * vc0));
      store_elem<T>(Vw, int64_t(surv) * HD + e1, round_once<T>(wv0 * vg1 + wv1 * vc1));
      sh.qk[0][e0] = double(k0);
      sh.qk[0][e1] = double(k1);
      double n2 = double(k0) * double(k0) + double(k1) * double(k1);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) n2 += __shfl_xor(n2, o);
      if (lane == 0) {
        const double nk = sqrt(n2);
        st16(meta_at(p, so + surv), ent_pack(nk, ps, 1));
        *reinterpret_cast<double *>(sum_at(p, so + surv)) = nk;
        reinterpret_cast<int *>(meta_at(p, so + gone))[3] = 0;
        p.votes[so + surv] = vote_e + vote_c;
        if (p.m) p.m[so + surv] = m_c + m_e;
        p.evict[so + gone] = 1;
        if (p.pairs) {
          p.pairs[(so + merged) * 2] = surv;
          p.pairs[(so + merged) * 2 + 1] = gone;
        }
        sh.qn[0] = nk;
      }
    }
    if (tid == 0) sh.n_cand = 0;
    __syncthreads();
    // ---- the merged key against every candidate: its own list, the other rows' lists, and
    // the heads for the next merge
    {
      const double nk = sh.qn[0];
      double qv[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) qv[v] = sh.qk[0][8 * e + v];
      double lc[PK];
      int lp[PK], ls[PK];
      list_clear(lc, lp, ls);
      Heads hn;
      hn.clear();
      // lane-permuted transposed reduction of the NS steps' partial dot products over the 16
      // lanes of a row group: slot i of lane e holds step i ^ own, and the lane ends with the
      // total of step own (two lanes per step; the first of them takes the row)
      const int own = perm_head<16, NS>(e);
      const bool lead = perm_rep_lane<16, NS>(own) == e;
      // Row jo's list after the merge (cs: the merged key's cosine with it): it drops an entry
      // of the merged pair, takes the merged entry when that beats one of its entries, or goes
      // stale; the list and its summary are rewritten only when they change.
      auto list_update = [&](int jo, int pj, double cs, Heads &hq) {
        const u32x4 r0 = ld16(rec_at(p, so + jo)), r1 = ld16(rec_at(p, so + jo) + 16);
        const u32x4 r2 = ld16(rec_at(p, so + jo) + 32), r3 = ld16(rec_at(p, so + jo) + 48);
        double oc[PK] = {ent_c(r0), ent_c(r1), ent_c(r2), ent_c(r3)};
        int os[PK] = {int(r0.z), int(r1.z), int(r2.z), int(r3.z)};
        int opp[PK] = {int(r0.w), int(r1.w), int(r2.w), int(r3.w)};
        bool change = os[0] == -1;
#pragma unroll
        for (int k = 0; k < PK; ++k)
          change |= os[k] >= 0 && (os[k] == surv || os[k] == gone || pm_better(cs, ps, oc[k], opp[k]));
        if (!change) {
          hq.row(oc[0], os[0], opp[0], pj, jo);
          return;
        }
        double jc[PK];
        int jp[PK], js[PK];
        list_clear(jc, jp, js);
        int n = 0;
        bool any = false;
        double last_c = -INFINITY, kept_c = -INFINITY;
        int last_p = NOPOS, kept_p = NOPOS;
#pragma unroll
        for (int k = 0; k < PK; ++k) {
          if (os[k] < 0) continue;
          any = true;
          last_c = oc[k];
          last_p = opp[k];
          if (os[k] == surv || os[k] == gone) continue;
          pk_insert(jc, jp, js, oc[k], opp[k], os[k]);
          kept_c = oc[k];
          kept_p = opp[k];
          ++n;
        }
        bool stale = false;
        if (n > 0) {
          // the merged entry joins when it ranks above the kept list's last entry
          if (pm_better(cs, ps, kept_c, kept_p)) pk_insert(jc, jp, js, cs, ps, surv);
        } else if (any && pm_better(cs, ps, last_c, last_p)) {
          // every other partner ranks below the old last entry, so below the merged one
          pk_insert(jc, jp, js, cs, ps, surv);
        } else {
          stale = true;
        }
        if (stale) {
          const double b = any ? last_c : INFINITY;
          rec_store_stale(p, so + jo, b);
          sum_store_stale(p, so + jo, b);
          jc[0] = b;
          js[0] = STALE;
        } else {
          rec_store(p, so + jo, jc, jp, js);
          sum_store_list(p, so + jo, jc, js);
        }
        hq.row(jc[0], js[0], jp[0], pj, jo);
      };
      for (int k0 = 0; k0 < n_live; k0 += PL_W * 4 * NS) {
        Chunk8<T> kc[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          const int k = k0 + (wave * NS + (i ^ own)) * 4 + gi;
          if (k < n_live) kc[i].load(Kc + int64_t(sh.live[k]) * HD * ES, e);
          else kc[i].zero();
        }
        // this lane's row: step own of its group; its summary (no list)
        const int ko = k0 + (wave * NS + own) * 4 + gi;
        const int jo = (lead && ko < n_live) ? sh.live[ko] : -1;
        u32x4 s0 = u32x4{0u, 0u, 0u, 0u}, s1 = u32x4{0u, 0u, SUM_NONE, SUM_NONE};
        if (jo >= 0) {
          s0 = ld16(sum_at(p, so + jo));
          s1 = ld16(sum_at(p, so + jo) + 16);
        }
        double part[NS];
#pragma unroll
        for (int i = 0; i < NS; ++i) {
          double dot = 0.0;
#pragma unroll
          for (int v = 0; v < 8; ++v) dot = fma(qv[v], kc[i].get(v), dot);
          part[i] = dot;
          __builtin_amdgcn_sched_barrier(0);   // one step's conversions live at a time
        }
        const double mine = preduce<16, NS, 0>(part);
        if (jo == gone) sh.gidx = ko;
        if (jo >= 0 && jo != surv && jo != gone) {
          const double nj = ent_c(s0);
          const int pj = int(s0.z);
          const double den = nk * nj;
          const double cs = den > 0.0 ? mine / den : 0.0;
          pk_offer(lc, lp, ls, cs, pj, jo);
          const uint32_t h0 = s1.z & 0xffffu;
          if (h0 == SUM_STALE) {
            hn.bound(ent_c(s1));   // a stale row keeps its bound
          } else if (h0 == SUM_NONE || sum_has(s1.z, s1.w, surv) || sum_has(s1.z, s1.w, gone) ||
                     cs >= double(__int_as_float(int(s0.w)))) {
            // the list may change (no entry, an entry of the merged pair, or the merged entry
            // at least as close as its last entry): after the pass
            const int t = atomicAdd(&sh.n_cand, 1);
            if (t < PL_CAND) {
              sh.cand_c[t] = cs;
              sh.cand_row[t] = jo;
              sh.cand_pos[t] = pj;
            } else {
              list_update(jo, pj, cs, hn);
            }
          } else {
            hn.sum_row(s0, s1, jo);   // unchanged
          }
        }
      }
      // ---- the rows whose list may change, with their lists loaded together
      __syncthreads();
      {
        const int nc = min(sh.n_cand, PL_CAND);
        for (int t = tid; t < nc; t += PL_NT) list_update(sh.cand_row[t], sh.cand_pos[t], sh.cand_c[t], hn);
      }
      // the merged row's list: best PK of the wave, then of the waves
      double wc_[PK];
      int wp_[PK], ws_[PK];
      wave_topk(lc, lp, ls, lane, wc_, wp_, ws_);
      if (lane == 0) {
#pragma unroll
        for (int k = 0; k < PK; ++k) {
          sh.lc[0][wave][k] = wc_[k];
          sh.lp[0][wave][k] = wp_[k];
          sh.ls[0][wave][k] = ws_[k];
        }
      }
      heads_to_lds(sh, hn, lane, wave);
      __syncthreads();
      double fc[PK];
      int fp[PK], fs[PK];
      final_list(sh, 0, lane, fc, fp, fs);
      if (tid == 0) {
        rec_store(p, so + surv, fc, fp, fs);
        sum_store_list(p, so + surv, fc, fs);
        const int g = sh.gidx;
        if (g >= 0 && g < n_live && sh.live[g] == gone) sh.live[g] = sh.live[n_live - 1];
        else p.status[0] = -7;   // cannot happen: the removed slot was a listed candidate
      }
      h.clear();
      h.row(fc[0], fs[0], fp[0], ps, surv);
      heads_from_lds(sh, h);
      // the chosen head's partner position (summaries do not carry it)
      if (h.s >= 0) h.pj = p.pos[so + h.sj];
    }
    --n_live;
    --live;
    ++merged;
  }
  if (tid == 0 && p.n_merged) p.n_merged[sc] = merged;
}

}  // namespace

hipError_t launch_prefill_merge(const PrefillMergeArgs &p, int dtype, hipStream_t st, hipEvent_t *marks) {
  const dim3 g1((p.capacity + 255) / 256, p.n_scopes), g2((p.capacity + PM_ROWS - 1) / PM_ROWS, p.n_scopes);
  const bool bf = dtype == 0;
  if (marks) hipEventRecord(marks[0], st);
  if (bf) hipLaunchKernelGGL(k_pm_prep<bf16_t>, g1, dim3(256), 0, st, p);
  else hipLaunchKernelGGL(k_pm_prep<float>, g1, dim3(256), 0, st, p);
  if (marks) hipEventRecord(marks[1], st);
  if (bf) hipLaunchKernelGGL(k_pm_rows<bf16_t>, g2, dim3(PM_NT), 0, st, p);
  else hipLaunchKernelGGL(k_pm_rows<float>, g2, dim3(PM_NT), 0, st, p);
  if (marks) hipEventRecord(marks[2], st);
  if (bf) hipLaunchKernelGGL(k_pm_loop<bf16_t>, dim3(p.n_scopes), dim3(PL_NT), 0, st, p);
  else hipLaunchKernelGGL(k_pm_loop<float>, dim3(p.n_scopes), dim3(PL_NT), 0, st, p);
  if (marks) hipEventRecord(marks[3], st);
  return hipGetLastError();
}

}  // namespace kvc
