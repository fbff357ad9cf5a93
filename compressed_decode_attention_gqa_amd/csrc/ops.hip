// Standalone entry-point kernels: utility update, the selection of one very
// large scope (a model-wide Top-K), the fp32 moment fold and KeepKV ZIP
// merging. (Selection and compaction over many scopes, and the bf16 moment
// fold, run on the grid-wide kernels of bulk.hip.)
#include "kvc_ops.h"
#include "kvc_kernels.h"

namespace kvc {

// ------------------------------------------------------------ utility update
// InertiaKV §3.1 eqs. (2)-(4).
__global__ __launch_bounds__(WG) void k_ema_update(float *m, const float *s, const int32_t *len,
                                                  int cap, int rule, float alpha) {
  const int scope = blockIdx.y;
  const int i = blockIdx.x * WG + threadIdx.x;
  const int L = len[scope];
  if (i >= L || i >= cap) return;
  const int64_t o = int64_t(scope) * cap + i;
  const double sv = s[o], mo = m[o], al = alpha;
  double r;
  if (rule == 0) r = sv;
  else if (rule == 1) r = mo + sv;
  else r = al * mo + (1.0 - al) * sv;
  m[o] = float(r);
}

// ------------------------------------------------------------ selection (device-wide, one scope)
// Radix select over n keys spread across many workgroups: per pass a global
// 256-bin histogram of the keys matching the current prefix, then one
// workgroup picks the digit. Keys must be distinct (distinct positions).
struct WideState {
  uint64_t prefix, mask;
  int32_t krem, done, k, pad;
  uint32_t hist[256];
};

__device__ __forceinline__ uint64_t wide_key(const float *key, const int32_t *pos, int64_t i) {
  return order_key(key[i], pos ? uint32_t(pos[i]) : uint32_t(i));
}

__global__ __launch_bounds__(WG) void k_wide_hist(const float *key, const int32_t *pos, int64_t n,
                                                 WideState *st, int shift) {
  __shared__ uint32_t hist[256];
  if (st->done) return;
  hist[threadIdx.x] = 0;
  __syncthreads();
  const uint64_t prefix = st->prefix, mask = st->mask;
  for (int64_t i = int64_t(blockIdx.x) * WG + threadIdx.x; i < n; i += int64_t(gridDim.x) * WG) {
    const uint64_t kk = wide_key(key, pos, i);
    if ((kk & mask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
  }
  __syncthreads();
  const uint32_t c = hist[threadIdx.x];
  if (c) atomicAdd(&st->hist[threadIdx.x], c);
}

__global__ __launch_bounds__(WG) void k_wide_pick(WideState *st, int shift) {
  __shared__ int red[8];
  if (st->done) return;
  const int tid = threadIdx.x;
  const int c = int(st->hist[tid]);
  int tot;
  const int excl = wg_exclusive_scan(c, red, &tot);
  const int krem = st->krem;
  __syncthreads();
  if (excl < krem && krem <= excl + c) {
    st->prefix |= uint64_t(tid) << shift;
    st->mask |= uint64_t(255) << shift;
    st->krem = krem - excl;
    if (c == krem - excl || shift == 0) st->done = 1;
  }
  __syncthreads();
  st->hist[tid] = 0;
}

__global__ __launch_bounds__(WG) void k_wide_flags(const float *key, const int32_t *pos, int64_t n,
                                                  const WideState *st, uint8_t *evict) {
  const uint64_t thr = st->prefix, mask = st->mask;
  for (int64_t i = int64_t(blockIdx.x) * WG + threadIdx.x; i < n; i += int64_t(gridDim.x) * WG)
    evict[i] = (wide_key(key, pos, i) & mask) <= thr;
}

__global__ void k_wide_init(WideState *st, int k, int32_t *n_evict) {
  if (threadIdx.x == 0) {
    st->prefix = 0;
    st->mask = 0;
    st->krem = k;
    st->k = k;
    st->done = k == 0 ? 1 : 0;
    if (n_evict) *n_evict = k;
  }
  st->hist[threadIdx.x] = 0;
}

__global__ void k_wide_clear(int64_t n, uint8_t *evict) {
  for (int64_t i = int64_t(blockIdx.x) * WG + threadIdx.x; i < n; i += int64_t(gridDim.x) * WG) evict[i] = 0;
}

size_t wide_state_bytes() { return sizeof(WideState); }

hipError_t launch_select_wide(const float *key, const int32_t *pos, int cap, int budget, uint8_t *evict,
                              int32_t *n_evict, void *ws, hipStream_t st) {
  WideState *w = reinterpret_cast<WideState *>(ws);
  const int k = max(0, cap - budget);
  const int grid = 2048;
  hipLaunchKernelGGL(k_wide_init, dim3(1), dim3(256), 0, st, w, k, n_evict);
  if (k == 0) {
    hipLaunchKernelGGL(k_wide_clear, dim3(grid), dim3(WG), 0, st, int64_t(cap), evict);
    return hipGetLastError();
  }
  for (int shift = 56; shift >= 0; shift -= 8) {
    hipLaunchKernelGGL(k_wide_hist, dim3(grid), dim3(WG), 0, st, key, pos, int64_t(cap), w, shift);
    hipLaunchKernelGGL(k_wide_pick, dim3(1), dim3(WG), 0, st, w, shift);
  }
  hipLaunchKernelGGL(k_wide_flags, dim3(grid), dim3(WG), 0, st, key, pos, int64_t(cap), w, evict);
  return hipGetLastError();
}

// ------------------------------------------------------------ moment fold
template <typename T>
__global__ __launch_bounds__(WG) void k_moment_update(CacheArgs c, const uint8_t *evict, int32_t *n,
                                                     float *sk, float *sv, float *S) {
  __shared__ FoldLds sh;
  const int scope = blockIdx.x / c.units, u = blockIdx.x - (blockIdx.x / c.units) * c.units;
  const int L = c.len[scope];
  const int64_t row0 = int64_t(scope) * c.scope_stride + int64_t(u) * c.unit_stride;
  const T *Kb = reinterpret_cast<const T *>(c.k) + row0 * HD;
  const T *Vb = reinterpret_cast<const T *>(c.v) + row0 * HD;
  const int64_t mu = blockIdx.x;
  fold_flagged<T>(Kb, Vb, evict + int64_t(scope) * c.capacity, L, n + mu, sk + mu * HD, sv + mu * HD,
                  S + mu * HD * HD, sh);
}

hipError_t launch_moment_update(const CacheArgs &c, const uint8_t *evict, int32_t *n, float *sk,
                                float *sv, float *S, hipStream_t st) {
  dim3 grid(c.n_scopes * c.units);
  if (c.dtype == 0) hipLaunchKernelGGL(k_moment_update<bf16_t>, grid, dim3(WG), 0, st, c, evict, n, sk, sv, S);
  else hipLaunchKernelGGL(k_moment_update<float>, grid, dim3(WG), 0, st, c, evict, n, sk, sv, S);
  return hipGetLastError();
}

// ------------------------------------------------------------ ZIP merge
// KeepKV eqs. (7)-(12): the single flagged entry e of each scope is merged into
// its live partner c of largest cos(k_e, k_c) (ties to the lower position),
// then dropped. k_merge_part: each workgroup takes a token range and stores its
// best (cosine, slot); k_merge_finish: one workgroup per scope picks the
// partner over the ranges, merges and compacts.
struct MergeLds {
  double ke[HD];
  double best_cos[4];
  int best_slot[4];
  int best_pos[4];
  int e, n_flagged;
  double lbar[2];
  double wgt[4];
};

__device__ __forceinline__ bool cos_better(double c1, int p1, double c2, int p2) {
  return c1 > c2 || (c1 == c2 && p1 < p2);
}

// The flagged slot of the scope (the largest one if several), or -1; *count
// (if non-null) receives the number of flagged slots.
// The flags are read 16 bytes per load over the 16-byte-aligned middle of
// [0, L) and byte by byte at its two ends; each thread reports its largest
// flagged slot and its count once.
__device__ __forceinline__ int merge_flagged(const uint8_t *flags, int L, int &sh_e, int *sh_n = nullptr,
                                             int *count = nullptr) {
  if (threadIdx.x == 0) {
    sh_e = -1;
    if (sh_n) *sh_n = 0;
  }
  __syncthreads();
  const int head = min(L, int((16u - (reinterpret_cast<uintptr_t>(flags) & 15u)) & 15u));
  const int nvec = (L - head) / 16, body_end = head + 16 * nvec;
  int e = -1, n = 0;
  for (int i = threadIdx.x; i < head; i += WG)
    if (flags[i]) {
      e = max(e, i);
      ++n;
    }
  for (int i = body_end + threadIdx.x; i < L; i += WG)
    if (flags[i]) {
      e = max(e, i);
      ++n;
    }
  for (int v = threadIdx.x; v < nvec; v += WG) {
    const u32x4 x = *reinterpret_cast<const u32x4 *>(flags + head + 16 * v);
    if ((x.x | x.y | x.z | x.w) != 0u) {
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const uint32_t w = b < 4 ? x.x : b < 8 ? x.y : b < 12 ? x.z : x.w;
        if ((w >> (8 * (b & 3))) & 255u) {
          e = max(e, head + 16 * v + b);
          ++n;
        }
      }
    }
  }
  if (e >= 0) {
    atomicMax(&sh_e, e);
    if (sh_n) atomicAdd(sh_n, n);
  }
  __syncthreads();
  if (count) *count = *sh_n;
  return sh_e;
}

// The decode step's selection in the merge kernels (MergeArgs::cand_key set): the
// entry of the lowest (utility, position) key over the scope's score-chunk
// candidates when the live length L is exactly one over the budget, else -1.
// Wave-level (all lanes active). The lane's first candidate is loaded at kernel
// entry, beside the length, for the chunks of the launch's length bound (those
// past the live length are masked once it is known); only chunks past 64 lanes
// or past the bound load afterwards.
struct MergeCand {
  uint64_t key;
  uint32_t pos;
  int slot;
};

__device__ __forceinline__ MergeCand merge_cand_load(const MergeArgs &mg, int scope) {
  const int lane = threadIdx.x & 63;
  MergeCand m{~0ull, 0xffffffffu, -1};
  if (lane < min(mg.cand_max, mg.n_score_chunks)) {
    const int64_t ci = int64_t(scope) * mg.n_score_chunks + lane;
    m.key = mg.cand_key[ci];
    m.pos = uint32_t(mg.cand_pos[ci]);
    m.slot = mg.cand_slot[ci];
  }
  return m;
}

__device__ int merge_step_pick(const MergeArgs &mg, MergeCand m, int scope, int L, int cap) {
  if (L > cap || L - mg.budget != 1) return -1;
  const int lane = threadIdx.x & 63;
  const int nch = (L + mg.score_chunk - 1) / mg.score_chunk;
  uint64_t best = ~0ull;
  uint32_t bpos = 0xffffffffu;
  int bslot = -1;
  if (lane < nch && lane < mg.cand_max) {
    best = m.key;
    bpos = m.pos;
    bslot = m.slot;
  }
  for (int ch = lane < mg.cand_max ? lane + 64 : lane; ch < nch; ch += 64) {
    const int64_t ci = int64_t(scope) * mg.n_score_chunks + ch;
    const uint64_t key = mg.cand_key[ci];
    const uint32_t p = uint32_t(mg.cand_pos[ci]);
    const int sl = mg.cand_slot[ci];
    if (key_pos_less(key, p, best, bpos)) {
      best = key;
      bpos = p;
      bslot = sl;
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t k2 = shfl_xor_u64(best, o);
    const uint32_t p2 = __shfl_xor(bpos, o);
    const int s2 = __shfl_xor(bslot, o);
    if (key_pos_less(k2, p2, best, bpos)) {
      best = k2;
      bpos = p2;
      bslot = s2;
    }
  }
  return __builtin_amdgcn_readfirstlane(bslot);
}

// Token slot order for the lane-permuted reduction of N per-token partial sums
// over a token's row of lanes: slot i of lane l holds token i ^ merge_perm(l).
// The exchange stages pair lane l with l ^ 16 (32-lane rows), l ^ 15, l ^ 7,
// l ^ 2 and l ^ 1; a linear map taking the first log2(N) of those masks to
// N/2, N/4, ..., 1 and the rest to 0 leaves lane l with the whole sums of
// token merge_perm(l).
template <int LPT, int N>
__device__ __forceinline__ int merge_perm(int l) {
  constexpr int o = LPT == 32 ? 1 : 0;
  constexpr auto T = [](int s) { return (2 << s) <= N ? N >> (s + 1) : 0; };
  constexpr int c0 = T(o + 3), c1 = T(o + 2), c2 = T(o + 1) ^ c0 ^ c1, c3 = T(o) ^ T(o + 1);
  constexpr int c4 = LPT == 32 ? T(0) : 0;
  return ((l & 1) ? c0 : 0) ^ ((l & 2) ? c1 : 0) ^ ((l & 4) ? c2 : 0) ^ ((l & 8) ? c3 : 0) ^ ((l & 16) ? c4 : 0);
}

template <typename T>
__global__ __launch_bounds__(WG) void k_merge_part(CacheArgs c, const uint8_t *evict, MergeArgs mg) {
  __shared__ MergeLds sh;
  constexpr int EPV = ElemTraits<T>::EPV, LPT = HD / EPV, TPI = 64 / LPT, RB = HD * int(sizeof(T));
  // A wave takes every STR-th group of TPI tokens of the workgroup's range, MU
  // groups per batch with all their loads in flight (the whole range of a
  // workgroup at the usual split count). The per-token sums are reduced so that
  // each lane ends with one token's, which it alone turns into a cosine.
  constexpr int STR = (WG / 64) * TPI, MU = 8;
  const int scope = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cb = lane % LPT, tg = lane / LPT, own = merge_perm<LPT, MU>(cb);
  const int64_t so = int64_t(scope) * c.capacity;
  // (a step's length over the capacity merges nothing: no token range then)
  const MergeCand cand0 = mg.cand_key ? merge_cand_load(mg, scope) : MergeCand{};
  const int Lstep = c.len[scope] + (mg.cand_key ? mg.append : 0);
  const int L = Lstep <= c.capacity ? Lstep : 0;
  const char *Kb = reinterpret_cast<const char *>(c.k) + int64_t(scope) * c.scope_stride * RB;
  const int per = (L + gridDim.x - 1) / gridDim.x;
  const int t0 = blockIdx.x * per, t1 = min(L, t0 + per);

  // two batches of loads in flight per wave (A and B in turn); a load past the range reads the
  // range's last row (a line already in L2), so every batch is issued the same way and its
  // registers need no copy that would wait for it
  u32x4 kvA[MU], kvB[MU];
  int pvA, pvB;
  auto issue = [&](u32x4 (&kv)[MU], int &pv, int b0) {
#pragma unroll
    for (int i = 0; i < MU; ++i) {
      const int tok = min(b0 + (i ^ own) * STR + tg, t1 - 1);
      kv[i] = ld16(Kb + int64_t(max(tok, 0)) * RB + 16 * cb);
    }
    const int mine = min(b0 + own * STR + tg, t1 - 1);
    pv = c.pos[so + max(mine, 0)];
  };
  int base = t0 + wave * TPI;
  // these loads do not depend on the flagged slot
  issue(kvA, pvA, base);
  issue(kvB, pvB, base + MU * STR);
  const int e = mg.cand_key ? merge_step_pick(mg, cand0, scope, Lstep, c.capacity)
                : mg.e_slot  ? mg.e_slot[int64_t(scope) * mg.e_stride]
                             : merge_flagged(evict + so, L, sh.e);

  double best = -INFINITY;
  int bslot = -1, bpos = 0x7fffffff;
  if (e >= 0 && t0 < t1) {
    const u32x4 kw = ld16(Kb + int64_t(e) * RB + 16 * cb);
    double ke[EPV];
    double ne = 0.0;
#pragma unroll
    for (int j = 0; j < EPV; ++j) {
      ke[j] = double(ElemTraits<T>::get(kw, j));
      ne = fma(ke[j], ke[j], ne);
    }
    ne = sqrt(group_sum_f64<LPT>(ne));
    // the cosines of one batch with k_e; each lane ends with its token's (whole sums)
    auto batch = [&](const u32x4 (&kv)[MU], int pv, int b0) {
      double pd[MU], pn[MU];
#pragma unroll
      for (int i = 0; i < MU; ++i) {
        double dot = 0.0, nn = 0.0;
#pragma unroll
        for (int j = 0; j < EPV; ++j) {
          const double x = double(ElemTraits<T>::get(kv[i], j));
          dot = fma(ke[j], x, dot);
          nn = fma(x, x, nn);
        }
        pd[i] = dot;
        pn[i] = nn;
      }
      const double dot = preduce<LPT, MU, 0>(pd);
      const double nn = preduce<LPT, MU, 0>(pn);
      const int tok = b0 + own * STR + tg;
      if (tok < t1 && tok != e) {
        const double den = ne * sqrt(nn);
        const double cs = den > 0.0 ? dot / den : 0.0;
        if (cos_better(cs, pv, best, bpos)) {
          best = cs;
          bslot = tok;
          bpos = pv;
        }
      }
    };
    for (;;) {
      batch(kvA, pvA, base);
      issue(kvA, pvA, base + 2 * MU * STR);
      base += MU * STR;
      if (base >= t1) break;
      batch(kvB, pvB, base);
      issue(kvB, pvB, base + 2 * MU * STR);
      base += MU * STR;
      if (base >= t1) break;
    }
  }
  // workgroup argmax
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double b2 = __shfl_xor(best, o);
    const int s2 = __shfl_xor(bslot, o), p2 = __shfl_xor(bpos, o);
    if (s2 >= 0 && (bslot < 0 || cos_better(b2, p2, best, bpos))) {
      best = b2;
      bslot = s2;
      bpos = p2;
    }
  }
  if (lane == 0) {
    sh.best_cos[wave] = best;
    sh.best_slot[wave] = bslot;
    sh.best_pos[wave] = bpos;
  }
  __syncthreads();
  if (tid == 0) {
    double b = -INFINITY;
    int s = -1, p = 0x7fffffff;
    for (int w = 0; w < 4; ++w) {
      const int sw = sh.best_slot[w];
      if (sw < 0) continue;
      const int pw = sh.best_pos[w];
      if (s < 0 || cos_better(sh.best_cos[w], pw, b, p)) {
        b = sh.best_cos[w];
        s = sw;
        p = pw;
      }
    }
    const int64_t pi = int64_t(scope) * gridDim.x + blockIdx.x;
    mg.part_cos[pi] = b;
    mg.part_slot[2 * pi] = s;
    mg.part_slot[2 * pi + 1] = p;
  }
}

template <typename T>
__global__ __launch_bounds__(WG) void k_merge_finish(CacheArgs c, const uint8_t *evict, MergeArgs mg) {
  __shared__ MergeLds sh;
  constexpr int RB = HD * int(sizeof(T)), NV = RB / 16;
  const int scope = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t so = int64_t(scope) * c.capacity;
  const MergeCand cand0 = mg.cand_key ? merge_cand_load(mg, scope) : MergeCand{};
  const int L = c.len[scope] + (mg.cand_key ? mg.append : 0);
  const T *Kb = reinterpret_cast<const T *>(c.k) + int64_t(scope) * c.scope_stride * HD;
  const T *Vb = reinterpret_cast<const T *>(c.v) + int64_t(scope) * c.scope_stride * HD;
  // the ranges' partners (at most 64 ranges) load beside the flagged slot
  double pc = -INFINITY;
  int ps = -1, pp = 0x7fffffff;
  if (wave == 0 && lane < mg.n_splits) {
    const int64_t pi = int64_t(scope) * mg.n_splits + lane;
    pc = mg.part_cos[pi];
    ps = mg.part_slot[2 * pi];
    pp = mg.part_slot[2 * pi + 1];
  }
  // what does not depend on the pair, requested before it is known: the last slot's row
  // (threads HD .. HD + 2 NV - 1), vote, utility and position, which fill the dropped
  // slot; the query heads' elements lane and lane + 64 (the two waves that form the
  // reference logits)
  const bool Lok = L >= 1 && L <= c.capacity;
  const int last = L - 1;
  const int mvc = tid - HD;   // threads HD .. HD + 2 NV - 1 carry the moved row
  const bool mv_thread = mvc >= 0 && mvc < 2 * NV;
  u32x4 mvec = u32x4(0u);
  if (Lok && mv_thread)
    mvec = ld16(reinterpret_cast<const char *>(mvc < NV ? Kb : Vb) + int64_t(last) * RB + 16 * (mvc % NV));
  int vl = 0, pl = 0;
  float ml = 0.f;
  if (Lok && tid == 0) {
    if (c.votes) vl = c.votes[so + last];
    if (c.m) ml = c.m[so + last];
    pl = c.pos[so + last];
  }
  constexpr int GQ = 8;   // query heads per KV head, at most
  double qd[GQ][2];
  if (wave < 2) {
    const T *q = reinterpret_cast<const T *>(mg.q) + int64_t(scope) * mg.G * HD;
#pragma unroll
    for (int g = 0; g < GQ; ++g)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) qd[g][jj] = g < mg.G ? double(load_elem<T>(q, g * HD + lane + 64 * jj)) : 0.0;
  }
  int n_flagged = 1;
  int e;
  if (mg.cand_key) {
    // the step's selection, and the length and status a finish would have set; the
    // length is written after a barrier, once every wave has read it
    if (L > c.capacity) {
      if (tid == 0 && mg.status) mg.status[0] = -4;
      return;
    }
    e = merge_step_pick(mg, cand0, scope, L, c.capacity);
    if (e < 0) {
      __syncthreads();
      if (tid == 0) {
        if (L - mg.budget > 1 && mg.status) mg.status[0] = -3;   // one merge per step
        c.len[scope] = L;
      }
      return;
    }
  } else {
    e = mg.e_slot ? mg.e_slot[int64_t(scope) * mg.e_stride]
                  : merge_flagged(evict + so, L, sh.e, &sh.n_flagged, &n_flagged);
    if (e < 0) return;
  }
  if (n_flagged > 1) {   // one merge per scope and call: leave the scope as it is
    if (tid == 0 && mg.status) mg.status[0] = -3;
    return;
  }
  if (wave == 0) {   // the partner over the ranges: a wave argmax
    double b = ps >= 0 ? pc : -INFINITY;
    int s = ps, p = ps >= 0 ? pp : 0x7fffffff;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const double b2 = __shfl_xor(b, o);
      const int s2 = __shfl_xor(s, o), p2 = __shfl_xor(p, o);
      if (s2 >= 0 && (s < 0 || cos_better(b2, p2, b, p))) {
        b = b2;
        s = s2;
        p = p2;
      }
    }
    if (lane == 0) sh.best_slot[0] = s;
  }
  __syncthreads();
  const int cs = sh.best_slot[0];
  if (cs < 0) {   // a single live entry: nothing to merge into
    if (tid == 0 && mg.cand_key) c.len[scope] = L;
    return;
  }

  // Dropping e lets the last live slot fill its hole. The merged entry goes
  // straight to where it ends: slot e when the partner is that last slot (then
  // nothing else moves), else the partner's slot, with the last slot's row
  // moved into e unless e is the last slot itself.
  const int dst = cs == last ? e : cs;
  const bool move = e < last && cs != last;
  // every row this call reads, before any of it is written
  double kek = 0.0, kck = 0.0, vek = 0.0, vck = 0.0;
  if (tid < HD) {
    kek = double(load_elem<T>(Kb, int64_t(e) * HD + tid));
    kck = double(load_elem<T>(Kb, int64_t(cs) * HD + tid));
    vek = double(load_elem<T>(Vb, int64_t(e) * HD + tid));
    vck = double(load_elem<T>(Vb, int64_t(cs) * HD + tid));
  }
  const bool mover = move && mv_thread;
  char *mrow = reinterpret_cast<char *>(mvc < NV ? c.k : c.v) +
               (int64_t(scope) * c.scope_stride * HD) * int(sizeof(T)) + int64_t(last) * RB + 16 * (mvc % NV);
  int ve = 1, vc = 1, pcs = 0;
  float me = 0.f, mc = 0.f;
  if (tid == 0) {
    if (c.votes) {
      ve = c.votes[so + e];
      vc = c.votes[so + cs];
    }
    if (c.m) {
      me = c.m[so + e];
      mc = c.m[so + cs];
    }
    pcs = c.pos[so + cs];
  }

  // reference logits: mean over the G query heads of scale * q_g . k
  if (wave < 2) {
    const int x = wave == 0 ? e : cs;
    double acc = 0.0;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const double kx = double(load_elem<T>(Kb, int64_t(x) * HD + lane + 64 * jj));
      double qs = 0.0;
#pragma unroll
      for (int g = 0; g < GQ; ++g)
        if (g < mg.G) qs += qd[g][jj] * kx;
      acc += qs;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) sh.lbar[wave] = acc * mg.scale / double(mg.G);
  }
  __syncthreads();
  if (tid == 0) {
    const double le = sh.lbar[0], lc = sh.lbar[1];
    const double mu = fmax(le, lc);
    const double pe = c.votes ? double(ve) : 1.0;
    const double pcv = c.votes ? double(vc) : 1.0;
    const double we = pe * exp(le - mu), wc = pcv * exp(lc - mu);
    const double num = mu + log(we + wc) - log(pe + pcv);
    const double den = we * le + wc * lc;
    const bool guarded = fabs(den) < double(mg.eps) * exp(-mu);
    sh.wgt[0] = we / (we + wc);
    sh.wgt[1] = wc / (we + wc);
    sh.wgt[2] = guarded ? 0.5 : we * num / den;
    sh.wgt[3] = guarded ? 0.5 : wc * num / den;
  }
  __syncthreads();   // also orders every read above before the writes below
  if (tid < HD) {
    T *Kw = reinterpret_cast<T *>(c.k) + int64_t(scope) * c.scope_stride * HD;
    T *Vw = reinterpret_cast<T *>(c.v) + int64_t(scope) * c.scope_stride * HD;
    store_elem<T>(Kw, int64_t(dst) * HD + tid, round_once<T>(sh.wgt[2] * kek + sh.wgt[3] * kck));
    store_elem<T>(Vw, int64_t(dst) * HD + tid, round_once<T>(sh.wgt[0] * vek + sh.wgt[1] * vck));
  }
  if (mover) st16(mrow + int64_t(e - last) * RB, mvec);
  if (tid == 0) {
    if (c.votes) c.votes[so + dst] = ve + vc;
    if (c.m) c.m[so + dst] = mc + me;
    c.pos[so + dst] = pcs;
    if (move) {
      if (c.votes) c.votes[so + e] = vl;
      if (c.m) c.m[so + e] = ml;
      c.pos[so + e] = pl;
    }
    c.len[scope] = last;
  }
}

hipError_t launch_merge(const CacheArgs &c, const uint8_t *evict, const MergeArgs &mg, hipStream_t st) {
  const dim3 grid(mg.n_splits, c.n_scopes);
  if (c.dtype == 0) {
    hipLaunchKernelGGL(k_merge_part<bf16_t>, grid, dim3(WG), 0, st, c, evict, mg);
    hipLaunchKernelGGL(k_merge_finish<bf16_t>, dim3(c.n_scopes), dim3(WG), 0, st, c, evict, mg);
  } else {
    hipLaunchKernelGGL(k_merge_part<float>, grid, dim3(WG), 0, st, c, evict, mg);
    hipLaunchKernelGGL(k_merge_finish<float>, dim3(c.n_scopes), dim3(WG), 0, st, c, evict, mg);
  }
  return hipGetLastError();
}

}  // namespace kvc

namespace kvc {
// KeepKV notes, EMA score prediction eq. (14): the bias-corrected predicted score
// S^t / (1 - alpha^t) of the EMA state S^t after t updates from zero.
__global__ __launch_bounds__(WG) void k_ema_predict(const float *m, const int32_t *len, int cap, double alpha,
                                                   int t, float *out) {
  const int scope = blockIdx.y;
  const int i = blockIdx.x * WG + threadIdx.x;
  const int L = len ? len[scope] : cap;
  if (i >= L || i >= cap) return;
  const int64_t o = int64_t(scope) * cap + i;
  out[o] = float(double(m[o]) / (1.0 - pow(alpha, double(t))));
}

hipError_t launch_ema_predict(const float *m, const int32_t *len, int n_scopes, int cap, float alpha, int t,
                              float *out, hipStream_t st) {
  dim3 grid((cap + WG - 1) / WG, n_scopes);
  hipLaunchKernelGGL(k_ema_predict, grid, dim3(WG), 0, st, m, len, cap, double(alpha), t, out);
  return hipGetLastError();
}

hipError_t launch_ema_update(float *m, const float *s, const int32_t *len, int n_scopes, int cap,
                             int rule, float alpha, hipStream_t st) {
  dim3 grid((cap + WG - 1) / WG, n_scopes);
  hipLaunchKernelGGL(k_ema_update, grid, dim3(WG), 0, st, m, s, len, cap, rule, alpha);
  return hipGetLastError();
}
}  // namespace kvc

// ------------------------------------------------------------ rank-stability diagnostic
// InertiaKV's rank-inertia measure (§3.1, Fig. 1): the Jaccard similarity |A and B| / |A or B|
// of two kept sets over the same slots. One workgroup per scope; lane counts by wave ballots.
namespace kvc {
namespace {
__global__ __launch_bounds__(WG) void k_jaccard(const uint8_t *a, const uint8_t *b, const int32_t *len, int cap,
                                                float *out) {
  __shared__ int inter[WG / 64], uni[WG / 64];
  const int sc = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = len ? min(max(len[sc], 0), cap) : cap;
  const uint8_t *pa = a + int64_t(sc) * cap, *pb = b + int64_t(sc) * cap;
  int ni = 0, nu = 0;
  for (int i0 = 0; i0 < L; i0 += WG) {
    const int i = i0 + tid;
    const bool ka = i < L && pa[i] != 0, kb = i < L && pb[i] != 0;
    const uint64_t bi = __ballot(ka && kb), bu = __ballot(ka || kb);
    if (lane == 0) {
      ni += __popcll(bi);
      nu += __popcll(bu);
    }
  }
  if (lane == 0) {
    inter[wave] = ni;
    uni[wave] = nu;
  }
  __syncthreads();
  if (tid == 0) {
    int ti = 0, tu = 0;
    for (int w = 0; w < WG / 64; ++w) {
      ti += inter[w];
      tu += uni[w];
    }
    out[sc] = tu > 0 ? float(double(ti) / double(tu)) : 1.0f;
  }
}
}  // namespace

hipError_t launch_jaccard(const uint8_t *a, const uint8_t *b, const int32_t *len, int n_scopes, int cap, float *out,
                          hipStream_t st) {
  hipLaunchKernelGGL(k_jaccard, dim3(n_scopes), dim3(WG), 0, st, a, b, len, cap, out);
  return hipGetLastError();
}
}  // namespace kvc
