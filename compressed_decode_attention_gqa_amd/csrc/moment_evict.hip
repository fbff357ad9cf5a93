// MomentKV moment-informed eviction (summary page, §4.2 "moment residual" and
// "moment-aware eviction score", Algorithm 1 phase 1) on per-KV-head scopes.
//
// For every live token j of a head, with the evicted set known through its sums
// (n_e, s_k, s_v, S):
//   r_j = v_j - v_bar - tau S_tilde (k_j - k_bar) / n_e = v_j - c - A k_j,
//   A = tau S_tilde / n_e,  c = v_bar - A k_bar,  S_tilde = S - s_v s_k^T / n_e,
//   score(j) = alpha_j ||r_j||  (r_j = v_j when n_e = 0),
// and the lowest score is evicted and folded into the sums before the next
// round. All residual arithmetic is float64.
//
// One round is two kernels:
//   k_me_score  (grid: chunks x scopes, 8 waves) stages -A in LDS as float64
//               MFMA A-fragments (128 KB), then each wave contracts it with 16
//               keys at a time on v_mfma_f64_16x16x4 (256 MFMAs per tile),
//               starting from the accumulator v_j - c, squares and sums the
//               residual rows, scores, and keeps its lowest candidate;
//   k_me_pick   (grid: scopes) takes the lowest chunk candidate (ties to the
//               lower position), flags it and folds its rows into the sums.
// When one chunk covers every scope (chunk >= capacity) the score kernel's
// workgroup picks and folds itself and the second kernel is not launched.
//
// The contraction runs on the float64 MFMA operator of kvc_f64mfma.h (the
// model -A in LDS; each lane's B values and accumulator rows are the same 32
// elements of its key and value rows).
#include "kvc_f64mfma.h"
#include "kvc_kernels.h"

namespace kvc {
namespace {

constexpr int ME_SWG = 512;     // score workgroup: 8 waves, two per SIMD, so one wave's
                                // per-tile vector work overlaps the other's MFMAs
constexpr int ME_SWAVES = ME_SWG / 64;
constexpr int ME_WAVES = WG / 64;
constexpr int ME_CPAD = 36;     // c is stored [g][36]: the four lane groups read distinct banks

struct MeLds {
  FmOperator op;                // -A (128 KB)
  double c[4 * ME_CPAD];        // c = v_bar - A k_bar (zero when n_e = 0), row a at (a/32)*36 + a%32
  double best[ME_SWAVES];
  int best_pos[ME_SWAVES], best_slot[ME_SWAVES];
};

// (score, pos) ascending; +inf for no candidate.
__device__ __forceinline__ bool me_less(double s, int p, double s2, int p2) {
  return s < s2 || (s == s2 && p < p2);
}

// Algorithm 1 steps 12-13 for evicted slot e of scope sc (fp32 sums, one fused
// multiply-add per element): s_k += k_e, s_v += v_e, S += v_e k_e^T, by NT threads.
template <typename T, int NT>
__device__ __forceinline__ void me_fold(const MomentEvictArgs &p, int sc, int e, int tid) {
  const int64_t row = int64_t(sc) * p.scope_stride + e;
  const T *kr = reinterpret_cast<const T *>(p.k) + row * HD;
  const T *vr = reinterpret_cast<const T *>(p.v) + row * HD;
  float *S = p.S + int64_t(sc) * HD * HD;
  constexpr int PER = HD * HD / 4 / NT;
  const int b0 = (tid & 31) * 4;   // every iteration covers the same four columns
  float4 s4[PER];
  float va[PER];
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int a = (tid + it * NT) >> 5;
    s4[it] = *reinterpret_cast<const float4 *>(S + a * HD + b0);
    va[it] = load_elem<T>(vr, a);
  }
  const float k0 = load_elem<T>(kr, b0), k1 = load_elem<T>(kr, b0 + 1), k2 = load_elem<T>(kr, b0 + 2),
              k3 = load_elem<T>(kr, b0 + 3);
  if (tid < HD) {
    p.sk[int64_t(sc) * HD + tid] += load_elem<T>(kr, tid);
    p.sv[int64_t(sc) * HD + tid] += load_elem<T>(vr, tid);
  }
#pragma unroll
  for (int it = 0; it < PER; ++it) {
    const int a = (tid + it * NT) >> 5;
    s4[it].x = fmaf(va[it], k0, s4[it].x);
    s4[it].y = fmaf(va[it], k1, s4[it].y);
    s4[it].z = fmaf(va[it], k2, s4[it].z);
    s4[it].w = fmaf(va[it], k3, s4[it].w);
    *reinterpret_cast<float4 *>(S + a * HD + b0) = s4[it];
  }
}

template <typename T>
__global__ __launch_bounds__(ME_SWG, 1) void k_me_score(MomentEvictArgs p, int iter) {
  __shared__ MeLds sh;
  const int sc = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = min(p.len[sc], p.capacity);
  const int k_sc = L - p.budget;
  if (p.fused_pick && iter == 0 && tid == 0) {
    // a live length beyond the capacity, or more evictions than the host bound allows rounds for
    if (p.len[sc] > p.capacity || k_sc > p.rounds) p.status[0] = -4;
    if (p.n_evict) p.n_evict[sc] = min(max(k_sc, 0), p.rounds);
  }
  if (iter > 0 && iter >= k_sc) return;
  const int j_begin = blockIdx.x * p.chunk;
  if (j_begin >= L) return;
  const int j_end = min(L, j_begin + p.chunk);

  // ---- stage -A = -tau S_tilde / n_e as fragments, and c = v_bar - A k_bar
  {
    constexpr int PER = HD * HD / 4 / ME_SWG;   // float4 of S per thread
    const int n = p.mom_n[sc];
    const float *S = p.S + int64_t(sc) * HD * HD;
    const float *sk = p.sk + int64_t(sc) * HD;
    const float *sv = p.sv + int64_t(sc) * HD;
    float4 s4[PER];
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int e4 = tid + it * ME_SWG;
      s4[it] = *reinterpret_cast<const float4 *>(S + (e4 >> 5) * HD + (e4 & 31) * 4);
    }
    // this thread's four columns are the same in every iteration
    const int b0 = (tid & 31) * 4;
    float4 sk4 = *reinterpret_cast<const float4 *>(sk + b0);
    const double inv_n = n > 0 ? 1.0 / double(n) : 0.0;
    const double f = -p.scale * inv_n;
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int a = (tid + it * ME_SWG) >> 5;
      const double sva = double(sv[a]) * inv_n;
      double dot = 0.0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const double skb = t == 0 ? sk4.x : t == 1 ? sk4.y : t == 2 ? sk4.z : sk4.w;
        const double sab = t == 0 ? s4[it].x : t == 1 ? s4[it].y : t == 2 ? s4[it].z : s4[it].w;
        const double an = n > 0 ? f * (sab - sva * skb) : 0.0;   // -A[a][b]
        fm_put(sh.op, a, b0 + t, an);
        dot = fma(an, skb * inv_n, dot);
      }
      // the 32 lanes of one row a hold its 128 columns: c[a] = v_bar[a] + sum_b (-A[a][b]) k_bar[b]
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) dot += __shfl_xor(dot, o);
      if ((lane & 31) == 0) sh.c[(a >> 5) * ME_CPAD + (a & 31)] = n > 0 ? sva + dot : 0.0;
    }
  }
  __syncthreads();

  // ---- residual tiles: wave w takes tiles w, w + 8, ...
  const int g = lane >> 4, jl = lane & 15;
  const int64_t row0 = int64_t(sc) * p.scope_stride;
  const char *kb = p.k, *vb = p.v;
  constexpr int ES = sizeof(T);
  const double *cg = sh.c + g * ME_CPAD;
  double best = __builtin_inf();
  int best_pos = 0x7fffffff, best_slot = -1;
  const int n_tiles = (j_end - j_begin + FM_TILE - 1) / FM_TILE;
  for (int tile = wave; tile < n_tiles; tile += ME_SWAVES) {
    const int j = j_begin + tile * FM_TILE + jl;
    const int jc = min(j, j_end - 1);
    const int64_t slot = int64_t(sc) * p.capacity + jc;
    const float al_t = p.alpha[slot];
    const int ps_t = p.pos[slot];
    const int ev_t = iter > 0 ? p.evict[slot] : 0;
    const int64_t off = ((row0 + jc) * HD + 32 * g) * ES;
    FmRow<T> kr, vr;
    kr.load(kb + off);
    vr.load(vb + off);
    double x[32];
#pragma unroll
    for (int s = 0; s < 32; ++s) x[s] = kr.get(s);
    fm_d4 acc[FM_RT];
#pragma unroll
    for (int rt = 0; rt < FM_RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[rt][r] = vr.get(4 * rt + r) - cg[4 * rt + r];
    fm_apply(sh.op, lane, x, acc);
    double ss = 0.0;
#pragma unroll
    for (int rt = 0; rt < FM_RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) ss = fma(acc[rt][r], acc[rt][r], ss);
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (j < j_end && ev_t == 0) {
      const double score = double(al_t) * sqrt(ss);
      if (iter == 0 && g == 0) {
        p.evict[slot] = 0;
        if (p.score_out) p.score_out[slot] = float(score);
      }
      if (me_less(score, ps_t, best, best_pos)) {
        best = score;
        best_pos = ps_t;
        best_slot = j;
      }
    }
  }
  // ---- lowest (score, pos) of the workgroup
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double ob = __shfl_xor(best, o);
    const int op = __shfl_xor(best_pos, o), os = __shfl_xor(best_slot, o);
    if (me_less(ob, op, best, best_pos)) {
      best = ob;
      best_pos = op;
      best_slot = os;
    }
  }
  if (lane == 0) {
    sh.best[wave] = best;
    sh.best_pos[wave] = best_pos;
    sh.best_slot[wave] = best_slot;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < ME_SWAVES; ++w)
      if (me_less(sh.best[w], sh.best_pos[w], best, best_pos)) {
        best = sh.best[w];
        best_pos = sh.best_pos[w];
        best_slot = sh.best_slot[w];
      }
    if (!p.fused_pick) {
      const int64_t ci = int64_t(sc) * p.n_chunks + blockIdx.x;
      p.cand_score[ci] = best;
      p.cand_pos[ci] = best_pos;
      p.cand_slot[ci] = best_slot;
    } else {
      // one chunk holds the whole scope: this workgroup's lowest is the scope's
      const bool take = iter < k_sc && best_slot >= 0;
      sh.best_slot[0] = take ? best_slot : -1;
      if (take) {
        p.evict[int64_t(sc) * p.capacity + best_slot] = 1;
        if (p.order) p.order[int64_t(sc) * p.capacity + iter] = best_slot;
        p.mom_n[sc] += 1;
      }
    }
  }
  if (!p.fused_pick) return;
  __syncthreads();
  const int e = sh.best_slot[0];
  if (e >= 0) me_fold<T, ME_SWG>(p, sc, e, tid);
}

// Lowest chunk candidate of the scope -> evicted; fold its rows into the sums
// (Algorithm 1 steps 11-13: n_e += 1, s_k += k, s_v += v, S += v k^T, fp32).
template <typename T>
__global__ __launch_bounds__(WG) void k_me_pick(MomentEvictArgs p, int iter) {
  __shared__ double wb[ME_WAVES];
  __shared__ int wp[ME_WAVES], ws[ME_WAVES];
  __shared__ int pick;
  const int sc = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = min(p.len[sc], p.capacity);
  const int k_sc = L - p.budget;
  if (iter == 0 && tid == 0) {
    // a live length beyond the capacity, or more evictions than the host bound allows rounds for
    if (p.len[sc] > p.capacity || k_sc > p.rounds) p.status[0] = -4;
    if (p.n_evict) p.n_evict[sc] = min(max(k_sc, 0), p.rounds);
  }
  if (iter >= k_sc) return;
  const int n_ch = (L + p.chunk - 1) / p.chunk;
  double best = __builtin_inf();
  int best_pos = 0x7fffffff, best_slot = -1;
  for (int c = tid; c < n_ch; c += WG) {
    const int64_t ci = int64_t(sc) * p.n_chunks + c;
    const double s = p.cand_score[ci];
    const int ps = p.cand_pos[ci], sl = p.cand_slot[ci];
    if (sl >= 0 && me_less(s, ps, best, best_pos)) {
      best = s;
      best_pos = ps;
      best_slot = sl;
    }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double ob = __shfl_xor(best, o);
    const int op = __shfl_xor(best_pos, o), os = __shfl_xor(best_slot, o);
    if (os >= 0 && (best_slot < 0 || me_less(ob, op, best, best_pos))) {
      best = ob;
      best_pos = op;
      best_slot = os;
    }
  }
  if (lane == 0) {
    wb[wave] = best;
    wp[wave] = best_pos;
    ws[wave] = best_slot;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < ME_WAVES; ++w)
      if (ws[w] >= 0 && (best_slot < 0 || me_less(wb[w], wp[w], best, best_pos))) {
        best = wb[w];
        best_pos = wp[w];
        best_slot = ws[w];
      }
    pick = best_slot;
    if (best_slot >= 0) {
      p.evict[int64_t(sc) * p.capacity + best_slot] = 1;
      if (p.order) p.order[int64_t(sc) * p.capacity + iter] = best_slot;
      p.mom_n[sc] += 1;
    }
  }
  __syncthreads();
  const int e = pick;
  if (e >= 0) me_fold<T, WG>(p, sc, e, tid);
}

}  // namespace

hipError_t launch_moment_evict(const MomentEvictArgs &p, int dtype, int rounds, hipStream_t st) {
  const dim3 sgrid(p.n_chunks_used, p.n_scopes);
  for (int it = 0; it < rounds; ++it) {
    if (dtype == 0) {
      hipLaunchKernelGGL(k_me_score<bf16_t>, sgrid, dim3(ME_SWG), 0, st, p, it);
      if (!p.fused_pick) hipLaunchKernelGGL(k_me_pick<bf16_t>, dim3(p.n_scopes), dim3(WG), 0, st, p, it);
    } else {
      hipLaunchKernelGGL(k_me_score<float>, sgrid, dim3(ME_SWG), 0, st, p, it);
      if (!p.fused_pick) hipLaunchKernelGGL(k_me_pick<float>, dim3(p.n_scopes), dim3(WG), 0, st, p, it);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvc
