// LaProx prefill scoring (notes on "Reformulating KV Cache Eviction Problem
// for Long-Context LLM Inference": key design 1, the indicator
// ||A[:, i]||_2 ||(V W_O)[i, :]||_2; key design 2, per-layer normalisation;
// the GQA paragraph, group-averaged attention of the last w queries).
//
// Per unit (layer l, KV head h) with G query heads and w window queries, the
// R = G w window rows (g, j) attend causally: row j sits at position
// N - w + j. Kernels, in launch order:
//   k_lap_gram     M = W_bar W_bar^T (d x d, float64) on v_mfma_f64_16x16x4,
//                  W_bar = sum of the group's W_O^g blocks summed in float64
//                  while its column blocks are staged in LDS; two halves of D
//                  per unit, summed when M is staged.
//   k_lap_window<1> float64 logits of the block's 128 window rows against 16
//                  keys at a time on v_mfma_f64_16x16x4 (tau Q as the operator
//                  in LDS), per-row running max and sum of exp -> partials per
//                  2048-token workgroup.
//   k_lap_rowfin   combines the workgroup partials of every row (fixed order).
//   k_lap_window<2> recomputes the logits; A = exp(l - M) / Z; the group mean
//                  over the G heads of each window row by DPP sums over adjacent
//                  lanes; its square summed over the block's rows -> c^2.
//   k_lap_r2       r_i^2 = ||v_i W_bar||^2 = v_i M v_i^T (the Gram identity:
//                  a d x d instead of a d x D contraction per token) on the
//                  float64 MFMA operator of kvc_f64mfma.h, M staged in LDS.
//   k_lap_p        p_i = c_i r_i (float64) and per-chunk partial sums.
//   k_lap_norm     per-layer sum in fixed order, score = p / sum.
// The model-wide Top-K (key design 3) is kvc_select_evict over the scores.
#include "kvc_f64mfma.h"
#include "kvc_laprox.h"

namespace kvc {
namespace {

// ---------------------------------------------------------------- geometry
constexpr int WM_NT = 512;          // window workgroup: 8 waves, two per SIMD
constexpr int WM_TILE = 2048;       // tokens per window workgroup (16 tiles per wave)
constexpr int WM_ROWS = 128;        // window rows per operator block
constexpr int RPW = 8;              // the row count R = G w must be a multiple of this
constexpr int RB = HD * 2;          // bytes per bf16 row

constexpr int GR_KS = 2;            // halves of D per unit in the Gram kernel
constexpr int GR_NT = 512;          // Gram workgroup: 8 waves, wave w owns output rows 16 w .. + 15
constexpr int GR_KB = 32;           // columns of W_bar per LDS block
constexpr int GR_LD = GR_KB + 2;    // doubles per LDS row (34: 16-byte reads of a 16-lane phase hit distinct banks)

constexpr int R2_NT = 512;          // r^2 workgroup: 8 waves, two per SIMD
constexpr int R2_TOK = 2048;        // tokens per r^2 workgroup (16 tiles per wave)

constexpr int P_CHUNK = 4096;       // tokens per partial sum of p

struct LapArgs {
  const char *q, *k, *v, *wo;
  int n_layers, H, n_kv, N, w, D, G, R, nh, ntiles, nchunks;
  double scale;
  float *score;
  double *gram;               // [units][GR_KS][d][d]
  double *tM, *tZ;            // [units][R][ntiles]
  double *rM, *rZ;            // [units][R]
  float *c2;                  // [units][nh][N]
  float *r2;                  // [units][N]
  double *psum;               // [units][nchunks]
  int64_t kstride;            // rows from one unit's keys to the next (N for LaProx)
  // KeepKV window initialisation of the EMA utility: pass 2 sums gamma_j * (group-mean
  // weight) over the window rows instead of its square, gamma_j = (1 - alpha) alpha^(w-1-j)
  int ema;
  double alpha;
  float *m_out;               // [units] x m_stride utilities (tokens [0, N))
  int64_t m_stride;
};

// ---------------------------------------------------------------- Gram matrix
// grid (units, GR_KS), 512 threads: partial M[a][c] = sum over this half of D of
// W_bar[a][b] W_bar[c][b]. Blocks of 32 columns of W_bar (all 128 rows) are
// summed over the group in float64 and staged in LDS (double-buffered, one
// barrier per block); in a block, lane group kg = lane / 16 carries columns
// 8 kg + s' at MFMA step s' (the contraction order is free), so each lane reads
// 64 contiguous bytes per row. Wave w computes output rows 16 w .. + 15 against
// all eight 16-column tiles.
__global__ __launch_bounds__(GR_NT, 1) void k_lap_gram(const LapArgs a) {
  __shared__ __attribute__((aligned(16))) double blk[2][HD][GR_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.x, half = blockIdx.y;
  const int l = u / a.n_kv, h = u % a.n_kv;
  const int D = a.D, Dh = D / GR_KS, nblk = Dh / GR_KB;
  const uint16_t *wo = reinterpret_cast<const uint16_t *>(a.wo);
  // staging task: row tid / 4, columns 8 (tid % 4) .. + 7 of the block
  const int srow = tid >> 2, scol = (tid & 3) * 8;
  u32x4 raw[8];   // the group's G 16-byte vectors (G <= 8)
  auto fetch = [&](int b) {
    const int col = half * Dh + b * GR_KB + scol;
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (g < a.G) {
        const int64_t head = int64_t(l) * a.H + h * a.G + g;
        raw[g] = ld16(wo + (head * HD + srow) * D + col);
      }
  };
  auto stage = [&](int buf) {
    double sum[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sum[e] = 0.0;
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (g < a.G)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] += double(ElemTraits<bf16_t>::get(raw[g], e));
#pragma unroll
    for (int e = 0; e < 8; e += 2) *reinterpret_cast<fm_d2 *>(&blk[buf][srow][scol + e]) = fm_d2{sum[e], sum[e + 1]};
  };
  fm_d4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = fm_d4{0.0, 0.0, 0.0, 0.0};
  const int m = lane & 15, kg = lane >> 4;
  fetch(0);
  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    stage(buf);
    __syncthreads();
    if (b + 1 < nblk) fetch(b + 1);
    const double *arow = &blk[buf][16 * wave + m][8 * kg];
#pragma unroll
    for (int sh = 0; sh < 2; ++sh) {          // steps 4 sh .. 4 sh + 3
      const fm_d2 a0 = *reinterpret_cast<const fm_d2 *>(arow + 4 * sh);
      const fm_d2 a1 = *reinterpret_cast<const fm_d2 *>(arow + 4 * sh + 2);
      fm_d2 bq[8][2];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const double *brow = &blk[buf][16 * ct + m][8 * kg + 4 * sh];
        bq[ct][0] = *reinterpret_cast<const fm_d2 *>(brow);
        bq[ct][1] = *reinterpret_cast<const fm_d2 *>(brow + 2);
      }
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0.x, bq[ct][0].x, acc[ct], 0, 0, 0);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0.y, bq[ct][0].y, acc[ct], 0, 0, 0);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1.x, bq[ct][1].x, acc[ct], 0, 0, 0);
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1.y, bq[ct][1].y, acc[ct], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // D[16 wave + kg + 4 r][16 ct + m]
  double *out = a.gram + (int64_t(u) * GR_KS + half) * HD * HD;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(16 * wave + kg + 4 * r) * HD + 16 * ct + m] = acc[ct][r];
}

// ---------------------------------------------------------------- window passes
__device__ __forceinline__ float dpp_f32_stage(float x, int s) {
  int v = __float_as_int(x);
  switch (s) {
    case 0: v = __builtin_amdgcn_mov_dpp(v, 0xB1, 0xf, 0xf, true); break;    // lane ^ 1
    case 1: v = __builtin_amdgcn_mov_dpp(v, 0x4E, 0xf, 0xf, true); break;    // lane ^ 2
    case 2: v = __builtin_amdgcn_mov_dpp(v, 0x141, 0xf, 0xf, true); break;   // 7 - lane in 8
    default: v = __builtin_amdgcn_mov_dpp(v, 0x140, 0xf, 0xf, true); break;  // 15 - lane in 16
  }
  return __int_as_float(v);
}

// Sum over aligned blocks of 2^(S1) lanes, applying stages [S0, S1).
template <int S0, int S1>
__device__ __forceinline__ float block_sum(float x) {
#pragma unroll
  for (int s = S0; s < S1; ++s) x += dpp_f32_stage(x, s);
  return x;
}

template <int G>
__device__ __forceinline__ constexpr int ilog2c() { return G >= 8 ? 3 : G >= 4 ? 2 : G >= 2 ? 1 : 0; }

// Window passes on the float64 MFMA, transposed: tau Q (a block of window rows
// x d) is the operator in LDS as B fragments and 16 keys at a time are the A
// operand, so lane l ends with the logits of operator rows 16 ct + l % 16
// (ct = 0..7) for tokens l / 16 + 4 r (r = 0..3) of the tile. The operator rows
// are head-major: row 16 ct + jl holds head g = ct / (8 / G) of window row
// jj = hb 128 / G + (ct % (8 / G)) 16 + jl, so the G heads of a window row sit
// in one lane and the group mean is an in-lane sum.
// grid (ntiles, nh, units), 512 threads, wave w takes tiles w, w + 8, ...
//   PASS 1: per row, the running max and sum of e^{l - max} over the lane's
//           tokens (plain fp32 exp of the float64 difference, summed per tile
//           in fp32 and across tiles in float64); combined over the lane groups
//           and waves -> one partial per (row, workgroup).
//   PASS 2: A = e^{l - M} / Z (split exp), the mean over the G heads, its square
//           summed over the block's window rows -> c^2 per token.
// Window rows past w have a zero operator row and are masked; tiles wholly
// before the causal window and inside the chunk skip the per-logit mask.
template <int G>
__device__ __forceinline__ int win_row(int hb, int ct, int jl, int *jj) {
  constexpr int CPG = 8 / G;          // column tiles per head
  const int g = ct / CPG;
  *jj = hb * (128 / G) + (ct % CPG) * 16 + jl;
  return g;
}

template <int G, int PASS>
__global__ __launch_bounds__(WM_NT, 1) void k_lap_window(const LapArgs a) {
  __shared__ FmOperator qop;
  __shared__ double redm[WM_NT / 64][128], redz[WM_NT / 64][128];
  constexpr int CPG = 8 / G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x, hb = blockIdx.y, u = blockIdx.z;
  const int l = u / a.n_kv, h = u % a.n_kv;
  const int N = a.N, w = a.w, R = a.R;
  const int t0 = tile * WM_TILE, t1 = min(N, t0 + WM_TILE);
  {
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(a.q);
    for (int e = tid; e < HD * HD; e += WM_NT) {
      const int r = e >> 7, b = e & 127;
      int jj;
      const int g = win_row<G>(hb, r >> 4, r & 15, &jj);
      double v = 0.0;
      if (jj < w) {
        const int64_t head = int64_t(l) * a.H + h * G + g;
        v = double(bf16_to_f32(qb[(head * w + jj) * HD + b])) * a.scale;
      }
      fm_put_t(qop, r, b, v);
    }
  }
  const int jl = lane & 15, tq = lane >> 4;
  float gam[CPG];          // EMA weight of each of the lane's window rows (0 past the window)
#pragma unroll
  for (int c8 = 0; c8 < CPG; ++c8) {
    const int jj = hb * (128 / G) + c8 * 16 + jl;
    gam[c8] = (a.ema && jj < w) ? float((1.0 - a.alpha) * pow(a.alpha, double(w - 1 - jj))) : 0.f;
  }
  int plim[FM_RT];         // last key each of the lane's rows attends to (-1: not a row)
  double Mrow[FM_RT], Zrow[FM_RT];
  float iz[FM_RT];
#pragma unroll
  for (int ct = 0; ct < FM_RT; ++ct) {
    int jj;
    const int g = win_row<G>(hb, ct, jl, &jj);
    const int row = jj * G + g;
    plim[ct] = jj < w ? N - w + jj : -1;
    if (PASS == 1) {
      Mrow[ct] = -INFINITY;
      Zrow[ct] = 0.0;
    } else {
      Mrow[ct] = jj < w ? a.rM[int64_t(u) * R + row] : 0.0;
      const double Z = jj < w ? a.rZ[int64_t(u) * R + row] : 0.0;
      iz[ct] = Z > 0.0 ? float(1.0 / Z) : 0.f;
    }
  }
  __syncthreads();

  const char *Kb = a.k + int64_t(u) * a.kstride * RB;
  const int n16 = (t1 - t0 + FM_TILE - 1) / FM_TILE;
  for (int t = wave; t < n16; t += WM_NT / 64) {
    const int tb = t0 + t * FM_TILE;
    FmRow<bf16_t> kr;
    kr.load(Kb + int64_t(min(tb + jl, t1 - 1)) * RB + 64 * tq);
    double x[32];
#pragma unroll
    for (int s = 0; s < 32; ++s) x[s] = kr.get(s);
    fm_d4 acc[FM_RT];
#pragma unroll
    for (int ct = 0; ct < FM_RT; ++ct) acc[ct] = fm_d4{0.0, 0.0, 0.0, 0.0};
    fm_apply_t(qop, lane, x, acc);
    // every token of the tile is inside the chunk and before the first window row
    const bool whole = tb + FM_TILE <= t1 && tb + FM_TILE - 1 <= N - w;
    if (!whole) {
#pragma unroll
      for (int ct = 0; ct < FM_RT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tok = tb + tq + 4 * r;
          if (!(tok < t1 && tok <= plim[ct])) acc[ct][r] = -INFINITY;
        }
    }
    if (PASS == 1) {
#pragma unroll
      for (int ct = 0; ct < FM_RT; ++ct) {
        const double mx = fmax(fmax(acc[ct][0], acc[ct][1]), fmax(acc[ct][2], acc[ct][3]));
        if (mx > Mrow[ct]) {
          if (Mrow[ct] > -INFINITY) Zrow[ct] *= exp(Mrow[ct] - mx);
          Mrow[ct] = mx;
        }
        if (Mrow[ct] > -INFINITY) {
          float z = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) z += expf(float(acc[ct][r] - Mrow[ct]));
          Zrow[ct] += double(z);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tok = tb + tq + 4 * r;
        float sq = 0.f;
#pragma unroll
        for (int c8 = 0; c8 < CPG; ++c8) {
          float sum = 0.f;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const int ct = g * CPG + c8;
            sum += exp_split(acc[ct][r] - Mrow[ct]) * iz[ct];
          }
          const float mean = sum * (1.f / float(G));
          sq += a.ema ? gam[c8] * mean : mean * mean;
        }
        // the 16 lanes of a row of lanes hold 16 window rows each
        const float c2 = block_sum<0, 4>(sq);
        if (jl == 0 && tok < t1) a.c2[(int64_t(u) * a.nh + hb) * N + tok] = c2;
      }
    }
  }

  if (PASS == 1) {
    // operator rows 16 ct + jl: combine the four token groups of the wave, then the waves
#pragma unroll
    for (int ct = 0; ct < FM_RT; ++ct) {
#pragma unroll
      for (int o = 16; o < 64; o <<= 1) {
        const double M2 = __shfl_xor(Mrow[ct], o), Z2 = __shfl_xor(Zrow[ct], o);
        const double Mn = fmax(Mrow[ct], M2);
        double Z = 0.0;
        if (Mrow[ct] > -INFINITY) Z += Zrow[ct] * exp(Mrow[ct] - Mn);
        if (M2 > -INFINITY) Z += Z2 * exp(M2 - Mn);
        Mrow[ct] = Mn;
        Zrow[ct] = Z;
      }
      if (tq == 0) {
        redm[wave][16 * ct + jl] = Mrow[ct];
        redz[wave][16 * ct + jl] = Zrow[ct];
      }
    }
    __syncthreads();
    if (tid < 128) {
      int jj;
      const int g = win_row<G>(hb, tid >> 4, tid & 15, &jj);
      if (jj < w) {
        double M = -INFINITY;
#pragma unroll
        for (int wv = 0; wv < WM_NT / 64; ++wv) M = fmax(M, redm[wv][tid]);
        double Z = 0.0;
#pragma unroll
        for (int wv = 0; wv < WM_NT / 64; ++wv)
          if (redm[wv][tid] > -INFINITY) Z += redz[wv][tid] * exp(redm[wv][tid] - M);
        const int64_t o = (int64_t(u) * R + jj * G + g) * a.ntiles + tile;
        a.tM[o] = M;
        a.tZ[o] = Z;
      }
    }
  }
}

// grid (ceil(N / 256), units): the EMA utility of each token, summed over the window-row blocks.
__global__ __launch_bounds__(256) void k_ema_fin(const LapArgs a) {
  const int tok = blockIdx.x * 256 + threadIdx.x, u = blockIdx.y;
  if (tok >= a.N) return;
  float m = 0.f;
  for (int hb = 0; hb < a.nh; ++hb) m += a.c2[(int64_t(u) * a.nh + hb) * a.N + tok];
  a.m_out[int64_t(u) * a.m_stride + tok] = m;
}

// grid (ceil(units R / 256)), 256 threads: each thread combines one row's tiles in order.
__global__ __launch_bounds__(256) void k_lap_rowfin(const LapArgs a, int n_rows) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= n_rows) return;
  const double *pm = a.tM + int64_t(r) * a.ntiles, *pz = a.tZ + int64_t(r) * a.ntiles;
  double M = -INFINITY;
  for (int t = 0; t < a.ntiles; ++t) M = fmax(M, pm[t]);
  double Z = 0.0;
  for (int t = 0; t < a.ntiles; ++t)
    if (pm[t] > -INFINITY) Z += pz[t] * exp(pm[t] - M);
  a.rM[r] = M;
  a.rZ[r] = Z;
}

// ---------------------------------------------------------------- r^2 = v M v^T on float64 MFMA
// grid (ceil(N / R2_TOK), units), 512 threads. M (the sum of the two Gram
// halves) is staged as the float64 MFMA operator; wave w takes the 16-token
// tiles w, w + 8, ... of the workgroup's range. A lane's B values are elements
// [32 g, 32 g + 32) of its token's value row, and its accumulator rows are
// the same elements of M v, so r^2 = sum over its 32 products, then over g.
__global__ __launch_bounds__(R2_NT, 1) void k_lap_r2(const LapArgs a) {
  __shared__ FmOperator op;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.y, N = a.N;
  const int t0 = blockIdx.x * R2_TOK, t1 = min(N, t0 + R2_TOK);
  {
    const double *M0 = a.gram + int64_t(u) * GR_KS * HD * HD;
    for (int e = tid; e < HD * HD; e += R2_NT) {
      double m = 0.0;
#pragma unroll
      for (int k = 0; k < GR_KS; ++k) m += M0[k * HD * HD + e];
      fm_put(op, e >> 7, e & 127, m);
    }
  }
  __syncthreads();
  const int g = lane >> 4, jl = lane & 15;
  const char *Vb = a.v + int64_t(u) * N * RB;
  const int n_tiles = (t1 - t0 + FM_TILE - 1) / FM_TILE;
  for (int tile = wave; tile < n_tiles; tile += R2_NT / 64) {
    const int j = t0 + tile * FM_TILE + jl;
    FmRow<bf16_t> vr;
    vr.load(Vb + int64_t(min(j, t1 - 1)) * RB + 64 * g);
    double x[32];
#pragma unroll
    for (int s = 0; s < 32; ++s) x[s] = vr.get(s);
    fm_d4 acc[FM_RT];
#pragma unroll
    for (int rt = 0; rt < FM_RT; ++rt) acc[rt] = fm_d4{0.0, 0.0, 0.0, 0.0};
    fm_apply(op, lane, x, acc);
    double r2 = 0.0;
#pragma unroll
    for (int rt = 0; rt < FM_RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) r2 = fma(x[4 * rt + r], acc[rt][r], r2);
    r2 += __shfl_xor(r2, 16);
    r2 += __shfl_xor(r2, 32);
    if (g == 0 && j < t1) a.r2[int64_t(u) * N + j] = float(r2);
  }
}

// ---------------------------------------------------------------- product and normalisation
// grid (nchunks, units), 256 threads: p = c r into score, chunk sums of p.
__global__ __launch_bounds__(256) void k_lap_p(const LapArgs a) {
  __shared__ double red[4];
  const int ch = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int N = a.N;
  const int i0 = ch * P_CHUNK, i1 = min(N, i0 + P_CHUNK);
  double s = 0.0;
  for (int i = i0 + tid; i < i1; i += 256) {
    double c2 = 0.0;
    for (int hf = 0; hf < a.nh; ++hf) c2 += double(a.c2[(int64_t(u) * a.nh + hf) * N + i]);
    const double p = sqrt(c2) * sqrt(double(a.r2[int64_t(u) * N + i]));
    a.score[int64_t(u) * N + i] = float(p);
    s += p;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((tid & 63) == 0) red[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) a.psum[int64_t(u) * a.nchunks + ch] = (red[0] + red[1]) + (red[2] + red[3]);
}

// grid (nchunks, units), 256 threads: layer sum (fixed order) and score = p / sum.
__global__ __launch_bounds__(256) void k_lap_norm(const LapArgs a) {
  __shared__ double sig;
  const int ch = blockIdx.x, u = blockIdx.y, tid = threadIdx.x;
  const int l = u / a.n_kv;
  if (tid == 0) {
    double s = 0.0;
    for (int h = 0; h < a.n_kv; ++h)
      for (int c = 0; c < a.nchunks; ++c) s += a.psum[(int64_t(l) * a.n_kv + h) * a.nchunks + c];
    sig = s;
  }
  __syncthreads();
  const double inv = sig > 0.0 ? 1.0 / sig : 0.0;
  const int N = a.N;
  const int i0 = ch * P_CHUNK, i1 = min(N, i0 + P_CHUNK);
  // score holds p rounded to float; recompute p in float64 for the quotient
  for (int i = i0 + tid; i < i1; i += 256) {
    double c2 = 0.0;
    for (int hf = 0; hf < a.nh; ++hf) c2 += double(a.c2[(int64_t(u) * a.nh + hf) * N + i]);
    const double p = sqrt(c2) * sqrt(double(a.r2[int64_t(u) * N + i]));
    a.score[int64_t(u) * N + i] = float(p * inv);
  }
}

struct LapLayout {
  size_t gram, tM, tZ, rM, rZ, c2, r2, psum, total;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

LapLayout lap_layout(int n_layers, int H, int n_kv, int N, int w, int D) {
  const int64_t units = int64_t(n_layers) * n_kv;
  const int G = H / n_kv, R = G * w;
  const int nh = (w + WM_ROWS / G - 1) / (WM_ROWS / G), ntiles = (N + WM_TILE - 1) / WM_TILE, nchunks = (N + P_CHUNK - 1) / P_CHUNK;
  LapLayout L{};
  size_t o = 0;
  L.gram = o;  o = align256(o + size_t(units) * GR_KS * HD * HD * 8);
  L.tM = o;    o = align256(o + size_t(units) * R * ntiles * 8);
  L.tZ = o;    o = align256(o + size_t(units) * R * ntiles * 8);
  L.rM = o;    o = align256(o + size_t(units) * R * 8);
  L.rZ = o;    o = align256(o + size_t(units) * R * 8);
  L.c2 = o;    o = align256(o + size_t(units) * nh * N * 4);
  L.r2 = o;    o = align256(o + size_t(units) * N * 4);
  L.psum = o;  o = align256(o + size_t(units) * nchunks * 8);
  L.total = o;
  return L;
}

template <int G>
hipError_t launch_window(const LapArgs &a, dim3 grid, hipStream_t st, int pass) {
  if (pass == 1) hipLaunchKernelGGL((k_lap_window<G, 1>), grid, dim3(WM_NT), 0, st, a);
  else hipLaunchKernelGGL((k_lap_window<G, 2>), grid, dim3(WM_NT), 0, st, a);
  return hipGetLastError();
}

hipError_t window_pass(const LapArgs &a, dim3 grid, hipStream_t st, int pass) {
  switch (a.G) {
    case 1: return launch_window<1>(a, grid, st, pass);
    case 2: return launch_window<2>(a, grid, st, pass);
    case 4: return launch_window<4>(a, grid, st, pass);
    case 8: return launch_window<8>(a, grid, st, pass);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool laprox_shape_supported(int H, int n_kv, int N, int w, int D) {
  if (n_kv <= 0 || H % n_kv != 0) return false;
  const int G = H / n_kv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return false;
  return N > 0 && w > 0 && w <= N && (G * w) % RPW == 0 && D > 0 && D % 64 == 0;
}

size_t laprox_workspace_bytes(int n_layers, int H, int n_kv, int N, int w, int /*d*/, int D) {
  if (!laprox_shape_supported(H, n_kv, N, w, D) || n_layers <= 0) return 0;
  return lap_layout(n_layers, H, n_kv, N, w, D).total;
}

hipError_t launch_laprox(const void *q_win, const void *k, const void *v, const void *w_o, int n_layers,
                         int H, int n_kv, int N, int w, int D, double scale, float *score, void *ws,
                         hipStream_t st, hipEvent_t *marks) {
  const LapLayout L = lap_layout(n_layers, H, n_kv, N, w, D);
  char *base = static_cast<char *>(ws);
  LapArgs a{};
  a.q = static_cast<const char *>(q_win);
  a.k = static_cast<const char *>(k);
  a.v = static_cast<const char *>(v);
  a.wo = static_cast<const char *>(w_o);
  a.n_layers = n_layers;
  a.H = H;
  a.n_kv = n_kv;
  a.N = N;
  a.w = w;
  a.D = D;
  a.G = H / n_kv;
  a.R = a.G * w;
  a.nh = (w + WM_ROWS / a.G - 1) / (WM_ROWS / a.G);
  a.ntiles = (N + WM_TILE - 1) / WM_TILE;
  a.nchunks = (N + P_CHUNK - 1) / P_CHUNK;
  a.scale = scale;
  a.score = score;
  a.gram = reinterpret_cast<double *>(base + L.gram);
  a.tM = reinterpret_cast<double *>(base + L.tM);
  a.tZ = reinterpret_cast<double *>(base + L.tZ);
  a.rM = reinterpret_cast<double *>(base + L.rM);
  a.rZ = reinterpret_cast<double *>(base + L.rZ);
  a.c2 = reinterpret_cast<float *>(base + L.c2);
  a.r2 = reinterpret_cast<float *>(base + L.r2);
  a.psum = reinterpret_cast<double *>(base + L.psum);
  a.kstride = N;
  const int units = n_layers * n_kv;

  // marks (optional): an event before the first kernel and after each of the seven
  auto mark = [&](int i) { return marks ? hipEventRecord(marks[i], st) : hipSuccess; };
  hipError_t e = mark(0);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lap_gram, dim3(units, GR_KS), dim3(GR_NT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(1)) != hipSuccess) return e;
  const dim3 wgrid(a.ntiles, a.nh, units);
  if ((e = window_pass(a, wgrid, st, 1)) != hipSuccess || (e = mark(2)) != hipSuccess) return e;
  const int n_rows = units * a.R;
  hipLaunchKernelGGL(k_lap_rowfin, dim3((n_rows + 255) / 256), dim3(256), 0, st, a, n_rows);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(3)) != hipSuccess) return e;
  if ((e = window_pass(a, wgrid, st, 2)) != hipSuccess || (e = mark(4)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_lap_r2, dim3((N + R2_TOK - 1) / R2_TOK, units), dim3(R2_NT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(5)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_lap_p, dim3(a.nchunks, units), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(6)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_lap_norm, dim3(a.nchunks, units), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(7);
}

struct EmaLayout {
  size_t tM, tZ, rM, rZ, c2, total;
};

EmaLayout ema_layout(int units, int G, int N, int w) {
  const int R = G * w, nh = (w + WM_ROWS / G - 1) / (WM_ROWS / G), ntiles = (N + WM_TILE - 1) / WM_TILE;
  EmaLayout L{};
  size_t o = 0;
  L.tM = o;  o = align256(o + size_t(units) * R * ntiles * 8);
  L.tZ = o;  o = align256(o + size_t(units) * R * ntiles * 8);
  L.rM = o;  o = align256(o + size_t(units) * R * 8);
  L.rZ = o;  o = align256(o + size_t(units) * R * 8);
  L.c2 = o;  o = align256(o + size_t(units) * nh * N * 4);
  L.total = o;
  return L;
}

size_t ema_window_workspace_bytes(int units, int G, int N, int w) { return ema_layout(units, G, N, w).total; }

hipError_t launch_ema_window(const void *q_win, const void *k, int64_t kstride, int units, int G, int w, int N,
                             double scale, double alpha, float *m, int64_t m_stride, void *ws, hipStream_t st,
                             hipEvent_t *marks) {
  const EmaLayout L = ema_layout(units, G, N, w);
  char *base = static_cast<char *>(ws);
  LapArgs a{};
  a.q = static_cast<const char *>(q_win);
  a.k = static_cast<const char *>(k);
  a.n_layers = units;
  a.H = G;
  a.n_kv = 1;
  a.N = N;
  a.w = w;
  a.G = G;
  a.R = G * w;
  a.nh = (w + WM_ROWS / G - 1) / (WM_ROWS / G);
  a.ntiles = (N + WM_TILE - 1) / WM_TILE;
  a.scale = scale;
  a.tM = reinterpret_cast<double *>(base + L.tM);
  a.tZ = reinterpret_cast<double *>(base + L.tZ);
  a.rM = reinterpret_cast<double *>(base + L.rM);
  a.rZ = reinterpret_cast<double *>(base + L.rZ);
  a.c2 = reinterpret_cast<float *>(base + L.c2);
  a.kstride = kstride;
  a.ema = 1;
  a.alpha = alpha;
  a.m_out = m;
  a.m_stride = m_stride;
  auto mark = [&](int i) { return marks ? hipEventRecord(marks[i], st) : hipSuccess; };
  hipError_t e = mark(0);
  if (e != hipSuccess) return e;
  const dim3 wgrid(a.ntiles, a.nh, units);
  if ((e = window_pass(a, wgrid, st, 1)) != hipSuccess || (e = mark(1)) != hipSuccess) return e;
  const int n_rows = units * a.R;
  hipLaunchKernelGGL(k_lap_rowfin, dim3((n_rows + 255) / 256), dim3(256), 0, st, a, n_rows);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(2)) != hipSuccess) return e;
  if ((e = window_pass(a, wgrid, st, 2)) != hipSuccess || (e = mark(3)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_ema_fin, dim3((N + 255) / 256, units), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(4);
}

}  // namespace kvc
