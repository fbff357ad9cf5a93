// LaProx prefill scoring (notes on "Reformulating KV Cache Eviction Problem
// for Long-Context LLM Inference": key design 1, the indicator
// ||A[:, i]||_2 ||(V W_O)[i, :]||_2; key design 2, per-layer normalisation;
// the GQA paragraph, group-averaged attention of the last w queries).
//
// Per unit (layer l, KV head h) with G query heads and w window queries, the
// R = G w window rows (g, j) attend causally: row j sits at position
// N - w + j. Kernels, in launch order:
//   k_lap_wprep    W_bar = sum of the group's W_O^g blocks, summed in float64
//                  and split into bf16 hi + lo (residual below 2^-17 of each
//                  element), stored transposed [D][d] for the MFMA B operand.
//   k_lap_window<1> per token tile: float64 logits of 8 rows per wave
//                  (lane-permuted transposed reduction), per-row running max
//                  and sum of exp -> partials per tile.
//   k_lap_rowfin   combines the tile partials of every row (fixed order).
//   k_lap_window<2> recomputes the logits; A = exp(l - M) / Z; the group mean
//                  over the G heads of each window row by DPP sums; its square
//                  summed over the rows of the workgroup -> c^2 partials.
//   k_lap_vw       r_i^2 = ||v_i W_bar||^2 on MFMA (16x16x32 bf16, fp32
//                  accumulate; hi and lo both accumulate into the same tile),
//                  squares summed in float64; B tiles staged in LDS.
//   k_lap_p        p_i = c_i r_i (float64) and per-chunk partial sums.
//   k_lap_norm     per-layer sum in fixed order, score = p / sum.
// The model-wide Top-K (key design 3) is kvc_select_evict over the scores.
#include "kvc_device.h"
#include "kvc_laprox.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- geometry
constexpr int LW = 8;               // waves per window workgroup
constexpr int LNT = 64 * LW;        // window workgroup threads
constexpr int RPW = 8;              // window rows per wave
constexpr int RPG = LW * RPW;       // window rows per workgroup (64)
constexpr int TILE = 1024;          // tokens per window workgroup
constexpr int LLPT = 16;            // lanes per bf16 row (8 elements each)
constexpr int LTPI = 4;             // tokens per wave iteration
constexpr int LUNR = 4;             // iterations per sub-chunk (16 tokens)
constexpr int LCH = LTPI * LUNR;
constexpr int LPF = 2;              // sub-chunks of loads in flight
constexpr int RB = HD * 2;          // bytes per bf16 row

constexpr int VW_WAVES = 8;         // V W_bar workgroup: 8 waves x 64 tokens
constexpr int VW_NT = 64 * VW_WAVES;
constexpr int VW_MB = 4;            // 16-token M blocks per wave
constexpr int VW_TOK = VW_WAVES * VW_MB * 16;   // tokens per workgroup (512)
constexpr int VW_NS = 32;           // columns per LDS stage of W_bar^T
constexpr int VW_LDS_ROW = HD + 8;  // bf16 per LDS row of a B block (padded)

constexpr int P_CHUNK = 4096;       // tokens per partial sum of p

struct LapArgs {
  const char *q, *k, *v, *wo;
  int n_layers, H, n_kv, N, w, D, G, R, nh, ntiles, nchunks;
  double scale;
  float *score;
  uint16_t *wt_hi, *wt_lo;    // [units][D][d]
  double *tM, *tZ;            // [units][R][ntiles]
  double *rM, *rZ;            // [units][R]
  float *c2;                  // [units][nh][N]
  float *r2;                  // [units][N]
  double *psum;               // [units][nchunks]
};

// ---------------------------------------------------------------- W_bar
// grid (D / 64, d / 64, units), 256 threads: a 64 x 64 tile of W_bar, summed
// over the group in float64, split hi/lo and written transposed.
__global__ __launch_bounds__(256) void k_lap_wprep(const LapArgs a) {
  __shared__ float hi_t[64][65], lo_t[64][65];
  const int n0 = blockIdx.x * 64, r0 = blockIdx.y * 64, u = blockIdx.z;
  const int l = u / a.n_kv, h = u % a.n_kv;
  const int tid = threadIdx.x;
  const uint16_t *wo = reinterpret_cast<const uint16_t *>(a.wo);
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int rr = idx / 64, nn = idx % 64;   // W row (d index) rr, column nn: coalesced over nn
    double s = 0.0;
    for (int g = 0; g < a.G; ++g) {
      const int64_t head = int64_t(l) * a.H + h * a.G + g;
      s += double(bf16_to_f32(wo[(head * HD + r0 + rr) * a.D + n0 + nn]));
    }
    const uint16_t hb = f32_to_bf16(float(s));
    const double hv = double(bf16_to_f32(hb));
    const uint16_t lb = f32_to_bf16(float(s - hv));
    hi_t[rr][nn] = __uint_as_float(uint32_t(hb));
    lo_t[rr][nn] = __uint_as_float(uint32_t(lb));
  }
  __syncthreads();
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int nn = idx / 64, rr = idx % 64;   // transposed: coalesced over rr
    const int64_t o = (int64_t(u) * a.D + n0 + nn) * HD + r0 + rr;
    a.wt_hi[o] = uint16_t(__float_as_uint(hi_t[rr][nn]));
    a.wt_lo[o] = uint16_t(__float_as_uint(lo_t[rr][nn]));
  }
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

// PASS 1: row max / sum partials per tile. PASS 2: c^2 partials per token.
// grid (ntiles, nh, units), 512 threads. Wave w of workgroup half `hf` owns
// rows 64 hf + 8 w .. + 7 (row = j G + g); lanes hold them in the permuted
// order of preduce and end with row perm_head(lane % 16).
template <int G, int PASS>
__global__ __launch_bounds__(LNT, 1) void k_lap_window(const LapArgs a) {
  __shared__ float part[LW][TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = blockIdx.x, hf = blockIdx.y, u = blockIdx.z;
  const int l = u / a.n_kv, h = u % a.n_kv;
  const int N = a.N, w = a.w;
  const int row0 = hf * RPG + wave * RPW;
  const bool active = row0 < a.R;      // R is a multiple of 8: a wave is all in or all out
  const int cb = lane & (LLPT - 1), tg = lane >> 4;
  const int myr = perm_head<LLPT, RPW>(cb);
  const int rl = row0 + myr;           // the lane's reduced row
  const int jl = rl / G;
  const int plim = N - w + jl;         // last key the lane's row attends to
  const int t0 = tile * TILE, t1 = min(N, t0 + TILE);

  double qf[RPW][8];
  {
    const uint16_t *qb = reinterpret_cast<const uint16_t *>(a.q);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int row = active ? row0 + (i ^ myr) : 0;
      const int j = row / G, g = row - (row / G) * G;
      const int64_t head = int64_t(l) * a.H + h * G + g;
      const uint16_t *qr = qb + (head * w + j) * HD + cb * 8;
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[i][e] = double(bf16_to_f32(qr[e])) * a.scale;
    }
  }
  double Mr = 0.0;
  float izr = 0.f;
  if (PASS == 2 && active) {
    Mr = a.rM[int64_t(u) * a.R + rl];
    const double Z = a.rZ[int64_t(u) * a.R + rl];
    izr = Z > 0.0 ? float(1.0 / Z) : 0.f;
  }
  double Mrun = -INFINITY, Zrun = 0.0;
  const int dup = lane & 1;

  const char *Kb = a.k + int64_t(u) * N * RB;
  const int nsub = (t1 - t0 + LCH - 1) / LCH;
  u32x4 kr[LPF][LUNR];
  auto issue = [&](u32x4 (&r)[LUNR], int c) {
#pragma unroll
    for (int it = 0; it < LUNR; ++it) {
      const int tok = min(t0 + c * LCH + it * LTPI + tg, N - 1);
      r[it] = ld16(Kb + int64_t(tok) * RB + 16 * cb);
    }
  };
  if (active) {
#pragma unroll
    for (int s = 0; s < LPF; ++s) issue(kr[s], s);
  }
  for (int base = 0; active && base < nsub; base += LPF) {
#pragma unroll
    for (int s = 0; s < LPF; ++s) {
      const int c = base + s;
      if (c < nsub) {
        double lg[LUNR];
#pragma unroll
        for (int it = 0; it < LUNR; ++it) {
          double acc[RPW];
#pragma unroll
          for (int i = 0; i < RPW; ++i) acc[i] = 0.0;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double ke = double(ElemTraits<bf16_t>::get(kr[s][it], e));
#pragma unroll
            for (int i = 0; i < RPW; ++i) acc[i] = fma(qf[i][e], ke, acc[i]);
          }
          lg[it] = preduce<LLPT, RPW, 0>(acc);
          const int tok = t0 + c * LCH + it * LTPI + tg;
          if (tok >= t1 || tok > plim) lg[it] = -INFINITY;
        }
        if (PASS == 1) {
          // lane `dup` takes iterations dup and dup + 2 of its row
          const double xa = lg[dup], xb = lg[dup + 2];
          const double Mn = fmax(Mrun, fmax(xa, xb));
          if (Mn > Mrun) {
            if (Mrun > -INFINITY) Zrun *= exp(Mrun - Mn);
            Mrun = Mn;
          }
          Zrun += double(exp_split(xa - Mrun)) + double(exp_split(xb - Mrun));
        } else {
#pragma unroll
          for (int it = 0; it < LUNR; ++it) {
            const float A = exp_split(lg[it] - Mr) * izr;
            // mean over the G heads of the window row: blocks of 2G lanes, each head twice
            const float ab = block_sum<0, ilog2c<G>() + 1>(A) * (1.f / float(2 * G));
            const float sq = block_sum<ilog2c<G>() + 1, 4>(ab * ab) * (1.f / float(2 * G));
            if (cb == 0) part[wave][c * LCH + it * LTPI + tg] = sq;
          }
        }
      }
      issue(kr[s], base + s + LPF);
    }
  }

  if (PASS == 1) {
    // combine the lanes of each row: dup pair and the four token groups
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      if (o != 1 && o != 16 && o != 32) continue;
      const double M2 = __shfl_xor(Mrun, o), Z2 = __shfl_xor(Zrun, o);
      const double Mn = fmax(Mrun, M2);
      double Z = 0.0;
      if (Mrun > -INFINITY) Z += Zrun * exp(Mrun - Mn);
      if (M2 > -INFINITY) Z += Z2 * exp(M2 - Mn);
      Mrun = Mn;
      Zrun = Z;
    }
    if (active && tg == 0 && dup == 0) {
      const int64_t o = (int64_t(u) * a.R + rl) * a.ntiles + tile;
      a.tM[o] = Mrun;
      a.tZ[o] = Zrun;
    }
  } else {
    __syncthreads();
    const int nt = t1 - t0;
    for (int t = tid; t < nt; t += LNT) {
      double s = 0.0;
#pragma unroll
      for (int wv = 0; wv < LW; ++wv)
        if (hf * RPG + wv * RPW < a.R) s += double(part[wv][t]);
      a.c2[(int64_t(u) * a.nh + hf) * N + t0 + t] = float(s);
    }
  }
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

// ---------------------------------------------------------------- V W_bar on MFMA
// grid (ceil(N / 512), units), 512 threads. Wave w holds the A fragments (V
// rows) of tokens t0 + 64 w + 16 mb + (lane % 16), d elements 32 ks + 8 (lane / 16) ..
// + 7. W_bar^T (hi and lo) is staged through LDS in stages of 32 columns
// ([hi/lo][column][d], rows padded against bank conflicts), double-buffered,
// with each thread's two 16-byte vectors of a stage loaded three stages
// ahead; one barrier per stage.
__global__ __launch_bounds__(VW_NT, 1) void k_lap_vw(const LapArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t bt[2][2][VW_NS][VW_LDS_ROW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int u = blockIdx.y;
  const int N = a.N, D = a.D;
  const int t0 = blockIdx.x * VW_TOK + wave * (VW_MB * 16);
  const int m = lane & 15, kq = lane >> 4;

  bf16x8 av[VW_MB][4];
  {
    const char *Vb = a.v + int64_t(u) * N * RB;
#pragma unroll
    for (int mb = 0; mb < VW_MB; ++mb) {
      const int tok = min(t0 + 16 * mb + m, N - 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 x = ld16(Vb + int64_t(tok) * RB + (32 * ks + 8 * kq) * 2);
        av[mb][ks] = __builtin_bit_cast(bf16x8, x);
      }
    }
  }
  // the two B vectors this thread stages per stage: the hi and the lo vector of
  // column tid / 16 of the stage, d elements 8 (tid % 16) .. + 7
  const int nn = (tid >> 4) & 31, ee = tid & 15;
  const uint16_t *src_hi = a.wt_hi + int64_t(u) * D * HD + ee * 8;
  const uint16_t *src_lo = a.wt_lo + int64_t(u) * D * HD + ee * 8;
  const int nst = D / VW_NS;
  constexpr int PD = 3;                  // stages of loads in flight
  u32x4 sreg[PD][2];
  auto load_stage = [&](u32x4 (&r)[2], int st) {
    const int col = min(st, nst - 1) * VW_NS + nn;
    r[0] = ld16(src_hi + int64_t(col) * HD);
    r[1] = ld16(src_lo + int64_t(col) * HD);
  };
  auto store_stage = [&](const u32x4 (&r)[2], int buf) {
    *reinterpret_cast<u32x4 *>(&bt[buf][0][nn][ee * 8]) = r[0];
    *reinterpret_cast<u32x4 *>(&bt[buf][1][nn][ee * 8]) = r[1];
  };
#pragma unroll
  for (int p = 0; p < PD; ++p) load_stage(sreg[p], p);
  store_stage(sreg[0], 0);
  load_stage(sreg[0], PD);
  __syncthreads();

  double rs[VW_MB][4];
#pragma unroll
  for (int mb = 0; mb < VW_MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[mb][i] = 0.0;

  for (int sb = 0; sb < nst; sb += PD) {
#pragma unroll
    for (int p = 0; p < PD; ++p) {
      const int st = sb + p;
      if (st < nst) {
        const int cur = st & 1;
#pragma unroll
        for (int half = 0; half < VW_NS / 16; ++half) {
          f32x4 acc[VW_MB];
#pragma unroll
          for (int mb = 0; mb < VW_MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const u32x4 bx = *reinterpret_cast<const u32x4 *>(&bt[cur][q][16 * half + m][32 * ks + 8 * kq]);
              const bf16x8 bv = __builtin_bit_cast(bf16x8, bx);
#pragma unroll
              for (int mb = 0; mb < VW_MB; ++mb)
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mb][ks], bv, acc[mb], 0, 0, 0);
            }
          }
#pragma unroll
          for (int mb = 0; mb < VW_MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) rs[mb][i] = fma(double(acc[mb][i]), double(acc[mb][i]), rs[mb][i]);
        }
        // stage st + 1 (loaded PD - 1 stages ago) into the other buffer, whose
        // readers finished before the last barrier; its registers take stage st + 1 + PD
        const int nxt = (p + 1) % PD;
        if (st + 1 < nst) {
          store_stage(sreg[nxt], cur ^ 1);
          load_stage(sreg[nxt], st + 1 + PD);
        }
        __syncthreads();
      }
    }
  }
  // rs[mb][i]: token 16 mb + 4 (lane / 16) + i, columns = lane % 16 (mod 16):
  // sum over the 16 lanes of each row of lanes
#pragma unroll
  for (int mb = 0; mb < VW_MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      double x = rs[mb][i];
      x += dpp_f64<0xB1>(x);
      x += dpp_f64<0x4E>(x);
      x += dpp_f64<0x141>(x);
      x += dpp_f64<0x140>(x);
      rs[mb][i] = x;
    }
  if (m == 0) {
#pragma unroll
    for (int mb = 0; mb < VW_MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * mb + 4 * kq + i;
        if (tok < N) a.r2[int64_t(u) * N + tok] = float(rs[mb][i]);
      }
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
  size_t wt_hi, wt_lo, tM, tZ, rM, rZ, c2, r2, psum, total;
};

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

LapLayout lap_layout(int n_layers, int H, int n_kv, int N, int w, int D) {
  const int64_t units = int64_t(n_layers) * n_kv;
  const int G = H / n_kv, R = G * w;
  const int nh = (R + RPG - 1) / RPG, ntiles = (N + TILE - 1) / TILE, nchunks = (N + P_CHUNK - 1) / P_CHUNK;
  LapLayout L{};
  size_t o = 0;
  L.wt_hi = o; o = align256(o + size_t(units) * D * HD * 2);
  L.wt_lo = o; o = align256(o + size_t(units) * D * HD * 2);
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
  if (pass == 1) hipLaunchKernelGGL((k_lap_window<G, 1>), grid, dim3(LNT), 0, st, a);
  else hipLaunchKernelGGL((k_lap_window<G, 2>), grid, dim3(LNT), 0, st, a);
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
  a.nh = (a.R + RPG - 1) / RPG;
  a.ntiles = (N + TILE - 1) / TILE;
  a.nchunks = (N + P_CHUNK - 1) / P_CHUNK;
  a.scale = scale;
  a.score = score;
  a.wt_hi = reinterpret_cast<uint16_t *>(base + L.wt_hi);
  a.wt_lo = reinterpret_cast<uint16_t *>(base + L.wt_lo);
  a.tM = reinterpret_cast<double *>(base + L.tM);
  a.tZ = reinterpret_cast<double *>(base + L.tZ);
  a.rM = reinterpret_cast<double *>(base + L.rM);
  a.rZ = reinterpret_cast<double *>(base + L.rZ);
  a.c2 = reinterpret_cast<float *>(base + L.c2);
  a.r2 = reinterpret_cast<float *>(base + L.r2);
  a.psum = reinterpret_cast<double *>(base + L.psum);
  const int units = n_layers * n_kv;

  // marks (optional): an event before the first kernel and after each of the seven
  auto mark = [&](int i) { return marks ? hipEventRecord(marks[i], st) : hipSuccess; };
  hipError_t e = mark(0);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lap_wprep, dim3(D / 64, HD / 64, units), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(1)) != hipSuccess) return e;
  const dim3 wgrid(a.ntiles, a.nh, units);
  if ((e = window_pass(a, wgrid, st, 1)) != hipSuccess || (e = mark(2)) != hipSuccess) return e;
  const int n_rows = units * a.R;
  hipLaunchKernelGGL(k_lap_rowfin, dim3((n_rows + 255) / 256), dim3(256), 0, st, a, n_rows);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(3)) != hipSuccess) return e;
  if ((e = window_pass(a, wgrid, st, 2)) != hipSuccess || (e = mark(4)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_lap_vw, dim3((N + VW_TOK - 1) / VW_TOK, units), dim3(VW_NT), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(5)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_lap_p, dim3(a.nchunks, units), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(6)) != hipSuccess) return e;
  hipLaunchKernelGGL(k_lap_norm, dim3(a.nchunks, units), dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return mark(7);
}

}  // namespace kvc
