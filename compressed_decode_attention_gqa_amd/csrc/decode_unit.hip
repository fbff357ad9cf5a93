// Decode step with one workgroup per scope, for launches with one attention
// unit per scope, enough scopes to fill the device (the layer stack of a model:
// 256 KV heads) and at most one eviction per scope (the steady state of a
// fixed budget).
//
// Streaming: eight waves (two per SIMD, so one wave's arithmetic overlaps the
// other's memory waits; four for eight-head groups) keep PF sub-chunks of CHW
// tokens of 16-byte K/V loads in flight each. Sub-chunks are handed out in
// order by an LDS counter (a wave takes the next one when a load slot frees),
// so every wave streams until the scope's last sub-chunk and the reads of a
// workgroup stay close together; each workgroup starts at its own sub-chunk
// (a hash of its index) and wraps around, so the workgroups' concurrent reads
// spread over the memory channels; a step at an odd position walks the other
// way, so it first reads the rows the previous step read last, which the
// memory-side cache still holds. Full sub-chunks are addressed as one
// uniform base plus the lane's 16-byte offset; only the last sub-chunk clamps
// per lane and substitutes the appended row. Logits are float64 (exact
// bf16/fp32 products); each lane keeps its query heads in the lane-permuted
// order of preduce, so the transposed reduction leaves one head's logit per
// lane without selects. Each lane forms one weight exp(l - m_c) relative to
// its sub-chunk's own maximum m_c (float64 argument split into float hi +
// lo), and the sub-chunk's maximum and weight sum are kept per head: the
// normaliser and the per-token weights then do not depend on which wave took
// which sub-chunk (the epilogue sums the sub-chunks in a fixed order). The
// value sums run against each wave's running maximum, rescaled only when it
// moves. Per-token weights (with their shift counts, for weights below
// float32's range), utilities (float64) and votes of the scope live in LDS.
//
// Epilogue (same workgroup): combine the waves' partials (one lane per
// (wave, head)), write o and lse, score every token, update the utility, take
// the eviction by argmin over (m, slot) with a tie count carried through the
// same reduction (the float64 utility is ranked before it is stored as
// float32; ties are broken by position), fold it into the moments and
// fill its slot with the last one. The moment sums and the last row are
// loaded before scoring so the fold does not wait on memory. Barriers order
// LDS only, so those loads (and the streaming's last, unused prefetches) stay
// in flight across them; no global location is written by one thread and
// read or rewritten by another.
#include <algorithm>
#include <type_traits>

#include "kvc_epilogue.h"
#include "kvc_stream.h"

namespace kvc {


int decode_unit_chunk_tokens(int dtype) {
  return dtype == 0 ? UnitGeometry<bf16_t>::CHW : UnitGeometry<float>::CHW;
}

// Dynamic LDS: per-token weights e[ld][G], sub-chunk maxima and weight sums
// [nsub][G] (double each), utilities m[ld] (double), votes[ld] and the weights'
// shift counts sh[ld][G] (bytes); ld = lds_len rounded up to whole sub-chunks.
struct UnitLdsLayout {
  int ld;
  size_t e, f, z, m, v, sh, total;
};

__host__ __device__ inline UnitLdsLayout unit_lds_layout(int chw, int G, int lds_len, bool votes) {
  UnitLdsLayout l{};
  l.ld = (lds_len + chw - 1) / chw * chw;
  size_t o = 0;
  l.e = o;
  o += size_t(G) * l.ld * 4;
  o = (o + 15) & ~size_t(15);
  l.f = o;
  o += size_t(l.ld / chw) * G * 8;
  l.z = o;
  o += size_t(l.ld / chw) * G * 8;
  l.m = o;
  o += size_t(l.ld) * 8;
  l.v = o;
  if (votes) o += size_t(l.ld) * 4;
  o = (o + 15) & ~size_t(15);
  l.sh = o;
  o += size_t(l.ld) * G;
  l.total = (o + 15) & ~size_t(15);
  return l;
}

// The G shift counts of one token (bytes sh[i*G .. i*G + G - 1]) as one integer.
template <int G>
__device__ __forceinline__ uint64_t token_shifts(const uint8_t *sh, int i) {
  if constexpr (G == 1) return sh[i];
  else if constexpr (G == 2) return *reinterpret_cast<const uint16_t *>(sh + 2 * i);
  else if constexpr (G == 4) return *reinterpret_cast<const uint32_t *>(sh + 4 * i);
  else return *reinterpret_cast<const uint64_t *>(sh + 8 * i);
}

// Waves and prefetch depth of the per-unit (groups) kernel: four waves at depth
// two, so two workgroups share a CU and one's epilogue overlaps the other's
// streaming; eight-head groups need all of a SIMD's registers for one wave and
// keep the default geometry (four waves, one workgroup per CU).
template <int G>
struct GrpGeo {
  static constexpr int NW = G >= 8 ? 0 : 4, PF = G >= 8 ? 0 : 2, MINB = G >= 8 ? 1 : 2;
};

template <typename T, int G, int NWO = 0, int PFO = 0>
struct UnitLds {
  using Geo = UnitGeometry<T, G, NWO, PFO>;
  float w[Geo::NW][Geo::UNR][Geo::TPI][G];      // streaming: weights for the value sums
  // the epilogue's space (apart from the weights: a wave stores its partials as soon
  // as its streaming ends, while other waves still use theirs)
  struct {
    double pM[Geo::NW][G], zw[Geo::NW][G];
    float pO[Geo::NW][G][HD];
    double M[G];
    float fac[Geo::NW][G];
    uint64_t wkey[Geo::NW];
    int wslot[Geo::NW], wcnt[Geo::NW];
    int tie_pos, tie_slot;
    float rowk[HD], rowv[HD];
  } ep;
  int next_sub;   // the next sub-chunk to hand out
};

template <typename T, int NWO, int PFO>
static size_t unit_static_lds(int G) {
  switch (G) {
    case 1: return sizeof(UnitLds<T, 1, NWO, PFO>);
    case 2: return sizeof(UnitLds<T, 2, NWO, PFO>);
    case 4: return sizeof(UnitLds<T, 4, NWO, PFO>);
    default: return sizeof(UnitLds<T, 8, NWO, PFO>);
  }
}

size_t decode_unit_lds_bytes(int dtype, int G, int lds_len, bool votes) {
  const size_t st = dtype == 0 ? unit_static_lds<bf16_t, 0, 0>(G) : unit_static_lds<float, 0, 0>(G);
  return st + unit_lds_layout(decode_unit_chunk_tokens(dtype), G, lds_len, votes).total;
}

size_t decode_unit_groups_lds_bytes(int dtype, int G, int lds_len, bool votes) {
  // the static part is largest for the four-wave geometry at every G
  const size_t st = dtype == 0 ? std::max(unit_static_lds<bf16_t, 4, 2>(G), unit_static_lds<bf16_t, 0, 0>(G))
                               : std::max(unit_static_lds<float, 4, 2>(G), unit_static_lds<float, 0, 0>(G));
  return st + unit_lds_layout(decode_unit_chunk_tokens(dtype), G, lds_len, votes).total;
}


// Token i's score numerator: sum over the G heads of its weight (token-major in
// e_lds) times its sub-chunk's factor exp(m_c - M) / Z (f_lds), and for a weight
// stored shifted, times exp(-SHIFT_STEP * shift). The shifted form is taken for a
// whole wave only when one of its tokens needs it; a head without a shift
// multiplies by exactly 1, so both forms agree.
template <int G>
__device__ __forceinline__ double token_score(const float *e_lds, const double *f_lds, const uint8_t *s_lds, int i,
                                              int c) {
  float ev[G];
  if constexpr (G == 1) {
    ev[0] = e_lds[i];
  } else if constexpr (G == 2) {
    const float2 v = *reinterpret_cast<const float2 *>(e_lds + 2 * i);
    ev[0] = v.x; ev[1] = v.y;
  } else {
#pragma unroll
    for (int q = 0; q < G / 4; ++q) {
      const float4 v = *reinterpret_cast<const float4 *>(e_lds + G * i + 4 * q);
      ev[4 * q] = v.x; ev[4 * q + 1] = v.y; ev[4 * q + 2] = v.z; ev[4 * q + 3] = v.w;
    }
  }
  const uint64_t shw = token_shifts<G>(s_lds, i);
  double acc = 0.0;
#pragma unroll
  for (int g = 0; g < G; ++g) acc += double(ev[g]) * f_lds[c * G + g];
  if (__builtin_expect(__ballot(shw != 0) != 0, 0)) {
    if (shw != 0) {
      acc = 0.0;
#pragma unroll
      for (int g = 0; g < G; ++g)
        acc += double(ev[g]) * f_lds[c * G + g] * shift_scale(int((shw >> (8 * g)) & 255u));
    }
  }
  return acc;
}

// GRP: one workgroup per attention unit of every scope (blockIdx.x = scope *
// attn_units + unit), attending only, with no append: o, lse and, when scores are
// refreshed, the unit's per-token sum over its heads of the vote-weighted
// attention weights into wsum (the groups score kernel then averages them over
// each group's units and chains the utility updates).
template <typename T, int G, bool VOTES, bool GRP = false>
__global__ __launch_bounds__((UnitGeometry<T, G, GRP ? GrpGeo<G>::NW : 0, GRP ? GrpGeo<G>::PF : 0>::NT),
                             GRP ? GrpGeo<G>::MINB : 1)
void k_decode_unit(const StepArgs a) {
  using TR = ElemTraits<T>;
  using Geo = UnitGeometry<T, G, GRP ? GrpGeo<G>::NW : 0, GRP ? GrpGeo<G>::PF : 0>;
  constexpr int EPV = Geo::EPV, LPT = Geo::LPT, TPI = Geo::TPI, UNR = Geo::UNR;
  constexpr int CHW = Geo::CHW, PF = Geo::PF, NW = Geo::NW, NT = Geo::NT, RB = Geo::RB;
  constexpr int D = LPT / G;                         // lanes sharing one (token, head) logit
  constexpr int ITL = (UNR + D - 1) / D;             // weights a lane forms per sub-chunk
  static_assert(NW * G <= 64, "the combine runs in one wave");

  __shared__ UnitLds<T, G, GRP ? GrpGeo<G>::NW : 0, GRP ? GrpGeo<G>::PF : 0> sh;
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int lds_len = a.lds_len;
  const UnitLdsLayout lay = unit_lds_layout(CHW, G, lds_len, VOTES);
  float *e_lds = reinterpret_cast<float *>(dyn + lay.e);
  double *f_lds = reinterpret_cast<double *>(dyn + lay.f);
  double *z_lds = reinterpret_cast<double *>(dyn + lay.z);
  double *m_lds = reinterpret_cast<double *>(dyn + lay.m);
  int *v_lds = reinterpret_cast<int *>(dyn + lay.v);
  uint8_t *s_lds = reinterpret_cast<uint8_t *>(dyn + lay.sh);

  // the wave index as a scalar (uniform per wave), so values derived from it stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int gu = blockIdx.x;
  const int scope = GRP ? gu / a.attn_units : gu;
  const int unit = GRP ? a.attn_unit0 + (gu - scope * a.attn_units) : a.attn_unit0;
  const int cap = a.capacity;
  const int64_t sc = int64_t(scope) * cap;
  int L = a.len[scope] + a.append;
  const bool overflow = L > cap || L > lds_len;
  if (overflow) L = 0;
  const int Lold = L - (L > 0 ? a.append : 0);

  // Key rows load non-temporally: for a per-scope step the memory-side cache then keeps
  // the value rows, about half of a step's bytes, which fit in it, and the next step
  // (walking the other way) finds them there (with every row allocating, each step's rows
  // evicted the ones the next step reads first). A groups call streams every later layer
  // of a model once, far more than that cache holds: none of its rows allocates.
  UnitStream<T, VOTES, !GRP, true, GRP> W;
  {
    const int64_t row0 = int64_t(scope) * a.scope_stride + int64_t(unit) * a.unit_stride;
    W.Kb = a.k + row0 * RB;
    W.Vb = a.v + row0 * RB;
    W.Kn = a.k_new + (int64_t(scope) * a.units + unit) * RB;
    W.Vn = a.v_new + (int64_t(scope) * a.units + unit) * RB;
    // without utilities (attention only), the staged values are never used:
    // read the positions in their place so the loads stay in bounds
    W.mrow = a.m ? a.m + sc : reinterpret_cast<const float *>(a.pos + sc);
    W.vrow = VOTES ? a.votes + sc : nullptr;
    W.L = L;
    W.Lold = Lold;
    W.append = a.append;
    W.lane = lane;
    W.cb = lane % LPT;
    W.tg = lane / LPT;
  }
  const int cb = W.cb, tg = W.tg;
  const int myh = perm_head<LPT, G>(cb);
  const int dup = lane & (D - 1);

  // queries scaled by tau (exact in float64: bf16/fp32 times a float), slot i
  // holding head i ^ myh
  double qf[G][EPV];
  {
    const T *qp = reinterpret_cast<const T *>(a.q) + int64_t(gu) * G * HD;
#pragma unroll
    for (int i = 0; i < G; ++i)
#pragma unroll
      for (int j = 0; j < EPV; ++j)
        qf[i][j] = double(load_elem<T>(qp, (i ^ myh) * HD + cb * EPV + j)) * a.scale;
  }
  float oacc[G][EPV];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < EPV; ++j) oacc[g][j] = 0.f;
  double Mrun = -INFINITY;

  const int nsub = L > 0 ? (L + CHW - 1) / CHW : 0;
  const bool rev = !GRP && (a.t & 1) != 0;   // walk order of this step
  // Each workgroup starts its walk at its own sub-chunk (a multiplicative hash of its
  // index, fixed across steps) and wraps around: workgroups that all started at the
  // same offset of their regions read rows that collide in the memory channels. A
  // forward walk from rot ends at rot - 1, where the next step's backward walk starts.
  const int rot = nsub > 0 ? int((uint32_t(gu) * 2654435761u) % uint32_t(nsub)) : 0;
  auto sub_of = [&](int n) {
    int c = rev ? rot - 1 - n : rot + n;
    c += c < 0 ? nsub : 0;
    c -= c >= nsub ? nsub : 0;
    return c;
  };
  if (tid == 0) sh.next_sub = NW * PF;
  __syncthreads();
  u32x4 kr[PF][UNR], vr[PF][UNR];
  float mv[PF];
  int vv[PF];
  int cs[PF];   // the sub-chunk (in walk order) of each load slot
#pragma unroll
  for (int s = 0; s < PF; ++s) {
    cs[s] = wave + NW * s;
    const bool live = cs[s] < nsub;
    W.issue(kr[s], vr[s], mv[s], vv[s], live ? sub_of(cs[s]) : 0, live);
  }
  for (;;) {
    bool more = false;
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const bool cur = cs[s] < nsub;
      if (cur) {
        const int c = sub_of(cs[s]);
        const bool tail = (c + 1) * CHW > L;
        // scope arrays of this sub-chunk into LDS
        if (lane < CHW) {
          if (!GRP) m_lds[c * CHW + lane] = double(mv[s]);
          if (VOTES) v_lds[c * CHW + lane] = vv[s];
        }
        double lg[UNR];
#pragma unroll
        for (int it = 0; it < UNR; ++it) {
          double acc[G];
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g] = 0.0;
#pragma unroll
          for (int j = 0; j < EPV; ++j) {
            const double kj = double(TR::get(kr[s][it], j));
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = fma(qf[g][j], kj, acc[g]);
          }
          lg[it] = preduce<LPT, G, 0>(acc);
          if (tail && c * CHW + it * TPI + tg >= L) lg[it] = -INFINITY;
        }
        double mx = lg[0];
#pragma unroll
        for (int it = 1; it < UNR; ++it) mx = fmax(mx, lg[it]);
#pragma unroll
        for (int o = LPT; o < 64; o <<= 1) mx = fmax(mx, __shfl_xor(mx, o));
        if (__ballot(mx > Mrun)) {
          const double Mnew = fmax(Mrun, mx);
          const double f = Mrun > -INFINITY ? exp(Mrun - Mnew) : 0.0;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float fg = float(readlane_f64(f, perm_rep_lane<LPT, G>(g)));
#pragma unroll
            for (int j = 0; j < EPV; ++j) oacc[g][j] *= fg;
          }
          Mrun = Mnew;
        }
        // weights relative to the sub-chunk's maximum; the value sums take them
        // times exp(m_c - Mrun) <= 1
        const float rc = exp_split(mx - Mrun);
        double zc = 0.0;
        __builtin_amdgcn_wave_barrier();
        // one weight per (token, head): lane `dup` takes iterations dup, dup + D, ...
#pragma unroll
        for (int r = 0; r < ITL; ++r) {
          const int it = dup + D * r;
          // the token's vote: lane tok - c * CHW loaded it with this sub-chunk (read
          // with every lane active: the source lane may form no weight itself)
          const int vt = VOTES ? __shfl(vv[s], min(it, UNR - 1) * TPI + tg) : 1;
          if (it < UNR) {
            double x = lg[0];
#pragma unroll
            for (int i2 = 1; i2 < UNR; ++i2) x = it == i2 ? lg[i2] : x;
            const int tok = c * CHW + it * TPI + tg;
            int shc;
            const float e = exp_shifted(x - mx, shc);
            const float p = (!VOTES || (a.append && tok == L - 1)) ? 1.f : float(vt);
            // a shifted weight is below exp(-SHIFT_STEP) of the maximum: nothing in o or Z
            const float pe = shc ? 0.f : p * e;
            zc += double(pe);
            sh.w[wave][it][tg][myh] = pe * rc;
            if (tok < L) {
              e_lds[tok * G + myh] = e;
              s_lds[tok * G + myh] = uint8_t(shc);
            }
          }
        }
        // the sub-chunk's weight sum per head: over the lanes holding that head
#pragma unroll
        for (int o = 1; o < D; o <<= 1) zc += __shfl_xor(zc, o);
#pragma unroll
        for (int o = LPT; o < 64; o <<= 1) zc += __shfl_xor(zc, o);
        if (tg == 0 && dup == 0) {
          f_lds[c * G + myh] = mx;
          z_lds[c * G + myh] = zc;
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int it = 0; it < UNR; ++it) {
          float wv[G];
#pragma unroll
          for (int g = 0; g < G; ++g) wv[g] = sh.w[wave][it][tg][g];
#pragma unroll
          for (int j = 0; j < EPV; ++j) {
            const float vj = TR::get(vr[s][it], j);
#pragma unroll
            for (int g = 0; g < G; ++g) oacc[g][j] = fmaf(wv[g], vj, oacc[g][j]);
          }
        }
        __builtin_amdgcn_wave_barrier();
        // the refill's loads stay after the value sums: the slot's registers are free
        // then and the loads can land in them
        __builtin_amdgcn_sched_barrier(0);
      }
      // the slot's next sub-chunk
      int nc = cs[s];
      if (cur) {
        int got = 0;
        if (lane == 0) got = atomicAdd(&sh.next_sub, 1);
        nc = __builtin_amdgcn_readfirstlane(got);
      }
      cs[s] = nc;
      // every pass refills every slot, a finished one with one row (see
      // UnitStream::issue): the slot's registers then have one definition in the
      // loop, which they keep without a copy that would wait for the loads
      const bool live = nc < nsub;
      W.issue(kr[s], vr[s], mv[s], vv[s], live ? sub_of(nc) : 0, live);
      more |= live;
    }
    // out once no slot got a sub-chunk: the last pass's refills are all the one row
    if (!more) break;
  }

  // ---- this wave's partials (running maximum per head; value sums over the wave's
  // token groups by lane swaps) into LDS (their space is the wave's own: no wait
  // for the waves that still stream)
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < EPV; ++j) {
      float x = oacc[g][j];
      if constexpr (LPT == 16) x += lane_xor16(x);
      x += lane_xor32(x);
      oacc[g][j] = x;
    }
  if (lane < LPT) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int j = 0; j < EPV; ++j) sh.ep.pO[wave][g][cb * EPV + j] = oacc[g][j];
  }
  if (tg == 0 && dup == 0) sh.ep.pM[wave][myh] = Mrun;

  // ---- loads the epilogue needs, issued by each wave as its streaming ends (the
  // other waves may still stream): its share of the moment sums, the last live row
  const bool step = a.mode != 0;
  const int k = step ? max(0, L - a.budget) : 0;
  const bool fold = !GRP && !overflow && step && k == 1 && a.mom_S != nullptr;
  const int64_t mu = int64_t(scope) * a.units + unit;
  float4 Sreg[Geo::NS4];
  float skv = 0.f;
  if (fold) {
    const float4 *S4 = reinterpret_cast<const float4 *>(a.mom_S + mu * HD * HD);
#pragma unroll
    for (int j = 0; j < Geo::NS4; ++j) Sreg[j] = ld_nt4(S4 + tid + NT * j);
    if (tid < 2 * HD) skv = tid < HD ? a.mom_sk[mu * HD + tid] : a.mom_sv[mu * HD + tid - HD];
  }
  // the last live row (the appended one when appending): one 16-byte vector per
  // thread, K in threads [0, NV), V in [NV, 2 NV)
  constexpr int NV = RB / 16;
  const int lastc = tid % NV;
  const bool lastK = tid < NV, lastV = tid >= NV && tid < 2 * NV;
  u32x4 lastrow = u32x4(0u);
  if (!GRP && L > 0 && (lastK || lastV)) {
    const char *src = a.append ? (lastK ? W.Kn : W.Vn) : (lastK ? W.Kb : W.Vb) + int64_t(L - 1) * RB;
    lastrow = ld16(src + 16 * lastc);
  }
  lds_barrier();
  if (overflow || k > 1) {
    // k > 1 cannot happen: the host launches this kernel only when
    // lds_len <= budget + 1, and L <= lds_len here
    if (tid == 0) {
      a.status[0] = overflow ? -4 : -3;
      if (a.mode == 2) a.list[sc] = -1;
    }
    return;
  }

  int last_pos = a.t;
  if (!GRP && !a.append && L > 0) last_pos = a.pos[sc + L - 1];

  // ---- the head maxima M (over the waves' running maxima) and the normalisers
  // Z = sum_c z_c exp(m_c - M) in a fixed order: thread t takes the (sub-chunk,
  // head) entries t, t + NT, ... (its head is t % G), then a fixed tree over
  // the threads of each head; f_lds becomes exp(m_c - M)
  const int nsubL = (L + CHW - 1) / CHW;
  {
    const int g = tid % G;
    double M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmax(M, sh.ep.pM[w][g]);
    double zp = 0.0;
    for (int idx = tid; idx < nsubL * G; idx += NT) {
      // exp(m_c - M) <= 1: to about one float ulp (the per-token weights are floats
      // too) in float32's normal range, in float64 below it, where the scores of a
      // sub-chunk far below the head maximum still rank on their float64 values
      const double d = f_lds[idx] - M;
      const double ex = d >= -SHIFT_STEP ? double(exp_split(d)) : d > -1.0e30 ? exp(d) : 0.0;
      zp += z_lds[idx] * ex;
      f_lds[idx] = ex;
    }
#pragma unroll
    for (int o = G; o < 64; o <<= 1) zp += __shfl_xor(zp, o);
    if (lane < G) sh.ep.zw[wave][lane] = zp;
    if (tid < G) sh.ep.M[tid] = M;
  }
  lds_barrier();
  {
    // this thread's sub-chunk factors become exp(m_c - M) / Z (its entries all belong to
    // head tid % G; Z summed over the waves in the same order as below)
    const int g = tid % G;
    double Z = 0.0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) Z += sh.ep.zw[w2][g];
    const double iZ = Z > 0.0 ? 1.0 / Z : 0.0;
    for (int idx = tid; idx < nsubL * G; idx += NT) f_lds[idx] *= iZ;
  }
  if (tid < NW * G) {   // Z per head (the same sum in every thread of the head), the waves' factors
    const int w = tid / G, g = tid % G;
    double Z = 0.0;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) Z += sh.ep.zw[w2][g];
    const double M = sh.ep.M[g], pm = sh.ep.pM[w][g];
    sh.ep.fac[w][g] = (Z > 0.0 && pm > -INFINITY) ? float(double(exp_split(pm - M)) / Z) : 0.f;
    if (w == 0) {
      a.lse[int64_t(gu) * G + g] = Z > 0.0 ? float(M + log(Z)) : -INFINITY;
    }
  }
  lds_barrier();
  for (int idx = tid; idx < G * HD; idx += NT) {
    const int g = idx / HD, e = idx - (idx / HD) * HD;
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) acc = fmaf(sh.ep.pO[w][g][e], sh.ep.fac[w][g], acc);
    st_nt(&a.out[(int64_t(gu) * G + g) * HD + e], acc);
  }

  const bool score = a.refresh && (step || a.s != nullptr);

  if constexpr (GRP) {
    // the unit's per-token weight sums (the score's numerator over this unit's heads)
    if (a.refresh) {
      double *wrow = a.wsum + int64_t(gu) * a.wsum_stride;
      for (int i = tid; i < L; i += NT) {
        const double acc = token_score<G>(e_lds, f_lds, s_lds, i, i / CHW);
        st_nt(&wrow[i], VOTES ? acc * double(v_lds[i]) : acc);
      }
    }
    return;
  }

  // ---- score, utility; per thread the smallest (m, slot) and how many slots hold that m
  const double inv_heads = 1.0 / double(G);
  const double alpha = double(a.alpha);
  uint64_t bestm = ~0ull;
  int bslot = 0x7fffffff, bcnt = 0;
#pragma unroll 2
  for (int i = tid; i < L; i += NT) {
    const bool isnew = a.append && i == L - 1;
    const double mold = m_lds[i];
    double mval = isnew ? 0.0 : mold;
    if (score) {
      double acc = token_score<G>(e_lds, f_lds, s_lds, i, i / CHW);
      if (VOTES && !isnew) acc *= double(v_lds[i]);
      const double sv = acc * inv_heads;
      if (a.s) st_nt(&a.s[sc + i], float(sv));
      if (step) mval = apply_rule(a.rule, alpha, mval, sv);
    }
    if ((step && score) || isnew) st_nt(&a.m[sc + i], float(mval));
    m_lds[i] = mval;
    const uint64_t om = orderable_f64(mval);
    if (om < bestm) {
      bestm = om;
      bslot = i;
      bcnt = 1;
    } else if (om == bestm) {
      ++bcnt;
    }
  }
  int e1 = -1;
  if (k == 1) {
    wave_reduce_key_slot_cnt(bestm, bslot, bcnt, [&](uint64_t m2, int s2, int c2) {
      if (m2 < bestm) {
        bestm = m2;
        bslot = s2;
        bcnt = c2;
      } else if (m2 == bestm) {
        bslot = min(bslot, s2);
        bcnt += c2;
      }
    });
    if (lane == 0) {
      sh.ep.wkey[wave] = bestm;
      sh.ep.wslot[wave] = bslot;
      sh.ep.wcnt[wave] = bcnt;
    }
    if (tid == 0) {
      sh.ep.tie_pos = 0x7fffffff;
      sh.ep.tie_slot = 0x7fffffff;
    }
    lds_barrier();
    uint64_t mmin = sh.ep.wkey[0];
    int smin = sh.ep.wslot[0], ties = sh.ep.wcnt[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      const uint64_t m2 = sh.ep.wkey[w];
      if (m2 < mmin) {
        mmin = m2;
        smin = sh.ep.wslot[w];
        ties = sh.ep.wcnt[w];
      } else if (m2 == mmin) {
        smin = min(smin, sh.ep.wslot[w]);
        ties += sh.ep.wcnt[w];
      }
    }
    if (ties > 1) {
      // exact utility ties: the smallest position among them goes
      for (int i = tid; i < L; i += NT) {
        if (orderable_f64(m_lds[i]) == mmin) {
          const int p = (a.append && i == L - 1) ? a.t : a.pos[sc + i];
          atomicMin(&sh.ep.tie_pos, p);
        }
      }
      lds_barrier();
      for (int i = tid; i < L; i += NT) {
        if (orderable_f64(m_lds[i]) == mmin) {
          const int p = (a.append && i == L - 1) ? a.t : a.pos[sc + i];
          if (p == sh.ep.tie_pos) atomicMin(&sh.ep.tie_slot, i);
        }
      }
      lds_barrier();
      smin = sh.ep.tie_slot;
    }
    e1 = smin;
  }

  // ---- append: the new row, vote and position at slot L - 1
  if (a.append && L > 0) {
    if (lastK) st16(const_cast<char *>(W.Kb) + int64_t(L - 1) * RB + 16 * lastc, lastrow);
    if (lastV) st16(const_cast<char *>(W.Vb) + int64_t(L - 1) * RB + 16 * lastc, lastrow);
    if (tid == 0) {
      if (VOTES) a.votes[sc + L - 1] = 1;
      a.pos[sc + L - 1] = a.t;
    }
  }
  if (!step || k == 0) {
    if (a.evict_out)
      for (int i = tid; i < L; i += NT) a.evict_out[sc + i] = 0;
    if (tid == 0) {
      if (a.mode == 2) a.list[sc] = -1;   // nothing for the merge kernels
      a.len[scope] = L;
    }
    return;
  }

  // ---- one eviction: flags, fold, fill the hole with the last slot
  if (a.evict_out)
    for (int i = tid; i < L; i += NT) a.evict_out[sc + i] = (i == e1);
  if (tid == 0) a.list[sc] = e1;
  if (fold) {
    if (e1 == L - 1) {
      if (lastK || lastV) {
        float *dst = lastK ? sh.ep.rowk : sh.ep.rowv;
#pragma unroll
        for (int j = 0; j < EPV; ++j) dst[lastc * EPV + j] = TR::get(lastrow, j);
      }
    } else if (lastK || lastV) {
      const u32x4 r = ld16((lastK ? W.Kb : W.Vb) + int64_t(e1) * RB + 16 * lastc);
      float *dst = lastK ? sh.ep.rowk : sh.ep.rowv;
#pragma unroll
      for (int j = 0; j < EPV; ++j) dst[lastc * EPV + j] = TR::get(r, j);
    }
    lds_barrier();
    // S[r][c] += v_e[r] k_e[c]: thread tid owns columns 4 (tid % 32) .. + 3 of
    // rows tid / 32 + (NT / 32) j
    const int col = 4 * (tid & 31), row0 = tid >> 5;
    const float4 k4 = *reinterpret_cast<const float4 *>(&sh.ep.rowk[col]);
    float4 *S4 = reinterpret_cast<float4 *>(a.mom_S + mu * HD * HD);
#pragma unroll
    for (int j = 0; j < Geo::NS4; ++j) {
      const float va = sh.ep.rowv[row0 + (NT / 32) * j];
      float4 x = Sreg[j];
      x.x = fmaf(va, k4.x, x.x);
      x.y = fmaf(va, k4.y, x.y);
      x.z = fmaf(va, k4.z, x.z);
      x.w = fmaf(va, k4.w, x.w);
      st_nt4(S4 + tid + NT * j, x);
    }
    if (tid < HD) st_nt(&a.mom_sk[mu * HD + tid], skv + sh.ep.rowk[tid]);
    else if (tid < 2 * HD) st_nt(&a.mom_sv[mu * HD + tid - HD], skv + sh.ep.rowv[tid - HD]);
    if (tid == 0) a.mom_n[mu] += 1;
  }
  if (a.mode == 2) {
    if (tid == 0) a.len[scope] = L;
    return;
  }
  if (e1 < L - 1) {
    // the last slot's row (held in registers) moves into the hole
    if (lastK || lastV) st16(const_cast<char *>(lastK ? W.Kb : W.Vb) + int64_t(e1) * RB + 16 * lastc, lastrow);
    if (tid == 0) {
      if (VOTES) a.votes[sc + e1] = a.append ? 1 : v_lds[L - 1];
      a.pos[sc + e1] = last_pos;
    }
    // the thread that stored slot e1's utility in the score pass overwrites it
    if (tid == e1 % NT) a.m[sc + e1] = float(m_lds[L - 1]);
  }
  if (tid == 0) a.len[scope] = L - 1;
}

template <typename T, int G, bool VOTES>
static hipError_t launch_unit_tgv(const StepArgs &a, hipStream_t st) {
  using Geo = UnitGeometry<T, G>;
  const size_t dyn = unit_lds_layout(Geo::CHW, G, a.lds_len, VOTES).total;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_decode_unit<T, G, VOTES>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(dyn));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode_unit<T, G, VOTES>), dim3(a.n_scopes), dim3(Geo::NT), dyn, st, a);
  return hipGetLastError();
}

template <typename T, int G>
static hipError_t launch_unit_tg(const StepArgs &a, hipStream_t st) {
  return a.votes ? launch_unit_tgv<T, G, true>(a, st) : launch_unit_tgv<T, G, false>(a, st);
}

template <typename T>
static hipError_t launch_unit_g(const StepArgs &a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_unit_tg<T, 1>(a, st);
    case 2: return launch_unit_tg<T, 2>(a, st);
    case 4: return launch_unit_tg<T, 4>(a, st);
    case 8: return launch_unit_tg<T, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_unit(const StepArgs &a, int dtype, int G, hipStream_t st) {
  return dtype == 0 ? launch_unit_g<bf16_t>(a, G, st) : launch_unit_g<float>(a, G, st);
}

template <typename T, int G, bool VOTES>
static hipError_t launch_unit_groups_tgv(const StepArgs &a, hipStream_t st) {
  using Geo = UnitGeometry<T, G, GrpGeo<G>::NW, GrpGeo<G>::PF>;
  const size_t dyn = unit_lds_layout(Geo::CHW, G, a.lds_len, VOTES).total;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_decode_unit<T, G, VOTES, true>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, int(dyn));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_decode_unit<T, G, VOTES, true>), dim3(a.n_scopes * a.attn_units), dim3(Geo::NT), dyn, st,
                     a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_unit_groups_g(const StepArgs &a, int G, hipStream_t st) {
  const bool v = a.votes != nullptr;
  switch (G) {
    case 1: return v ? launch_unit_groups_tgv<T, 1, true>(a, st) : launch_unit_groups_tgv<T, 1, false>(a, st);
    case 2: return v ? launch_unit_groups_tgv<T, 2, true>(a, st) : launch_unit_groups_tgv<T, 2, false>(a, st);
    case 4: return v ? launch_unit_groups_tgv<T, 4, true>(a, st) : launch_unit_groups_tgv<T, 4, false>(a, st);
    case 8: return v ? launch_unit_groups_tgv<T, 8, true>(a, st) : launch_unit_groups_tgv<T, 8, false>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_unit_groups(const StepArgs &a, int dtype, int G, hipStream_t st) {
  return dtype == 0 ? launch_unit_groups_g<bf16_t>(a, G, st) : launch_unit_groups_g<float>(a, G, st);
}

}  // namespace kvc
