// Streaming geometry and sub-chunk loads shared by the decode kernels that
// stream K/V rows with 16-byte lanes (the per-scope and the split kernel).
#pragma once

#include "kvc_device.h"

namespace kvc {

// Eight waves (two per SIMD, at most 256 registers each) up to four heads per
// group; eight heads need more query and accumulator registers than that and
// run four waves with deeper prefetch. NWO, PFO (non-zero) set the waves and the
// prefetch depth instead (four waves at depth two: two workgroups per CU).
template <typename T, int G = 1, int NWO = 0, int PFO = 0>
struct UnitGeometry {
  static constexpr int EPV = ElemTraits<T>::EPV;
  static constexpr int LPT = HD / EPV;     // lanes per token row
  static constexpr int TPI = 64 / LPT;     // tokens per wave iteration
  static constexpr int UNR = 4;            // iterations per sub-chunk
  static constexpr int CHW = TPI * UNR;    // tokens per sub-chunk
  static constexpr int NW = NWO ? NWO : G >= 8 ? 4 : 8;   // waves
  static constexpr int PF = PFO ? PFO : 16 / NW;         // sub-chunks of loads in flight per wave
  // (Waves 0-3 finish streaming well before waves 4-7: a SIMD's issue
  // arbiter favours the older of its two waves. Giving them a larger share
  // of sub-chunks moves the imbalance without shortening the makespan.)
  static constexpr int NT = 64 * NW;       // threads
  static constexpr int RB = HD * int(sizeof(T));
  static constexpr int NS4 = HD * HD / 4 / NT;   // float4 of the moment matrix per thread
};

// Loads of one sub-chunk: K and V rows, and (MROW) the per-token utility and
// (VOTES) the vote. NTK, NTV: the key or value rows load non-temporally.
template <typename T, bool VOTES, bool MROW = true, bool NTK = false, bool NTV = false>
struct UnitStream {
  using Geo = UnitGeometry<T, 1>;
  static constexpr int UNR = Geo::UNR, TPI = Geo::TPI, CHW = Geo::CHW, RB = Geo::RB;
  const char *Kb, *Vb, *Kn, *Vn;
  const float *mrow;        // utilities of the scope (MROW)
  const int32_t *vrow;
  int L, Lold, append, lane, cb, tg;

  // Loads sub-chunk c; a slot with nothing left (live false) loads one row, the
  // same 16 bytes in every lane, so that every refill takes the same loads and
  // their registers: a refill under a condition leaves the compiler two versions
  // of the slot's registers to merge, and the merge waits for the loads.
  __device__ __forceinline__ void issue(u32x4 (&kr)[UNR], u32x4 (&vr)[UNR], float &mv, int &vv, int c,
                                        bool live = true) const {
    // the small loads first: they are used first, so waiting for them leaves the
    // rows of this and later sub-chunks in flight
    const int t1 = live ? min(c * CHW + (lane % CHW), max(Lold - 1, 0)) : 0;
    mv = MROW ? mrow[t1] : 0.f;
    if (VOTES) vv = vrow[t1];
    const char *kp[UNR], *vp[UNR];
    if (live && (c + 1) * CHW <= Lold) {
      // every token of the sub-chunk is an old, live entry: uniform base + lane offset
      const char *kb = Kb + int64_t(c) * CHW * RB + 16 * lane;
      const char *vb = Vb + int64_t(c) * CHW * RB + 16 * lane;
#pragma unroll
      for (int it = 0; it < UNR; ++it) {
        kp[it] = kb + it * TPI * RB;
        vp[it] = vb + it * TPI * RB;
      }
    } else if (live) {
#pragma unroll
      for (int it = 0; it < UNR; ++it) {
        const int tok = min(c * CHW + it * TPI + tg, L - 1);
        const bool isnew = append && tok == L - 1;
        kp[it] = (isnew ? Kn : Kb + int64_t(tok) * RB) + 16 * cb;
        vp[it] = (isnew ? Vn : Vb + int64_t(tok) * RB) + 16 * cb;
      }
    } else {
#pragma unroll
      for (int it = 0; it < UNR; ++it) {
        kp[it] = Kb;
        vp[it] = Vb;
      }
    }
#pragma unroll
    for (int it = 0; it < UNR; ++it) {
      if constexpr (NTK) kr[it] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)(kp[it]));
      else kr[it] = ld16g(kp[it]);
      if constexpr (NTV) vr[it] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)(vp[it]));
      else vr[it] = ld16g(vp[it]);
    }
  }
};

}  // namespace kvc
