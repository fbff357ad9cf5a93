// Device-side helpers shared by the kvc kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

constexpr int HD = 128;      // head dimension handled by every kernel
constexpr int WG = 256;      // threads per workgroup (4 waves of 64)

// 16-byte vector: one global/LDS access of 16 bytes per lane.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- element types
// Storage types of K/V/q: bf16 is carried as its 16-bit pattern.
struct bf16_t { uint16_t b; };

template <typename T> struct ElemTraits;
template <> struct ElemTraits<bf16_t> {
  static constexpr int EPV = 8;                   // elements per 16-byte vector
  __device__ static __forceinline__ float get(const u32x4 &v, int j) {
    uint32_t w = (j >> 1) == 0 ? v.x : (j >> 1) == 1 ? v.y : (j >> 1) == 2 ? v.z : v.w;
    return (j & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
  }
};
template <> struct ElemTraits<float> {
  static constexpr int EPV = 4;
  __device__ static __forceinline__ float get(const u32x4 &v, int j) {
    uint32_t w = j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
    return __uint_as_float(w);
  }
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// double -> bf16 bits, one rounding to nearest even: the float conversion made
// round-to-odd (truncated toward zero, last bit set when inexact) so the
// second rounding cannot land on a tie the first one created.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  const float f = float(x);
  uint32_t u = __float_as_uint(f);
  const double fd = double(f);
  if (fd != x) {
    if (fabs(fd) > fabs(x)) u -= 1u;   // rounded away from zero: one step back (sign-magnitude)
    u |= 1u;
  }
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// A double rounded once to the cache dtype, as a float.
template <typename T> __device__ __forceinline__ float round_once(double x);
template <> __device__ __forceinline__ float round_once<bf16_t>(double x) { return bf16_to_f32(f64_to_bf16(x)); }
template <> __device__ __forceinline__ float round_once<float>(double x) { return float(x); }

template <typename T> __device__ __forceinline__ float load_elem(const T *p, int64_t i);
template <> __device__ __forceinline__ float load_elem<bf16_t>(const bf16_t *p, int64_t i) {
  return bf16_to_f32(p[i].b);
}
template <> __device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }

template <typename T> __device__ __forceinline__ void store_elem(T *p, int64_t i, float x);
template <> __device__ __forceinline__ void store_elem<bf16_t>(bf16_t *p, int64_t i, float x) {
  p[i].b = f32_to_bf16(x);
}
template <> __device__ __forceinline__ void store_elem<float>(float *p, int64_t i, float x) { p[i] = x; }

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
// The same load through a global-memory pointer: where the address is selected among
// several pointers the compiler cannot tell it is global and would emit a flat load,
// which also holds up every wait for LDS results.
__device__ __forceinline__ u32x4 ld16g(const void *p) {
  return *(const __attribute__((address_space(1))) u32x4 *)(p);
}
__device__ __forceinline__ void st16(void *p, const u32x4 &v) { *reinterpret_cast<u32x4 *>(p) = v; }

// Non-temporal accesses, for results a kernel writes once at its end (scores,
// utilities, outputs) and for the moment sums it reads and rewrites there: on
// gfx950 these lines do not stay in the XCD's L2 as ordinary dirty lines, so the
// L2 write-back that ends every kernel has little left to write. (Loads that a
// latency-bound kernel waits on stay ordinary: non-temporal ones took longer.)
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt(float *p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt(double *p, double v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt4(float4 *p, const float4 &v) {
  const f32x4 x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>(p));
}
__device__ __forceinline__ float ld_nt(const float *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float4 ld_nt4(const float4 *p) {
  const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
  return make_float4(x.x, x.y, x.z, x.w);
}

// ---------------------------------------------------------------- cross-lane
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  int lo = __double2loint(x), hi = __double2hiint(x);
  lo = __builtin_amdgcn_mov_dpp(lo, CTRL, 0xf, 0xf, true);
  hi = __builtin_amdgcn_mov_dpp(hi, CTRL, 0xf, 0xf, true);
  return __hiloint2double(hi, lo);
}

// Sum over aligned groups of LANES lanes (16 or 32); every lane gets its group's sum.
template <int LANES>
__device__ __forceinline__ double group_sum_f64(double x) {
  x += dpp_f64<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_f64<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_f64<0x141>(x);   // row_half_mirror: pairs the two quads of each half-row
  x += dpp_f64<0x140>(x);   // row_mirror: pairs the two halves of each 16-lane row
  if constexpr (LANES == 32) x += __shfl_xor(x, 16);
  return x;
}

// Reductions over lanes whose index differs only in bits >= log2(STRIDE) (STRIDE a power of 2).
template <int STRIDE>
__device__ __forceinline__ double wave_max_strided(double x) {
#pragma unroll
  for (int o = STRIDE; o < 64; o <<= 1) x = fmax(x, __shfl_xor(x, o));
  return x;
}
template <int STRIDE>
__device__ __forceinline__ double wave_sum_strided(double x) {
#pragma unroll
  for (int o = STRIDE; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}
template <int STRIDE>
__device__ __forceinline__ float wave_sum_strided_f32(float x) {
#pragma unroll
  for (int o = STRIDE; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int o) {
  uint32_t lo = uint32_t(x), hi = uint32_t(x >> 32);
  lo = __shfl_xor(lo, o);
  hi = __shfl_xor(hi, o);
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint64_t y = shfl_xor_u64(x, o);
    x = y < x ? y : x;
  }
  return x;
}

// The value of lane l ^ 32 (or l ^ 16) through the gfx950 lane swaps, without LDS: a swap of
// x with itself leaves x[l ^ 32] in the first result on the upper half of the wave and in
// the second on the lower half (likewise for 16-lane halves of each 32).
__device__ __forceinline__ uint32_t lane_xor32(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return (threadIdx.x & 32) ? r[0] : r[1];
}
__device__ __forceinline__ uint32_t lane_xor16(uint32_t x) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return (threadIdx.x & 16) ? r[0] : r[1];
}
__device__ __forceinline__ float lane_xor32(float x) { return __uint_as_float(lane_xor32(__float_as_uint(x))); }
__device__ __forceinline__ float lane_xor16(float x) { return __uint_as_float(lane_xor16(__float_as_uint(x))); }
__device__ __forceinline__ uint64_t lane_xor32(uint64_t x) {
  return (uint64_t(lane_xor32(uint32_t(x >> 32))) << 32) | lane_xor32(uint32_t(x));
}
__device__ __forceinline__ uint64_t lane_xor16(uint64_t x) {
  return (uint64_t(lane_xor16(uint32_t(x >> 32))) << 32) | lane_xor16(uint32_t(x));
}
__device__ __forceinline__ int lane_xor32(int x) { return int(lane_xor32(uint32_t(x))); }
__device__ __forceinline__ int lane_xor16(int x) { return int(lane_xor16(uint32_t(x))); }

// The value a DPP pattern moves into this lane (all patterns used stay inside a 16-lane row).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(x), CTRL, 0xf, 0xf, true));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  return (uint64_t(dpp_u32<CTRL>(uint32_t(x >> 32))) << 32) | dpp_u32<CTRL>(uint32_t(x));
}

// Wave reduction over lane pairings that reach all 64 lanes in six stages: quad_perm
// [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror, then the 16- and 32-lane
// swaps. f(partner values...) combines a partner into this lane's state; every lane ends
// with the whole wave's result when f is associative and commutative.
template <class F>
__device__ __forceinline__ void wave_reduce_key_slot_cnt(uint64_t &key, int &slot, int &cnt, F f) {
  f(dpp_u64<0xB1>(key), int(dpp_u32<0xB1>(uint32_t(slot))), int(dpp_u32<0xB1>(uint32_t(cnt))));
  f(dpp_u64<0x4E>(key), int(dpp_u32<0x4E>(uint32_t(slot))), int(dpp_u32<0x4E>(uint32_t(cnt))));
  f(dpp_u64<0x141>(key), int(dpp_u32<0x141>(uint32_t(slot))), int(dpp_u32<0x141>(uint32_t(cnt))));
  f(dpp_u64<0x140>(key), int(dpp_u32<0x140>(uint32_t(slot))), int(dpp_u32<0x140>(uint32_t(cnt))));
  f(lane_xor16(key), lane_xor16(slot), lane_xor16(cnt));
  f(lane_xor32(key), lane_xor32(slot), lane_xor32(cnt));
}

// Exclusive prefix count of a 0/1 predicate within the wave, and the wave total.
__device__ __forceinline__ int wave_prefix_count(bool pred, int *total) {
  uint64_t b = __ballot(pred);
  *total = __popcll(b);
  return __builtin_amdgcn_mbcnt_hi(uint32_t(b >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(b), 0));
}

// ---------------------------------------------------------------- numerics
// exp(x) for x in float64 to about one float32 ulp: x = hi + lo with hi the
// nearest float; exp(hi) from the accurate float exp, times (1 + lo).
__device__ __forceinline__ float exp_split(double x) {
  if (!(x > -1.0e30)) return 0.0f;
  float hi = float(x);
  float lo = float(x - double(hi));
  float eh = expf(hi);
  return fmaf(eh, lo, eh);
}

// Weights far below the running maximum. float32 keeps exp(x) only down to
// x ~ -103 while float64 keeps it to x ~ -745, so a weight with x < -SHIFT_STEP
// is stored as exp(x + SHIFT_STEP * sh) (sh = the shift count, kept in a byte
// beside it, at most SHIFT_MAX) and stands for that value times
// exp(-SHIFT_STEP * sh). Scores formed from such weights then rank as the
// float64 ones do.
constexpr double SHIFT_STEP = 80.0;
constexpr int SHIFT_MAX = 9;

__device__ __forceinline__ float exp_shifted(double x, int &sh) {
  sh = 0;
  if (x >= -SHIFT_STEP) return exp_split(x);
  if (!(x > -1.0e30)) return 0.0f;
  sh = min(SHIFT_MAX, int(-x * (1.0 / SHIFT_STEP)));
  return exp_split(x + SHIFT_STEP * double(sh));
}

// exp(-SHIFT_STEP * sh), the factor a shifted weight stands for.
__device__ __forceinline__ double shift_scale(int sh) { return sh == 0 ? 1.0 : exp(-SHIFT_STEP * double(sh)); }

// Total order key of a float64 value: its bits mapped to an order-preserving
// unsigned integer (-0 folded onto +0). Utilities are ranked on this key of
// their float64 value, then by position.
__device__ __forceinline__ uint64_t orderable_f64(double d) {
  uint64_t b = uint64_t(__double_as_longlong(d));
  if (b == 0x8000000000000000ull) b = 0ull;
  return (b & 0x8000000000000000ull) ? ~b : (b | 0x8000000000000000ull);
}

// (key, position) strictly before (key2, position2).
__device__ __forceinline__ bool key_pos_less(uint64_t k1, uint32_t p1, uint64_t k2, uint32_t p2) {
  return k1 < k2 || (k1 == k2 && p1 < p2);
}

// Total order key of (value, position): float bits mapped to an order-preserving
// unsigned integer (-0 folded onto +0), position in the low 32 bits.
__device__ __forceinline__ uint32_t orderable_f32(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint64_t order_key(float value, uint32_t pos) {
  return (uint64_t(orderable_f32(value)) << 32) | pos;
}

// Workgroup barrier that orders LDS only: global loads and stores in flight
// stay in flight across it (__syncthreads also waits for them). Global memory
// written by one thread and read or rewritten by another needs __syncthreads.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


// Workgroup-wide exclusive scan of small non-negative ints; returns this
// thread's exclusive prefix and writes the total to *total. `red` is LDS of >= 4 ints.
__device__ __forceinline__ int wg_exclusive_scan(int v, int *red, int *total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < WG / 64; ++w) {
    int r = red[w];
    if (w < wave) off += r;
    tot += r;
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

}  // namespace kvc

namespace kvc {

// ---------------------------------------------------------------- transposed group reduction
// A token row is spread over LPT lanes (16 or 32); each lane holds partial dot
// products for the G heads. The reduction halves the head set at each of the
// first log2(G) exchange stages (a lane keeps the half selected by its lane
// bit and sends the other half to its partner), then sums the single
// remaining value over the rest. Every lane ends with the full dot product of
// one head, lane_head<LPT, G>(lane); the stages are DPP row mirrors / quad
// permutes (and a cross-row shuffle for 32-lane rows).
template <int LPT>
__device__ __forceinline__ double xchg_stage(double x, int stage) {
  constexpr int off = LPT == 32 ? 1 : 0;
  if (LPT == 32 && stage == 0) return __shfl_xor(x, 16);
  switch (stage - off) {
    case 0: return dpp_f64<0x140>(x);   // row_mirror: flips lane bit 3 (and bits 0-2)
    case 1: return dpp_f64<0x141>(x);   // row_half_mirror: flips bit 2 (and bits 0-1)
    case 2: return dpp_f64<0x4E>(x);    // quad_perm [2,3,0,1]: flips bit 1
    default: return dpp_f64<0xB1>(x);   // quad_perm [1,0,3,2]: flips bit 0
  }
}

template <int LPT, int N, int STAGE>
__device__ __forceinline__ double treduce(const double (&v)[N], int lane) {
  constexpr int NST = LPT == 32 ? 5 : 4;
  if constexpr (N == 1) {
    double x = v[0];
#pragma unroll
    for (int s = STAGE; s < NST; ++s) x += xchg_stage<LPT>(x, s);
    return x;
  } else {
    constexpr int bit = NST - 1 - STAGE;
    const bool up = (lane >> bit) & 1;
    double w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      const double send = up ? v[i] : v[N / 2 + i];
      const double keep = up ? v[N / 2 + i] : v[i];
      w[i] = keep + xchg_stage<LPT>(send, STAGE);
    }
    return treduce<LPT, N / 2, STAGE + 1>(w, lane);
  }
}

template <int LPT, int G>
__device__ __forceinline__ int lane_head(int lane) {
  constexpr int NST = LPT == 32 ? 5 : 4;
  int h = 0;
#pragma unroll
  for (int s = 0; (1 << s) < G; ++s) h = 2 * h + ((lane >> (NST - 1 - s)) & 1);
  return h;
}

// A lane holding head g's value, and whether this lane is the first of its
// (token, head) group.
template <int LPT, int G>
__device__ __forceinline__ int head_rep_lane(int g) {
  constexpr int NST = LPT == 32 ? 5 : 4;
  int gb = 0;
  while ((1 << gb) < G) ++gb;
  return g << (NST - gb);
}
template <int LPT, int G>
__device__ __forceinline__ bool head_leader(int lane) {
  constexpr int NST = LPT == 32 ? 5 : 4;
  int gb = 0;
  while ((1 << gb) < G) ++gb;
  return (lane & ((1 << (NST - gb)) - 1)) == 0;
}

// ---------------------------------------------- lane-permuted transposed reduction
// Variant of treduce without per-lane selects. Lane l of a token row keeps in
// register slot i the partial sum of head i ^ perm_head(l), where perm_head is
// linear over the lane bits and chosen so that, at each exchange stage, the
// partner lane's upper-half slots hold the heads of this lane's lower-half
// slots; slot i then simply adds the partner's slot N/2 + i. The stages pair
// lanes l and l ^ 16 (32-lane rows only), l ^ 15, l ^ 7, l ^ 2 and l ^ 1, so
// perm_head must map those masks to G/2, G/4, ... for the first log2(G)
// stages and to 0 afterwards; its coefficients below solve exactly that.
template <int G>
__host__ __device__ constexpr int stage_head_bit(int s) {
  return (s < (G >= 8 ? 3 : G >= 4 ? 2 : G >= 2 ? 1 : 0)) ? (G >> (s + 1)) : 0;
}

template <int LPT, int G>
__host__ __device__ constexpr int perm_head(int lane) {
  constexpr int off = LPT == 32 ? 1 : 0;
  const int c0 = stage_head_bit<G>(off + 3);
  const int c1 = stage_head_bit<G>(off + 2);
  const int c2 = stage_head_bit<G>(off + 1) ^ c0 ^ c1;
  const int c3 = stage_head_bit<G>(off) ^ stage_head_bit<G>(off + 1);
  const int c4 = LPT == 32 ? stage_head_bit<G>(0) : 0;
  return ((lane & 1) ? c0 : 0) ^ ((lane & 2) ? c1 : 0) ^ ((lane & 4) ? c2 : 0) ^ ((lane & 8) ? c3 : 0) ^
         ((lane & 16) ? c4 : 0);
}

// First lane of a token row whose reduced value is head g's.
template <int LPT, int G>
__host__ __device__ constexpr int perm_rep_lane(int g) {
  for (int l = 0; l < LPT; ++l)
    if (perm_head<LPT, G>(l) == g) return l;
  return 0;
}

template <int LPT, int N, int STAGE>
__device__ __forceinline__ double preduce(const double (&v)[N]) {
  constexpr int NST = LPT == 32 ? 5 : 4;
  if constexpr (N == 1) {
    double x = v[0];
#pragma unroll
    for (int s = STAGE; s < NST; ++s) x += xchg_stage<LPT>(x, s);
    return x;
  } else {
    double w[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[i] = v[i] + xchg_stage<LPT>(v[N / 2 + i], STAGE);
    return preduce<LPT, N / 2, STAGE + 1>(w);
  }
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
  return __hiloint2double(hi, lo);
}

}  // namespace kvc
