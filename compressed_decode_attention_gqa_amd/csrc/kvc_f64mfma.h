// A 128 x 128 float64 operator applied to 16-token tiles of 128-element rows on
// v_mfma_f64_16x16x4 (gfx950, wave64), for the path's float64 contractions:
// MomentKV's moment residual A k_j and LaProx's v_i M v_i^T.
//
// Lane layout of v_mfma_f64_16x16x4: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] and receives D[l / 16 + 4 r][l % 16], r = 0..3.
//
// z_j = X y_j for the 16 tokens j of a tile (y_j: a 128-element row). The
// contraction index b and the output index a are both permuted so that a lane
// reads 64 contiguous bytes of its token's row: at MFMA step s (0..31) lane
// group g = l / 16 carries b = 32 g + s, and output row i of row tile rt (0..7)
// is a = 32 (i % 4) + 4 rt + i / 4. The accumulator values a lane holds
// (i = g + 4 r) are then a = 32 g + 4 rt + r: the same elements [32 g, 32 g + 32)
// of its row as its B values. X is kept in LDS fragment by fragment (128 KB),
// each 64-lane fragment pair under an XOR swizzle.
#pragma once

#include "kvc_device.h"

namespace kvc {

typedef double fm_d4 __attribute__((ext_vector_type(4)));
typedef double fm_d2 __attribute__((ext_vector_type(2)));

constexpr int FM_TILE = 16;   // tokens per wave tile (MFMA N)
constexpr int FM_RT = 8;      // 16-row tiles of the 128 output rows
constexpr int FM_S2 = 16;     // pairs of MFMA k-steps (32 steps of 4)

struct FmOperator {
  fm_d2 a[FM_S2][FM_RT][64];
};

// Swizzled position of lane l's fragment pair for pair-step s2: a bijection on
// 0..63 that keeps each 16-lane phase of a read on distinct 16-byte bank groups
// and spreads the staging writes.
__device__ __forceinline__ int fm_swz(int s2, int l) { return l ^ (((s2 >> 1) ^ ((l >> 4) << 2)) & 15); }

// Store X[a][b] in its fragment slot.
__device__ __forceinline__ void fm_put(FmOperator &op, int a, int b, double v) {
  const int i = (a >> 5) + 4 * (a & 3), rt = (a & 31) >> 2, g = b >> 5, s = b & 31;
  op.a[s >> 1][rt][fm_swz(s >> 1, i + 16 * g)][s & 1] = v;
}

// acc[rt][r] += (X y)[32 g + 4 rt + r], with x[s] = y[32 g + s] the lane's B values.
__device__ __forceinline__ void fm_apply(const FmOperator &op, int lane, const double (&x)[32],
                                         fm_d4 (&acc)[FM_RT]) {
#pragma unroll
  for (int s2 = 0; s2 < FM_S2; ++s2) {
    fm_d2 af[FM_RT];
    const int pl = fm_swz(s2, lane);
#pragma unroll
    for (int rt = 0; rt < FM_RT; ++rt) af[rt] = op.a[s2][rt][pl];
#pragma unroll
    for (int rt = 0; rt < FM_RT; ++rt)
      acc[rt] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[rt].x, x[2 * s2], acc[rt], 0, 0, 0);
#pragma unroll
    for (int rt = 0; rt < FM_RT; ++rt)
      acc[rt] = __builtin_amdgcn_mfma_f64_16x16x4f64(af[rt].y, x[2 * s2 + 1], acc[rt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The transposed use: X as the B operand, the tokens' rows as the A operand.
// D[i][j] = sum_b y_i[b] X[16 ct + j][b] lands in lane l as
// acc[ct][r] = (X y_{l / 16 + 4 r})[16 ct + l % 16]: each lane holds 8 rows of X
// (one per column tile ct) for 4 tokens, and its A values x[s] = y_{l % 16}[32 g + s].
__device__ __forceinline__ void fm_put_t(FmOperator &op, int a, int b, double v) {
  const int ct = a >> 4, j = a & 15, g = b >> 5, s = b & 31;
  op.a[s >> 1][ct][fm_swz(s >> 1, j + 16 * g)][s & 1] = v;
}

// NCT < 8 uses only the operator's first NCT column tiles (rows 0 .. 16 NCT - 1).
template <int NCT = FM_RT>
__device__ __forceinline__ void fm_apply_t(const FmOperator &op, int lane, const double (&x)[32],
                                           fm_d4 (&acc)[NCT]) {
#pragma unroll
  for (int s2 = 0; s2 < FM_S2; ++s2) {
    fm_d2 bf[NCT];
    const int pl = fm_swz(s2, lane);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) bf[ct] = op.a[s2][ct][pl];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(x[2 * s2], bf[ct].x, acc[ct], 0, 0, 0);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
      acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(x[2 * s2 + 1], bf[ct].y, acc[ct], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// 32 consecutive elements of a row in the cache dtype (64 or 128 bytes).
template <typename T>
struct FmRow;
template <>
struct FmRow<bf16_t> {
  u32x4 w[4];
  __device__ __forceinline__ void load(const char *base) {
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = ld16(base + 16 * q);
  }
  __device__ __forceinline__ double get(int e) const { return double(ElemTraits<bf16_t>::get(w[e >> 3], e & 7)); }
};
template <>
struct FmRow<float> {
  u32x4 w[8];
  __device__ __forceinline__ void load(const char *base) {
#pragma unroll
    for (int q = 0; q < 8; ++q) w[q] = ld16(base + 16 * q);
  }
  __device__ __forceinline__ double get(int e) const { return double(ElemTraits<float>::get(w[e >> 2], e & 3)); }
};

}  // namespace kvc
