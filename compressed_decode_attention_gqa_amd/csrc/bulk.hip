// Device-wide eviction of k > 1 entries per scope (the first, bulk step that
// compresses a prefilled cache down to its budget, or any step whose scopes
// are far over budget). The epilogue kernels have already written the outputs,
// the new utilities and the appended row; these kernels finish the step over
// the whole grid instead of one workgroup per scope:
//
//   hist, pick x 8   radix select of the k lowest (utility, position) keys:
//              per pass a 256-bin histogram of each chunk's keys under the
//              current prefix, then one workgroup per scope sums the chunks and
//              picks the digit (InertiaKV §3.1: lowest utility first, ties to
//              the lower position). The fused step ranks float64 utilities: 8
//              passes over their 64-bit order key, then (only if equal values
//              straddle the cut) 4 passes over the positions of the tied entries
//   flags      evicted flags and per-chunk counts of evicted slots and movers
//   lists      evicted slots ascending; survivors at or above L - k ascending
//   fold       MomentKV §4.1 / Appendix A.1 moment sums of the evicted rows,
//              split over several workgroups per unit, partials summed in a
//              fixed order by a reduce kernel
//   move       hole filling: mover j goes to evicted slot j (the evicted slots
//              below L - k come first in the ascending list), then len = L - k
//
// (key, position) pairs are distinct because live positions are distinct, so
// the final cut takes its bin whole: slot i is evicted iff (hi & mask) <
// prefix, or (hi & mask) == prefix and (lo & lmask) <= lprefix, where hi is the
// 64-bit key and lo the tie key (lmask = 0 when the 64-bit keys decided).
#include "kvc_decode.h"
#include "kvc_device.h"
#include "kvc_kernels.h"

namespace kvc {

namespace {

constexpr int FOLD_NB = 16;                     // evicted rows staged per batch
constexpr int PART_STRIDE = HD * HD + 2 * HD;   // floats per fold partial: S, s_k, s_v

struct SlotKey {
  uint64_t hi;   // the 64-bit key
  uint32_t lo;   // tie key of equal 64-bit keys (positions; 0 when hi holds the position)
};

__device__ __forceinline__ SlotKey slot_key(const BulkArgs &b, int64_t sc, int i) {
  const uint32_t p = b.pos ? uint32_t(b.pos[sc + i]) : uint32_t(i);
  if (b.key64) return SlotKey{orderable_f64(b.key64[sc + i]), p};
  if (!b.protect) return SlotKey{order_key(b.key[sc + i], p), 0u};
  // (protected, value, position) in 1 + 32 + 31 bits: positions are non-negative int32
  const uint64_t prot = int32_t(p) >= b.protect_from ? 1ull : 0ull;
  return SlotKey{(prot << 63) | (uint64_t(orderable_f32(b.key[sc + i])) << 31) | uint64_t(p & 0x7fffffffu), 0u};
}

// ------------------------------------------------------------ standalone set-up
// Selection of the k = L - budget lowest keys of every scope (L = len or cap).
__global__ __launch_bounds__(WG) void k_bulk_sel_init(const BulkArgs b) {
  const int scope = blockIdx.x * WG + threadIdx.x;
  if (scope >= b.n_scopes) return;
  const int L = b.len ? min(b.len[scope], b.cap) : b.cap;
  const int k = max(0, L - b.budget);
  BulkScope &st = b.st[scope];
  st.prefix = 0;
  st.mask = 0;
  st.lprefix = 0;
  st.lmask = 0;
  st.krem = k;
  st.done = k == 0 ? 1 : 0;
  st.L = L;
  st.k = k;
  st.B = L - k;
  st.n_pairs = 0;
  st.run = 1;
  if (b.n_evict) b.n_evict[scope] = k;
}

// Given evicted flags: the live length of every scope; k and B follow from the counts.
__global__ __launch_bounds__(WG) void k_bulk_len_init(const BulkArgs b) {
  const int scope = blockIdx.x * WG + threadIdx.x;
  if (scope >= b.n_scopes) return;
  BulkScope &st = b.st[scope];
  st.L = b.len ? min(b.len[scope], b.cap) : b.cap;
  st.k = 0;
  st.B = st.L;
  st.n_pairs = 0;
  st.run = 1;
}

// Per chunk: flagged slots below L.
__global__ __launch_bounds__(WG) void k_bulk_count(const BulkArgs b) {
  __shared__ int red[8];
  const int scope = blockIdx.y, tid = threadIdx.x;
  const BulkScope &st = b.st[scope];
  if (!st.run) return;
  const int64_t sc = int64_t(scope) * b.cap;
  const int i0 = blockIdx.x * b.chunk, i1 = min(st.L, i0 + b.chunk);
  int n = 0;
  for (int i = i0 + tid; i < i1; i += WG) n += b.flags[sc + i] ? 1 : 0;
  int tot;
  wg_exclusive_scan(n, red, &tot);
  if (tid == 0) b.cnt[(int64_t(scope) * b.n_chunks + blockIdx.x) * 2] = tot;
}

// One workgroup per scope: k = sum of the chunk counts; B = L - k when the
// evicted slots are to be removed (compact), L when they are only folded.
__global__ __launch_bounds__(WG) void k_bulk_total(const BulkArgs b, const int compact) {
  __shared__ int red[8];
  const int scope = blockIdx.x, tid = threadIdx.x;
  BulkScope &st = b.st[scope];
  if (!st.run) return;
  int n = 0;
  for (int c = tid; c < b.n_chunks; c += WG) n += b.cnt[(int64_t(scope) * b.n_chunks + c) * 2];
  int tot;
  wg_exclusive_scan(n, red, &tot);
  if (tid == 0) {
    st.k = tot;
    st.B = compact ? st.L - tot : st.L;
    if (tot == 0) st.run = 0;
  }
}

// Per chunk: survivors at or above B (they fill the holes below B).
__global__ __launch_bounds__(WG) void k_bulk_movers(const BulkArgs b) {
  __shared__ int red[8];
  const int scope = blockIdx.y, tid = threadIdx.x;
  const BulkScope &st = b.st[scope];
  if (!st.run) return;
  const int64_t sc = int64_t(scope) * b.cap;
  const int i0 = max(st.B, int(blockIdx.x) * b.chunk), i1 = min(st.L, int(blockIdx.x) * b.chunk + b.chunk);
  int n = 0;
  for (int i = i0 + tid; i < i1; i += WG) n += b.flags[sc + i] ? 0 : 1;
  int tot;
  wg_exclusive_scan(n, red, &tot);
  if (tid == 0) b.cnt[(int64_t(scope) * b.n_chunks + blockIdx.x) * 2 + 1] = tot;
}

// ------------------------------------------------------------ radix select pass
// Each workgroup histograms the digit at `shift` of the keys of its chunk that
// match the current prefix and stores the 256 counts (plain stores: no
// device-scope atomics or fences); the pick kernel sums the chunks' counts.
// Phase 0 takes digits of the 64-bit key, phase 1 of the tie key among the
// entries whose 64-bit key equals the whole prefix.
__global__ __launch_bounds__(WG) void k_bulk_hist(const BulkArgs b, const int shift, const int phase) {
  __shared__ uint32_t hist[256];
  const int scope = blockIdx.y, tid = threadIdx.x;
  const BulkScope &st = b.st[scope];
  if (!st.run || st.done) return;     // the same for every workgroup of the scope
  const int L = st.L;
  const uint64_t prefix = st.prefix, mask = st.mask;
  const uint32_t lprefix = st.lprefix, lmask = st.lmask;
  hist[tid] = 0u;
  __syncthreads();
  const int64_t sc = int64_t(scope) * b.cap;
  const int i0 = blockIdx.x * b.chunk, i1 = min(L, i0 + b.chunk);
  const int lane = tid & 63;
  for (int base = i0; base < i1; base += WG) {
    const int i = base + tid;
    uint32_t bin = 0;
    bool hit = false;
    if (i < i1) {
      const SlotKey key = slot_key(b, sc, i);
      if (phase == 0) {
        hit = (key.hi & mask) == prefix;
        bin = uint32_t(key.hi >> shift) & 255u;
      } else {
        hit = key.hi == prefix && (key.lo & lmask) == lprefix;
        bin = (key.lo >> shift) & 255u;
      }
    }
    // Keys crowd into a few bins in the leading passes (utilities share their
    // exponent): the wave first adds the counts of up to two shared bins with
    // one atomic each, then the remaining lanes add one by one.
    uint64_t rem = __ballot(hit);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (!rem) break;
      const int first = __builtin_ctzll(rem);
      const uint32_t b0 = __shfl(bin, first);
      const uint64_t same = __ballot(hit && bin == b0) & rem;
      if (lane == first) atomicAdd(&hist[b0], uint32_t(__popcll(same)));
      rem &= ~same;
    }
    if ((rem >> lane) & 1ull) atomicAdd(&hist[bin], 1u);
  }
  __syncthreads();
  b.hpart[(int64_t(scope) * b.n_chunks + blockIdx.x) * 256 + tid] = hist[tid];
}

// One workgroup per scope: the bin holding the krem-th key under the prefix.
__global__ __launch_bounds__(WG) void k_bulk_pick(const BulkArgs b, const int shift, const int phase) {
  __shared__ int red[8];
  const int scope = blockIdx.x, tid = threadIdx.x;
  BulkScope &st = b.st[scope];
  if (!st.run || st.done) return;
  const int krem = st.krem;
  const uint32_t *h = b.hpart + int64_t(scope) * b.n_chunks * 256;
  int cnt = 0;
  for (int c = 0; c < b.n_chunks; ++c) cnt += int(h[c * 256 + tid]);
  int tot;
  const int excl = wg_exclusive_scan(cnt, red, &tot);
  if (excl < krem && krem <= excl + cnt) {
    if (phase == 0) {
      st.prefix |= uint64_t(tid) << shift;
      st.mask |= uint64_t(255) << shift;
    } else {
      st.lprefix |= uint32_t(tid) << shift;
      st.lmask |= 255u << shift;
    }
    st.krem = krem - excl;
    // the last digit of the deciding key: float keys carry the position, float64
    // keys hand equal values on to the position passes
    const bool last = shift == 0 && (phase == 1 || b.key64 == nullptr);
    if (cnt == krem - excl || last) st.done = 1;
  }
}

// ------------------------------------------------------------ flags and chunk counts
__global__ __launch_bounds__(WG) void k_bulk_flags(const BulkArgs b) {
  __shared__ int red[8];
  const int scope = blockIdx.y, tid = threadIdx.x;
  const BulkScope &st = b.st[scope];
  if (!st.run) return;
  const int L = st.L, B = st.B;
  const bool any = st.k > 0;
  const uint64_t prefix = st.prefix, mask = st.mask;
  const uint32_t lprefix = st.lprefix, lmask = st.lmask;
  const int64_t sc = int64_t(scope) * b.cap;
  const int i0 = blockIdx.x * b.chunk, i1 = min(L, i0 + b.chunk);
  int n_ev = 0, n_mv = 0;
  for (int i = i0 + tid; i < i1; i += WG) {
    const SlotKey key = slot_key(b, sc, i);
    const uint64_t km = key.hi & mask;
    const bool ev = any && (km < prefix || (km == prefix && (key.lo & lmask) <= lprefix));
    if (b.flags) b.flags[sc + i] = ev ? 1 : 0;
    if (b.flags2) b.flags2[sc + i] = ev ? 1 : 0;
    n_ev += ev ? 1 : 0;
    n_mv += (!ev && i >= B) ? 1 : 0;
  }
  int te, tm;
  wg_exclusive_scan(n_ev, red, &te);
  wg_exclusive_scan(n_mv, red, &tm);
  if (tid == 0) {
    int32_t *c = b.cnt + (int64_t(scope) * b.n_chunks + blockIdx.x) * 2;
    c[0] = te;
    c[1] = tm;
  }
}

// ------------------------------------------------------------ evicted and mover lists
// b.list: evicted slots ascending (k entries); b.list2: movers (survivors at or above B) ascending.
__global__ __launch_bounds__(WG) void k_bulk_lists(const BulkArgs b) {
  __shared__ int red[8];
  const int scope = blockIdx.y, tid = threadIdx.x;
  BulkScope &st = b.st[scope];
  if (!st.run) return;
  const int L = st.L, B = st.B;
  const int64_t sc = int64_t(scope) * b.cap;
  // bases: counts of the chunks before this one (n_chunks <= 256)
  int pe = 0, pm = 0;
  if (tid < int(blockIdx.x)) {
    const int32_t *c = b.cnt + (int64_t(scope) * b.n_chunks + tid) * 2;
    pe = c[0];
    pm = c[1];
  }
  int te, tm;
  wg_exclusive_scan(pe, red, &te);
  wg_exclusive_scan(pm, red, &tm);
  int base_e = te, base_m = tm;
  const int i0 = blockIdx.x * b.chunk, i1 = min(L, i0 + b.chunk);
  for (int base = i0; base < i1; base += WG) {
    const int i = base + tid;
    const bool ev = i < i1 && b.flags[sc + i];
    const bool mv = i < i1 && !ev && i >= B;
    int tot;
    const int r = wg_exclusive_scan((ev ? 1 : 0) | ((mv ? 1 : 0) << 16), red, &tot);
    if (ev) b.list[sc + base_e + (r & 0xffff)] = i;
    if (mv) b.list2[sc + base_m + (r >> 16)] = i;
    base_e += tot & 0xffff;
    base_m += tot >> 16;
  }
  if (blockIdx.x == gridDim.x - 1 && tid == 0) st.n_pairs = base_m;
}

// ------------------------------------------------------------ moment fold
// Workgroup f of a unit folds evicted-list entries [f*per, (f+1)*per). Thread t
// owns S rows {4r..4r+3, 64+4r..64+4r+3} x columns {4c..4c+3, 64+4c..64+4c+3}
// (r = t/16, c = t%16): per evicted row it reads 8 values of v and 8 of k from
// LDS (16-byte reads, consecutive lanes on consecutive addresses) for 64 fp32
// FMAs. Rows are staged 16 at a time, fp32 in LDS, double-buffered: the global
// loads of batch j+1 are in flight while batch j is folded.
struct BulkFoldLds {
  float kb[2][FOLD_NB][HD];
  float vb[2][FOLD_NB][HD];
  int32_t slots[WG];
};

template <typename T>
struct FoldStage {
  static constexpr int EPV = ElemTraits<T>::EPV;        // elements per 16 bytes
  static constexpr int CPR = HD / EPV;                  // 16-byte chunks per row
  static constexpr int NLD = FOLD_NB * CPR / WG;        // chunks per thread per matrix
};

template <typename T>
__device__ __forceinline__ void fold_load(u32x4 (&rk)[FoldStage<T>::NLD], u32x4 (&rv)[FoldStage<T>::NLD],
                                          const char *Kb, const char *Vb, const int32_t *slots, int e0,
                                          int ne) {
  using FS = FoldStage<T>;
#pragma unroll
  for (int h = 0; h < FS::NLD; ++h) {
    const int q = threadIdx.x + WG * h, e = q / FS::CPR, c = q % FS::CPR;
    if (e < ne) {
      const int64_t off = int64_t(slots[e0 + e]) * (HD * int64_t(sizeof(T))) + 16 * c;
      rk[h] = ld16(Kb + off);
      rv[h] = ld16(Vb + off);
    } else {
      rk[h] = u32x4(0u);
      rv[h] = u32x4(0u);
    }
  }
}

template <typename T>
__device__ __forceinline__ void fold_stage(const u32x4 (&rk)[FoldStage<T>::NLD],
                                           const u32x4 (&rv)[FoldStage<T>::NLD], float (*kb)[HD],
                                           float (*vb)[HD]) {
  using FS = FoldStage<T>;
  using TR = ElemTraits<T>;
#pragma unroll
  for (int h = 0; h < FS::NLD; ++h) {
    const int q = threadIdx.x + WG * h, e = q / FS::CPR, c = q % FS::CPR;
#pragma unroll
    for (int j = 0; j < FS::EPV; j += 4) {
      *reinterpret_cast<float4 *>(&kb[e][c * FS::EPV + j]) =
          make_float4(TR::get(rk[h], j), TR::get(rk[h], j + 1), TR::get(rk[h], j + 2), TR::get(rk[h], j + 3));
      *reinterpret_cast<float4 *>(&vb[e][c * FS::EPV + j]) =
          make_float4(TR::get(rv[h], j), TR::get(rv[h], j + 1), TR::get(rv[h], j + 2), TR::get(rv[h], j + 3));
    }
  }
}

template <typename T>
__global__ __launch_bounds__(WG) void k_bulk_fold(const StepArgs a, const BulkArgs b) {
  using FS = FoldStage<T>;
  __shared__ BulkFoldLds sh;
  const int tid = threadIdx.x;
  const int scope = blockIdx.y / a.units, u = blockIdx.y - scope * a.units;
  const BulkScope &st = b.st[scope];
  if (!st.run || st.k <= 0) return;
  const int k = st.k;
  const int per = (k + b.fold_splits - 1) / b.fold_splits;
  const int j0 = min(k, int(blockIdx.x) * per), j1 = min(k, j0 + per);
  const int64_t sc = int64_t(scope) * a.capacity;
  const int64_t row0 = int64_t(scope) * a.scope_stride + int64_t(u) * a.unit_stride;
  const char *Kb = a.k + row0 * (HD * int64_t(sizeof(T)));
  const char *Vb = a.v + row0 * (HD * int64_t(sizeof(T)));
  const int r4 = 4 * (tid >> 4), c4 = 4 * (tid & 15);

  float acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  float lin = 0.f;   // threads < HD: s_k element tid; others: s_v element tid - HD

  for (int w0 = j0; w0 < j1; w0 += WG) {
    const int nw = min(WG, j1 - w0);
    if (tid < nw) sh.slots[tid] = b.list[sc + w0 + tid];
    __syncthreads();
    const int nb = (nw + FOLD_NB - 1) / FOLD_NB;
    u32x4 rk[FS::NLD], rv[FS::NLD];
    fold_load<T>(rk, rv, Kb, Vb, sh.slots, 0, min(FOLD_NB, nw));
    for (int bt = 0; bt < nb; ++bt) {
      const int buf = bt & 1;
      const int ne = min(FOLD_NB, nw - bt * FOLD_NB);
      fold_stage<T>(rk, rv, sh.kb[buf], sh.vb[buf]);
      __syncthreads();
      if (bt + 1 < nb)
        fold_load<T>(rk, rv, Kb, Vb, sh.slots, (bt + 1) * FOLD_NB, min(FOLD_NB, nw - (bt + 1) * FOLD_NB));
      const float(*kb)[HD] = sh.kb[buf];
      const float(*vb)[HD] = sh.vb[buf];
#pragma unroll 2
      for (int e = 0; e < ne; ++e) {
        const float4 va = *reinterpret_cast<const float4 *>(&vb[e][r4]);
        const float4 vc = *reinterpret_cast<const float4 *>(&vb[e][64 + r4]);
        const float4 ka = *reinterpret_cast<const float4 *>(&kb[e][c4]);
        const float4 kc = *reinterpret_cast<const float4 *>(&kb[e][64 + c4]);
        const float vv[8] = {va.x, va.y, va.z, va.w, vc.x, vc.y, vc.z, vc.w};
        const float kk[8] = {ka.x, ka.y, ka.z, ka.w, kc.x, kc.y, kc.z, kc.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[i][j] = fmaf(vv[i], kk[j], acc[i][j]);
        lin += tid < HD ? kb[e][tid] : vb[e][tid - HD];
      }
    }
    __syncthreads();
  }

  // partial (or, with one split, the moment sums themselves)
  const int64_t mu = blockIdx.y;
  const bool direct = b.fold_splits == 1;
  float *S = direct ? a.mom_S + mu * HD * HD
                    : b.fpart + (int64_t(blockIdx.y) * b.fold_splits + blockIdx.x) * PART_STRIDE;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = i < 4 ? r4 + i : 64 + r4 + (i - 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float4 *p = reinterpret_cast<float4 *>(S + row * HD + (h ? 64 + c4 : c4));
      float4 x = make_float4(acc[i][4 * h], acc[i][4 * h + 1], acc[i][4 * h + 2], acc[i][4 * h + 3]);
      if (direct) {
        const float4 o = *p;
        x.x += o.x;
        x.y += o.y;
        x.z += o.z;
        x.w += o.w;
      }
      *p = x;
    }
  }
  if (direct) {
    if (tid < HD) a.mom_sk[mu * HD + tid] += lin;
    else a.mom_sv[mu * HD + tid - HD] += lin;
    if (tid == 0) a.mom_n[mu] += k;
  } else {
    S[HD * HD + tid] = lin;   // s_k then s_v
  }
}

// bf16 caches: the same fold on MFMA. S = V_E^T K_E is a d x k x d contraction
// over the evicted rows, so each stage of 32 rows is one 16x16x32 bf16 MFMA
// reduction step; the operands are the cache's own bf16 values, their products
// are exact in fp32 and the accumulation is fp32, as on the VALU. Wave w owns
// the 64 x 64 quadrant (rows 64*(w/2).., columns 64*(w%2)..) as 4 x 4 tiles.
// Rows are staged row-major in LDS with a 264-byte stride, so the eight
// 2-byte reads that build a fragment (rows 8g..8g+7 of one column for the four
// lane groups g) fall on distinct banks. s_v and s_k come from two more MFMAs
// per tile row / column with a fragment of ones (waves of the first quadrant
// column and row).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

constexpr int MF_ROWS = 32;   // evicted rows per stage: the MFMA reduction depth
constexpr int MF_RS = 132;    // LDS row stride, bf16 elements
constexpr int MF_WIN = 1024;  // evicted-list entries staged in LDS per window

struct MfmaFoldLds {
  uint16_t kr[2][MF_ROWS][MF_RS];
  uint16_t vr[2][MF_ROWS][MF_RS];
  int32_t slots[MF_WIN];
};

// Stage rows e0.. of the window: chunk q = tid + 256 h is row q / 16, 16-byte chunk q % 16.
// Rows past ne load row e0 again (every load unconditional, so the loads of the
// next stage stay in flight) and are zeroed when staged.
__device__ __forceinline__ void mf_load(u32x4 (&rk)[2], u32x4 (&rv)[2], const char *Kb, const char *Vb,
                                        const int32_t *slots, int e0, int ne) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = threadIdx.x + WG * h, e = q >> 4, c = q & 15;
    const int64_t off = int64_t(slots[e0 + (e < ne ? e : 0)]) * (HD * 2) + 16 * c;
    // read once (the evicted rows of a whole prompt): non-temporal
    rk[h] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)(Kb + off));
    rv[h] = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4 *)(Vb + off));
  }
}

__device__ __forceinline__ void mf_stage(const u32x4 (&rk)[2], const u32x4 (&rv)[2], int ne,
                                         uint16_t (*kr)[MF_RS], uint16_t (*vr)[MF_RS]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int q = threadIdx.x + WG * h, e = q >> 4, c = q & 15;
    const u32x4 zk = e < ne ? rk[h] : u32x4(0u), zv = e < ne ? rv[h] : u32x4(0u);
    uint2 *pk = reinterpret_cast<uint2 *>(&kr[e][8 * c]);
    uint2 *pv = reinterpret_cast<uint2 *>(&vr[e][8 * c]);
    pk[0] = make_uint2(zk.x, zk.y);
    pk[1] = make_uint2(zk.z, zk.w);
    pv[0] = make_uint2(zv.x, zv.y);
    pv[1] = make_uint2(zv.z, zv.w);
  }
}

// Fragment of column `col` over rows 8g..8g+7 of a staged matrix.
__device__ __forceinline__ bf16x8 mf_frag(const uint16_t (*m)[MF_RS], int g, int col) {
  u16x8 x;
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = m[8 * g + e][col];
  return __builtin_bit_cast(bf16x8, x);
}

// Accumulators of one workgroup's MFMA fold: wave w owns the 64 x 64 quadrant
// of S at rows 64*(w/2), columns 64*(w%2) as 4 x 4 tiles; accv / acck collect
// s_v / s_k.
struct MfmaAcc {
  f32x4 acc[4][4], accv[4], acck[4];
};

__device__ __forceinline__ void mf_zero(MfmaAcc &f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.accv[i] = f32x4(0.f);
    f.acck[i] = f32x4(0.f);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.acc[i][j] = f32x4(0.f);
  }
}

// Fold the nw rows whose slots are in sh.slots[0, nw) (unit rows at Kb, Vb).
__device__ __forceinline__ void mf_window(MfmaAcc &f, MfmaFoldLds &sh, const int nw, const char *Kb,
                                          const char *Vb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int iq = wave >> 1, jq = wave & 1, g = lane >> 4, l16 = lane & 15;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u16x8(uint16_t(0x3f80)));
  const int nst = (nw + MF_ROWS - 1) / MF_ROWS;
  // two stages of loads in flight: stage s is staged from register set s & 1,
  // which then takes the loads of stage s + 2
  u32x4 rk[2][2], rv[2][2];
  // (loads past the last stage repeat it, so every step issues the same loads and
  // the waits stay exact: stage s waits only for its own set)
  auto load_stage = [&](int s, u32x4 (&qk)[2], u32x4 (&qv)[2]) {
    s = min(s, nst - 1);
    mf_load(qk, qv, Kb, Vb, sh.slots, s * MF_ROWS, min(MF_ROWS, nw - s * MF_ROWS));
  };
  load_stage(0, rk[0], rv[0]);
  __builtin_amdgcn_sched_barrier(0);
  load_stage(1, rk[1], rv[1]);
  __builtin_amdgcn_sched_barrier(0);
  auto step = [&](const int s, u32x4 (&qk)[2], u32x4 (&qv)[2]) {
    const int buf = s & 1;
    mf_stage(qk, qv, min(MF_ROWS, nw - s * MF_ROWS), sh.kr[buf], sh.vr[buf]);
    __syncthreads();
    load_stage(s + 2, qk, qv);
    __builtin_amdgcn_sched_barrier(0);   // keep the next loads ahead of this stage's MFMAs
    bf16x8 af[4], bf[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      af[t] = mf_frag(sh.vr[buf], g, 64 * iq + 16 * t + l16);
      bf[t] = mf_frag(sh.kr[buf], g, 64 * jq + 16 * t + l16);
    }
#pragma unroll
    for (int ti = 0; ti < 4; ++ti)
#pragma unroll
      for (int tj = 0; tj < 4; ++tj)
        f.acc[ti][tj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ti], bf[tj], f.acc[ti][tj], 0, 0, 0);
    // (every wave forms both sums, branch-free; only one quadrant row / column stores them)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f.accv[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[t], ones, f.accv[t], 0, 0, 0);
      f.acck[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, bf[t], f.acck[t], 0, 0, 0);
    }
  };
  int s = 0;
  for (; s + 1 < nst; s += 2) {   // straight-line body: the same loads pending on every trip
    step(s, rk[0], rv[0]);
    step(s + 1, rk[1], rv[1]);
  }
  if (s < nst) step(s, rk[0], rv[0]);
  __syncthreads();
}

// Store (ADD false) or add (ADD true) the sums: S row-major, then s_k, s_v.
// D layout of a 16x16 tile: lane l holds rows 4(l/16)..+3, column l%16.
template <bool ADD>
__device__ __forceinline__ void mf_commit(const MfmaAcc &f, float *S, float *skd, float *svd) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int iq = wave >> 1, jq = wave & 1, g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int ti = 0; ti < 4; ++ti)
#pragma unroll
    for (int tj = 0; tj < 4; ++tj)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float *p = S + (64 * iq + 16 * ti + 4 * g + r) * HD + 64 * jq + 16 * tj + l16;
        *p = ADD ? *p + f.acc[ti][tj][r] : f.acc[ti][tj][r];
      }
  if (jq == 0 && l16 == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float *p = svd + 64 * iq + 16 * t + 4 * g + r;
        *p = ADD ? *p + f.accv[t][r] : f.accv[t][r];
      }
  }
  if (iq == 0 && g == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float *p = skd + 64 * jq + 16 * t + l16;
      *p = ADD ? *p + f.acck[t][0] : f.acck[t][0];
    }
  }
}

// Workgroup f of a unit folds evicted-list entries [f*per, (f+1)*per).
__global__ __launch_bounds__(WG, 2) void k_bulk_fold_mfma(const StepArgs a, const BulkArgs b) {
  __shared__ MfmaFoldLds sh;
  const int tid = threadIdx.x;
  const int scope = blockIdx.y / a.units, u = blockIdx.y - scope * a.units;
  const BulkScope &st = b.st[scope];
  if (!st.run || st.k <= 0) return;
  const int k = st.k;
  const int per = (k + b.fold_splits - 1) / b.fold_splits;
  const int j0 = min(k, int(blockIdx.x) * per), j1 = min(k, j0 + per);
  const int64_t sc = int64_t(scope) * a.capacity;
  const int64_t row0 = int64_t(scope) * a.scope_stride + int64_t(u) * a.unit_stride;
  const char *Kb = a.k + row0 * (HD * 2);
  const char *Vb = a.v + row0 * (HD * 2);
  MfmaAcc f;
  mf_zero(f);
  for (int w0 = j0; w0 < j1; w0 += MF_WIN) {
    const int nw = min(MF_WIN, j1 - w0);
    for (int e = tid; e < nw; e += WG) sh.slots[e] = b.list[sc + w0 + e];
    __syncthreads();
    mf_window(f, sh, nw, Kb, Vb);
  }
  const int64_t mu = blockIdx.y;
  if (b.fold_splits == 1) {
    mf_commit<true>(f, a.mom_S + mu * HD * HD, a.mom_sk + mu * HD, a.mom_sv + mu * HD);
    if (tid == 0) a.mom_n[mu] += k;
  } else {
    float *P = b.fpart + (int64_t(blockIdx.y) * b.fold_splits + blockIdx.x) * PART_STRIDE;
    mf_commit<false>(f, P, P + HD * HD, P + HD * HD + HD);
  }
}

// kvc_moment_update on bf16 caches: one workgroup per unit folds every flagged
// slot below the scope's length, the slots gathered window by window from the
// flags (no workspace).
__global__ __launch_bounds__(WG, 2) void k_moment_update_mfma(const CacheArgs c, const uint8_t *evict, int32_t *n,
                                                          float *sk, float *sv, float *S) {
  __shared__ MfmaFoldLds sh;
  __shared__ int red[8];
  const int tid = threadIdx.x;
  const int scope = blockIdx.x / c.units, u = blockIdx.x - scope * c.units;
  const int L = min(c.len[scope], c.capacity);
  const uint8_t *fl = evict + int64_t(scope) * c.capacity;
  const int64_t row0 = int64_t(scope) * c.scope_stride + int64_t(u) * c.unit_stride;
  const char *Kb = c.k + row0 * (HD * 2);
  const char *Vb = c.v + row0 * (HD * 2);
  constexpr int PER = MF_WIN / WG;   // slots a thread examines per window
  MfmaAcc f;
  mf_zero(f);
  int total = 0;
  for (int w0 = 0; w0 < L; w0 += MF_WIN) {
    bool hit[PER];
    int cnt = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = w0 + tid * PER + r;
      hit[r] = i < L && fl[i];
      cnt += hit[r] ? 1 : 0;
    }
    int nw;
    int at = wg_exclusive_scan(cnt, red, &nw);
#pragma unroll
    for (int r = 0; r < PER; ++r)
      if (hit[r]) sh.slots[at++] = w0 + tid * PER + r;
    __syncthreads();
    if (nw > 0) mf_window(f, sh, nw, Kb, Vb);
    total += nw;
  }
  if (total == 0) return;
  const int64_t mu = blockIdx.x;
  mf_commit<true>(f, S + mu * HD * HD, sk + mu * HD, sv + mu * HD);
  if (tid == 0) n[mu] += total;
}

// Sum of a unit's fold partials in split order, added to its moment sums.
__global__ __launch_bounds__(WG) void k_bulk_fold_reduce(const StepArgs a, const BulkArgs b) {
  const int tid = threadIdx.x;
  const int scope = blockIdx.x / a.units;
  const BulkScope &st = b.st[scope];
  if (!st.run || st.k <= 0) return;
  const int64_t mu = blockIdx.x;
  const float *P = b.fpart + mu * b.fold_splits * PART_STRIDE;
  constexpr int N4 = PART_STRIDE / 4;
  const int per = (N4 + gridDim.y - 1) / gridDim.y;
  const int q0 = blockIdx.y * per, q1 = min(N4, q0 + per);
  for (int q = q0 + tid; q < q1; q += WG) {
    float4 s = reinterpret_cast<const float4 *>(P)[q];
    for (int f = 1; f < b.fold_splits; ++f) {
      const float4 x = reinterpret_cast<const float4 *>(P + int64_t(f) * PART_STRIDE)[q];
      s.x += x.x;
      s.y += x.y;
      s.z += x.z;
      s.w += x.w;
    }
    float4 *dst = q < HD * HD / 4 ? reinterpret_cast<float4 *>(a.mom_S + mu * HD * HD) + q
                  : q < HD * HD / 4 + HD / 4
                      ? reinterpret_cast<float4 *>(a.mom_sk + mu * HD) + (q - HD * HD / 4)
                      : reinterpret_cast<float4 *>(a.mom_sv + mu * HD) + (q - HD * HD / 4 - HD / 4);
    float4 o = *dst;
    o.x += s.x;
    o.y += s.y;
    o.z += s.z;
    o.w += s.w;
    *dst = o;
  }
  if (blockIdx.y == 0 && tid == 0) a.mom_n[mu] += st.k;
}

// ------------------------------------------------------------ hole-filling moves
__global__ __launch_bounds__(WG) void k_bulk_move(const StepArgs a, const BulkArgs b, const int row_bytes) {
  const int scope = blockIdx.y, tid = threadIdx.x;
  const BulkScope &st = b.st[scope];
  if (!st.run) return;
  const int np = st.n_pairs;
  const int64_t sc = int64_t(scope) * a.capacity;
  const int cpr = row_bytes / 16;
  const int64_t items = int64_t(np) * a.units * 2 * cpr;
  for (int64_t idx = int64_t(blockIdx.x) * WG + tid; idx < items; idx += int64_t(gridDim.x) * WG) {
    const int c = int(idx % cpr);
    int64_t rest = idx / cpr;
    const int kv = int(rest & 1);
    rest >>= 1;
    const int u = int(rest % a.units);
    const int j = int(rest / a.units);
    const int src = b.list2[sc + j], dst = b.list[sc + j];
    char *base = (kv ? a.v : a.k) + (int64_t(scope) * a.scope_stride + int64_t(u) * a.unit_stride) * row_bytes;
    st16(base + int64_t(dst) * row_bytes + 16 * c, ld16(base + int64_t(src) * row_bytes + 16 * c));
  }
  for (int j = blockIdx.x * WG + tid; j < np; j += gridDim.x * WG) {
    const int src = b.list2[sc + j], dst = b.list[sc + j];
    if (a.votes) a.votes[sc + dst] = a.votes[sc + src];
    a.pos[sc + dst] = a.pos[sc + src];
    if (a.m) a.m[sc + dst] = a.m[sc + src];
  }
  if (blockIdx.x == 0 && tid == 0) a.len[scope] = st.L - st.k;
}

}  // namespace

static void launch_radix(const BulkArgs &b, hipStream_t st) {
  const dim3 chunks(b.n_chunks, b.n_scopes);
  for (int shift = 56; shift >= 0; shift -= 8) {
    hipLaunchKernelGGL(k_bulk_hist, chunks, dim3(WG), 0, st, b, shift, 0);
    hipLaunchKernelGGL(k_bulk_pick, dim3(b.n_scopes), dim3(WG), 0, st, b, shift, 0);
  }
  if (b.key64) {   // positions of equal float64 keys (the kernels return at once once done)
    for (int shift = 24; shift >= 0; shift -= 8) {
      hipLaunchKernelGGL(k_bulk_hist, chunks, dim3(WG), 0, st, b, shift, 1);
      hipLaunchKernelGGL(k_bulk_pick, dim3(b.n_scopes), dim3(WG), 0, st, b, shift, 1);
    }
  }
  hipLaunchKernelGGL(k_bulk_flags, chunks, dim3(WG), 0, st, b);
}

hipError_t launch_bulk(const StepArgs &a, const BulkArgs &b, int dtype, hipStream_t st) {
  const dim3 chunks(b.n_chunks, a.n_scopes);
  const int row_bytes = HD * (dtype == 0 ? 2 : 4);
  launch_radix(b, st);
  hipLaunchKernelGGL(k_bulk_lists, chunks, dim3(WG), 0, st, b);
  if (a.mom_S) {
    const dim3 fg(b.fold_splits, a.n_scopes * a.units);
    if (dtype == 0) hipLaunchKernelGGL(k_bulk_fold_mfma, fg, dim3(WG), 0, st, a, b);
    else hipLaunchKernelGGL(k_bulk_fold<float>, fg, dim3(WG), 0, st, a, b);
    if (b.fold_splits > 1)
      hipLaunchKernelGGL(k_bulk_fold_reduce, dim3(a.n_scopes * a.units, 4), dim3(WG), 0, st, a, b);
  }
  hipLaunchKernelGGL(k_bulk_move, dim3(b.move_blocks, a.n_scopes), dim3(WG), 0, st, a, b, row_bytes);
  return hipGetLastError();
}

// kvc_select_evict over many scopes: the radix select above for every scope.
hipError_t launch_bulk_select(const BulkArgs &b, hipStream_t st) {
  hipLaunchKernelGGL(k_bulk_sel_init, dim3((b.n_scopes + WG - 1) / WG), dim3(WG), 0, st, b);
  launch_radix(b, st);
  return hipGetLastError();
}

// kvc_compact (drop) from given flags: counts, lists and moves over the grid.
hipError_t launch_bulk_compact(const StepArgs &a, const BulkArgs &b, int dtype, hipStream_t st) {
  const dim3 chunks(b.n_chunks, b.n_scopes);
  hipLaunchKernelGGL(k_bulk_len_init, dim3((b.n_scopes + WG - 1) / WG), dim3(WG), 0, st, b);
  hipLaunchKernelGGL(k_bulk_count, chunks, dim3(WG), 0, st, b);
  hipLaunchKernelGGL(k_bulk_total, dim3(b.n_scopes), dim3(WG), 0, st, b, 1);
  hipLaunchKernelGGL(k_bulk_movers, chunks, dim3(WG), 0, st, b);
  hipLaunchKernelGGL(k_bulk_lists, chunks, dim3(WG), 0, st, b);
  hipLaunchKernelGGL(k_bulk_move, dim3(b.move_blocks, b.n_scopes), dim3(WG), 0, st, a, b, HD * (dtype == 0 ? 2 : 4));
  return hipGetLastError();
}

// kvc_moment_update on bf16 caches: one workgroup per unit on MFMA.
hipError_t launch_moment_update_mfma(const CacheArgs &c, const uint8_t *evict, int32_t *n, float *sk, float *sv,
                                     float *S, hipStream_t st) {
  hipLaunchKernelGGL(k_moment_update_mfma, dim3(c.n_scopes * c.units), dim3(WG), 0, st, c, evict, n, sk, sv, S);
  return hipGetLastError();
}

size_t bulk_part_floats() { return size_t(PART_STRIDE); }

}  // namespace kvc
