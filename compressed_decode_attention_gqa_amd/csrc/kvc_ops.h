// Workgroup-level selection, moment fold and compaction, shared by the fused
// decode step and the standalone entry points. One workgroup (256 threads)
// owns one scope while it runs these.
#pragma once

#include "kvc_device.h"

namespace kvc {

// ============================================================ selection
// Evicted set of size k among n entries under the total order of the 64-bit
// keys: (orderable float bits << 32) | position, ascending (InertiaKV §3.1:
// lowest utility first; ties to the lower position). Result: slot i is
// evicted iff (key(i) & mask) < thr, or (key(i) & mask) == thr and i is among
// the first `take_eq` such slots in ascending slot order.
struct SelectCut {
  uint64_t thr, mask;
  int take_eq, n_eq;
};

struct SelectLds {
  uint32_t hist[256];
  int red[8];
  uint64_t wmin[4];
  int wslot[4];
};

// Radix select of the k-th smallest key (1 <= k <= n), 8 bits per pass from
// the top; stops as soon as the bin holding the k-th key is taken whole.
template <class KeyFn>
__device__ SelectCut wg_select_cut(KeyFn key, int n, int k, SelectLds &sh) {
  const int tid = threadIdx.x;
  uint64_t prefix = 0, hmask = 0;
  int krem = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    sh.hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += WG) {
      uint64_t kk = key(i);
      if ((kk & hmask) == prefix) atomicAdd(&sh.hist[(kk >> shift) & 255u], 1u);
    }
    __syncthreads();
    const int c = int(sh.hist[tid]);
    int tot;
    const int excl = wg_exclusive_scan(c, sh.red, &tot);
    if (excl < krem && krem <= excl + c) {
      sh.red[4] = tid;
      sh.red[5] = krem - excl;
      sh.red[6] = c;
    }
    __syncthreads();
    const int digit = sh.red[4];
    krem = sh.red[5];
    const int cnt = sh.red[6];
    __syncthreads();
    prefix |= uint64_t(digit) << shift;
    hmask |= uint64_t(255) << shift;
    if (cnt == krem || shift == 0) return SelectCut{prefix, hmask, krem, cnt};
  }
  return SelectCut{prefix, hmask, krem, krem};  // not reached
}

// Writes flags[i] (u8) for i < n from the cut, optionally a second copy, and
// appends the evicted slots (ascending) to list. Returns the evicted count.
template <class KeyFn>
__device__ int wg_apply_cut(KeyFn key, int n, const SelectCut &cut, uint8_t *flags,
                            uint8_t *flags2, int32_t *list, SelectLds &sh) {
  const int tid = threadIdx.x;
  int eq_seen = 0, out_seen = 0;
  for (int base = 0; base < n; base += WG) {
    const int i = base + tid;
    bool lt = false, eq = false;
    if (i < n) {
      const uint64_t km = key(i) & cut.mask;
      lt = km < cut.thr;
      eq = km == cut.thr;
    }
    int eq_tot;
    const int eq_rank = eq_seen + wg_exclusive_scan(eq ? 1 : 0, sh.red, &eq_tot);
    const bool ev = lt || (eq && eq_rank < cut.take_eq);
    int ev_tot;
    const int ev_rank = out_seen + wg_exclusive_scan(ev ? 1 : 0, sh.red, &ev_tot);
    if (i < n) {
      if (flags) flags[i] = ev ? 1 : 0;
      if (flags2) flags2[i] = ev ? 1 : 0;
      if (ev && list) list[ev_rank] = i;
    }
    eq_seen += eq_tot;
    out_seen += ev_tot;
  }
  return out_seen;
}

// The k lowest (value, position) of n entries with float64 values (1 <= k <= n):
// a radix cut on the order key of the values; if the cut's bin holds equal
// values beyond the ones it must give up, a second cut on those entries'
// positions decides. Writes flags (and flags2) and the evicted slots
// ascending to list; returns the evicted count.
template <class ValFn, class PosFn>
__device__ int wg_select_f64_pos(ValFn val, PosFn pos, int n, int k, uint8_t *flags, uint8_t *flags2,
                                 int32_t *list, SelectLds &sh) {
  auto key = [&](int i) -> uint64_t { return orderable_f64(val(i)); };
  const SelectCut cut = wg_select_cut(key, n, k, sh);
  if (cut.take_eq == cut.n_eq) return wg_apply_cut(key, n, cut, flags, flags2, list, sh);
  auto tied = [&](int i) -> uint64_t {
    return (key(i) & cut.mask) == cut.thr ? uint64_t(uint32_t(pos(i))) : ~0ull;
  };
  const SelectCut cut2 = wg_select_cut(tied, n, cut.take_eq, sh);   // distinct positions
  auto evicted = [&](int i) -> uint64_t {
    const uint64_t km = key(i) & cut.mask;
    if (km < cut.thr) return 0ull;
    return (km == cut.thr && (tied(i) & cut2.mask) <= cut2.thr) ? 0ull : 1ull;
  };
  return wg_apply_cut(evicted, n, SelectCut{1ull, ~0ull, 0, 0}, flags, flags2, list, sh);
}

// argmin of key over [0, n): returns the slot (lowest slot among equal keys).
__device__ __forceinline__ int wg_argmin_finish(uint64_t best, int slot, SelectLds &sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint64_t b2 = shfl_xor_u64(best, o);
    int s2 = __shfl_xor(slot, o);
    if (b2 < best || (b2 == best && uint32_t(s2) < uint32_t(slot))) {
      best = b2;
      slot = s2;
    }
  }
  if (lane == 0) {
    sh.wmin[wave] = best;
    sh.wslot[wave] = slot;
  }
  __syncthreads();
  uint64_t b = sh.wmin[0];
  int s = sh.wslot[0];
#pragma unroll
  for (int w = 1; w < WG / 64; ++w) {
    if (sh.wmin[w] < b || (sh.wmin[w] == b && uint32_t(sh.wslot[w]) < uint32_t(s))) {
      b = sh.wmin[w];
      s = sh.wslot[w];
    }
  }
  __syncthreads();
  return s;
}

// ============================================================ moment fold
// MomentKV §4.1 / Appendix A.1: n += |E|, s_k += sum k_e, s_v += sum v_e,
// S += sum v_e k_e^T. Thread t owns the float4 columns 4*(t%32).. of S rows
// t/32 + 8j (j = 0..15); evicted rows are staged in LDS 16 at a time.
constexpr int FOLD_BATCH = 16;

struct FoldLds {
  float kb[FOLD_BATCH][HD];
  float vb[FOLD_BATCH][HD];
  int32_t slots[WG];
  int red[8];
};

struct FoldAcc {
  float s[16][4];
  float ksum, vsum;  // threads 0..127: k element tid; threads 128..255: v element tid-128
};

__device__ __forceinline__ void fold_zero(FoldAcc &f) {
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int c = 0; c < 4; ++c) f.s[j][c] = 0.f;
  f.ksum = f.vsum = 0.f;
}

// Fold `cnt` slots listed in sh.slots (LDS) of the unit whose rows start at Kb/Vb.
template <typename T>
__device__ void fold_slots(FoldAcc &f, const T *Kb, const T *Vb, int cnt, FoldLds &sh) {
  const int tid = threadIdx.x;
  const int col = 4 * (tid & 31), row0 = tid >> 5;
  for (int b0 = 0; b0 < cnt; b0 += FOLD_BATCH) {
    const int nb = min(FOLD_BATCH, cnt - b0);
    for (int idx = tid; idx < nb * HD; idx += WG) {
      const int e = idx / HD, c = idx - (idx / HD) * HD;
      const int64_t r = int64_t(sh.slots[b0 + e]) * HD + c;
      sh.kb[e][c] = load_elem<T>(Kb, r);
      sh.vb[e][c] = load_elem<T>(Vb, r);
    }
    __syncthreads();
    for (int e = 0; e < nb; ++e) {
      const float4 k4 = *reinterpret_cast<const float4 *>(&sh.kb[e][col]);
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float va = sh.vb[e][row0 + 8 * j];
        f.s[j][0] = fmaf(va, k4.x, f.s[j][0]);
        f.s[j][1] = fmaf(va, k4.y, f.s[j][1]);
        f.s[j][2] = fmaf(va, k4.z, f.s[j][2]);
        f.s[j][3] = fmaf(va, k4.w, f.s[j][3]);
      }
      if (tid < HD) f.ksum += sh.kb[e][tid];
      else f.vsum += sh.vb[e][tid - HD];
    }
    __syncthreads();
  }
}

// Add the accumulated fold of `count` tokens into the unit's statistics.
__device__ __forceinline__ void fold_commit(const FoldAcc &f, int count, int32_t *n, float *sk,
                                           float *sv, float *S) {
  const int tid = threadIdx.x;
  const int col = 4 * (tid & 31), row0 = tid >> 5;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float4 *p = reinterpret_cast<float4 *>(S + (row0 + 8 * j) * HD + col);
    float4 x = *p;
    x.x += f.s[j][0];
    x.y += f.s[j][1];
    x.z += f.s[j][2];
    x.w += f.s[j][3];
    *p = x;
  }
  if (tid < HD) sk[tid] += f.ksum;
  else sv[tid - HD] += f.vsum;
  if (tid == 0) *n += count;
}

// Fold every flagged slot in [0, L) (flags: u8 per slot) of one unit.
template <typename T>
__device__ void fold_flagged(const T *Kb, const T *Vb, const uint8_t *flags, int L, int32_t *n,
                             float *sk, float *sv, float *S, FoldLds &sh) {
  FoldAcc f;
  fold_zero(f);
  int total = 0;
  for (int base = 0; base < L; base += WG) {
    const int i = base + threadIdx.x;
    const bool ev = i < L && flags[i];
    int cnt;
    const int r = wg_exclusive_scan(ev ? 1 : 0, sh.red, &cnt);
    if (ev) sh.slots[r] = i;
    __syncthreads();
    if (cnt) fold_slots<T>(f, Kb, Vb, cnt, sh);
    total += cnt;
    __syncthreads();
  }
  if (total) fold_commit(f, total, n, sk, sv, S);
}

// ============================================================ compaction
// Hole-filling: with new length B = L - k, the j-th evicted slot below B
// receives the j-th surviving slot at or above B (ascending order).
struct ScopeRows {
  char *k, *v;              // cache base pointers
  int64_t row0;             // first row of unit 0 of this scope
  int64_t unit_stride;      // rows between units
  int units;
  int row_bytes;
  int32_t *votes, *pos;     // scope arrays (already offset), votes may be null
  float *m;                 // may be null
};

// Copy slot src -> dst for every unit and the scope arrays; called by one thread.
__device__ __forceinline__ void move_slot_thread(const ScopeRows &r, int src, int dst) {
  const int nv = r.row_bytes / 16;
  for (int u = 0; u < r.units; ++u) {
    const int64_t base = (r.row0 + int64_t(u) * r.unit_stride) * r.row_bytes;
    char *ks = r.k + base + int64_t(src) * r.row_bytes, *kd = r.k + base + int64_t(dst) * r.row_bytes;
    char *vs = r.v + base + int64_t(src) * r.row_bytes, *vd = r.v + base + int64_t(dst) * r.row_bytes;
    for (int c = 0; c < nv; ++c) {
      st16(kd + 16 * c, ld16(ks + 16 * c));
      st16(vd + 16 * c, ld16(vs + 16 * c));
    }
  }
  if (r.votes) r.votes[dst] = r.votes[src];
  r.pos[dst] = r.pos[src];
  if (r.m) r.m[dst] = r.m[src];
}

// Copy the 16-byte vectors of one K row and one V row per unit with the whole
// workgroup: vector i of unit u from (ksrc, vsrc)(u) to (kdst, vdst)(u), byte
// offsets given per unit by the callables. Each thread issues up to COPY_BATCH
// K and V loads before it stores any, so a copy over many units waits on memory
// once per batch instead of once per vector.
constexpr int COPY_BATCH = 8;
template <int BATCH = COPY_BATCH, class Src, class Dst>
__device__ __forceinline__ void copy_rows_wg(int units, int nv, Src src, Dst dst) {
  constexpr int COPY_BATCH = BATCH;
  const int total = units * nv;
  for (int base = 0; base < total; base += COPY_BATCH * WG) {
    u32x4 kx[COPY_BATCH], vx[COPY_BATCH];
#pragma unroll
    for (int b = 0; b < COPY_BATCH; ++b) {
      const int idx = base + b * WG + int(threadIdx.x);
      if (idx < total) {
        const int u = idx / nv, c = idx - (idx / nv) * nv;
        const char *ks, *vs;
        src(u, ks, vs);
        kx[b] = ld16(ks + 16 * c);
        vx[b] = ld16(vs + 16 * c);
      }
    }
#pragma unroll
    for (int b = 0; b < COPY_BATCH; ++b) {
      const int idx = base + b * WG + int(threadIdx.x);
      if (idx < total) {
        const int u = idx / nv, c = idx - (idx / nv) * nv;
        char *kd, *vd;
        dst(u, kd, vd);
        st16(kd + 16 * c, kx[b]);
        st16(vd + 16 * c, vx[b]);
      }
    }
  }
}

// Copy slot src -> dst with the whole workgroup (one pair of slots).
template <int BATCH = COPY_BATCH>
__device__ __forceinline__ void move_slot_wg(const ScopeRows &r, int src, int dst) {
  copy_rows_wg<BATCH>(
      r.units, r.row_bytes / 16,
      [&](int u, const char *&ks, const char *&vs) {
        const int64_t off = ((r.row0 + int64_t(u) * r.unit_stride) + src) * r.row_bytes;
        ks = r.k + off;
        vs = r.v + off;
      },
      [&](int u, char *&kd, char *&vd) {
        const int64_t off = ((r.row0 + int64_t(u) * r.unit_stride) + dst) * r.row_bytes;
        kd = r.k + off;
        vd = r.v + off;
      });
  if (threadIdx.x == 0) {
    if (r.votes) r.votes[dst] = r.votes[src];
    r.pos[dst] = r.pos[src];
    if (r.m) r.m[dst] = r.m[src];
  }
}

// Hole-filling for a general evicted set; `holes` is scratch of >= L ints.
__device__ void wg_compact_flags(const ScopeRows &r, const uint8_t *flags, int L, int k,
                                 int32_t *holes, int *red) {
  const int B = L - k;
  int seen = 0;
  for (int base = 0; base < B; base += WG) {
    const int i = base + threadIdx.x;
    const bool hole = i < B && flags[i];
    int tot;
    const int rk = seen + wg_exclusive_scan(hole ? 1 : 0, red, &tot);
    if (hole) holes[rk] = i;
    seen += tot;
  }
  __syncthreads();
  seen = 0;
  for (int base = B; base < L; base += WG) {
    const int i = base + threadIdx.x;
    const bool mover = i < L && !flags[i];
    int tot;
    const int rk = seen + wg_exclusive_scan(mover ? 1 : 0, red, &tot);
    if (mover) move_slot_thread(r, i, holes[rk]);
    seen += tot;
  }
}

}  // namespace kvc
