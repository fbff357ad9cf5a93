// C ABI of libkvc: argument validation, workspace layout and kernel dispatch.
// Every check runs on the host before anything is enqueued, so a call that
// returns an error has touched no device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "kvc.h"
#include "kvc_decode.h"
#include "kvc_groups.h"
#include "kvc_kernels.h"
#include "kvc_laprox.h"

namespace {

constexpr int kHD = 128;
constexpr int kTargetWorkgroups = 2048;   // workgroups per launch to aim for (bulk chunks, moves)
constexpr int kSplitWorkgroups = 256;     // split-K attention workgroups (512 threads) per launch
constexpr int kMinSubChunksPerSplit = 16;
constexpr int kMaxSubChunksPerSplit = 512;
// Epilogue score chunks: about kScoreWork (token, head) weights per workgroup,
// at least kScoreChunkMin tokens (the factor cache of a chunk then fits in LDS).
constexpr int kScoreWork = 2048;
constexpr int kScoreChunkMin = 64;
constexpr int kMergeSplitsMax = 64;
// Cosine-pass ranges: about two workgroups per CU in one round, so each wave's two batches of
// key loads stay in flight through a long range (2048 workgroups in two rounds took 25.5 us at
// 64 heads x 6554 slots, 512 in one 20.2 us, 256 20.8 us).
constexpr int kMergeWorkgroups = 512;
static_assert(kMergeSplitsMax <= 64, "k_merge_finish reads one range partner per lane of one wave");
// One workgroup per scope (no split-K) once there are this many single-unit
// scopes to spread over the 256 CUs, each scope's live length is bounded so
// its per-token state fits in LDS, and a step evicts at most one entry.
constexpr int kUnitMinScopes = 128;
// With fewer scopes the single launch still wins while one workgroup streams
// its scope's rows (about 25 GB/s per CU) faster than the split path's three
// dependent launches finish: up to this many K and V bytes per scope.
constexpr int64_t kUnitFewScopesMaxBytes = 256 << 10;
// Bulk eviction (k > 1): fold workgroups per launch to aim for, and the most per unit.
constexpr int kFoldWorkgroups = 1024;
constexpr int kFoldSplitsMax = 64;

// LDS a workgroup may allocate on the current device (160 KB on gfx950).
size_t device_lds_per_block() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 0;
  return size_t(v);
}

inline size_t align_up(size_t x, size_t a = 256) { return (x + a - 1) / a * a; }
inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int ceil_div(int64_t a, int64_t b) { return int((a + b - 1) / b); }

int validate_cache(const kvc_cache *c) {
  if (!c || !c->k || !c->v || !c->pos || !c->len) return KVC_ERR_ARG;
  if (c->dtype != KVC_BF16 && c->dtype != KVC_F32) return KVC_ERR_DTYPE;
  if (c->head_dim != kHD) return KVC_ERR_UNSUPPORTED;
  if (c->capacity <= 0 || c->n_scopes <= 0 || c->units_per_scope <= 0) return KVC_ERR_ARG;
  if (c->scope_stride < 0 || c->unit_stride < 0) return KVC_ERR_ARG;
  if (c->units_per_scope > 1 && c->unit_stride < c->capacity) return KVC_ERR_ARG;
  if (c->n_scopes > 1 && c->scope_stride < int64_t(c->capacity)) return KVC_ERR_ARG;
  if (!aligned16(c->k) || !aligned16(c->v)) return KVC_ERR_ALIGN;
  return KVC_OK;
}

bool valid_G(int G) { return G == 1 || G == 2 || G == 4 || G == 8; }

// ------------------------------------------------------------ decode workspace
struct DecodeLayout {
  int n_splits, nsub_cap, merge_splits;
  int bulk_chunks, bulk_chunk, fold_splits, move_blocks;
  size_t status, partM, partZ, partO, fac, subM, ews, ewsh, m64, flags, list, list2, cand_key, cand_slot, cand_pos;
  int n_score_chunks;
  size_t merge_cos, merge_slot, bulk_state, bulk_cnt, bulk_hist, fpart, steplen, total;
};

// Split-K workgroups per attention unit: one round of workgroups over the CUs
// (kSplitWorkgroups, one 512-thread workgroup per CU), more when a split would
// stream over kMaxSubChunksPerSplit sub-chunks (a shorter tail), and never so
// many that a split streams fewer than kMinSubChunksPerSplit (two per wave at
// the deepest prefetch) and its loads cannot stay in flight.
int split_count(int attn_units_total, int nsub) {
  const int want = std::max(ceil_div(kSplitWorkgroups, attn_units_total), ceil_div(nsub, kMaxSubChunksPerSplit));
  const int most = std::max(1, nsub / kMinSubChunksPerSplit);
  return std::max(1, std::min(want, most));
}

// Slot chunks per scope of the grid-wide select / count / list kernels: about
// kTargetWorkgroups per launch, at most 256 per scope, whole multiples of 256 slots.
void bulk_chunking(int n_scopes, int capacity, int &n_chunks, int &chunk) {
  n_chunks = std::max(1, std::min({ceil_div(kTargetWorkgroups, n_scopes), 256, ceil_div(capacity, 256)}));
  chunk = ceil_div(ceil_div(capacity, n_chunks), 256) * 256;
}

// Workspace of the grid-wide select (and compaction): per-scope state, chunk
// histograms and chunk counts.
struct SelectLayout {
  int n_chunks, chunk;
  size_t state, hist, cnt, total;
};

SelectLayout select_layout(int n_scopes, int capacity, size_t base = 0) {
  SelectLayout l{};
  bulk_chunking(n_scopes, capacity, l.n_chunks, l.chunk);
  size_t o = base;
  l.state = o; o = align_up(o + size_t(n_scopes) * sizeof(kvc::BulkScope));
  l.hist = o;  o = align_up(o + size_t(n_scopes) * l.n_chunks * 256 * 4);
  l.cnt = o;   o = align_up(o + size_t(n_scopes) * l.n_chunks * 8);
  l.total = o;
  return l;
}

DecodeLayout decode_layout(const kvc_cache *c, int G, int attn_units) {
  DecodeLayout d{};
  const int CH = kvc::decode_chunk_tokens(c->dtype);
  const int64_t nu = int64_t(c->n_scopes) * attn_units;
  const int CHW = kvc::decode_unit_chunk_tokens(c->dtype);
  d.nsub_cap = ceil_div(c->capacity, std::min(CH, CHW));
  d.n_splits = split_count(int(nu), ceil_div(c->capacity, CH));
  d.merge_splits = std::max(1, std::min(kMergeSplitsMax, ceil_div(kMergeWorkgroups, c->n_scopes)));
  // bulk eviction: slot chunks per scope (<= 256), fold splits per unit, move blocks per scope
  bulk_chunking(c->n_scopes, c->capacity, d.bulk_chunks, d.bulk_chunk);
  const int64_t units_total = int64_t(c->n_scopes) * c->units_per_scope;
  d.fold_splits = int(std::max<int64_t>(1, std::min<int64_t>(kFoldSplitsMax, (kFoldWorkgroups + units_total - 1) / units_total)));
  d.move_blocks = std::max(1, std::min(64, ceil_div(kTargetWorkgroups, c->n_scopes)));
  const int64_t cap = c->capacity;
  size_t o = 0;
  d.status = o;   o = align_up(o + 256);
  d.partM = o;    o = align_up(o + size_t(nu) * d.n_splits * G * 8);
  d.partZ = o;    o = align_up(o + size_t(nu) * d.n_splits * G * 8);
  d.partO = o;    o = align_up(o + size_t(nu) * d.n_splits * G * kHD * 4);
  d.fac = o;      o = align_up(o + size_t(nu) * d.n_splits * G * 4);
  d.subM = o;     o = align_up(o + size_t(nu) * d.nsub_cap * G * 8);
  d.ews = o;      o = align_up(o + size_t(nu) * G * cap * 4);
  d.ewsh = o;     o = align_up(o + size_t(nu) * G * cap);
  d.m64 = o;      o = align_up(o + size_t(c->n_scopes) * cap * 8);
  d.flags = o;    o = align_up(o + size_t(c->n_scopes) * cap);
  d.list = o;     o = align_up(o + size_t(c->n_scopes) * cap * 4);
  d.list2 = o;    o = align_up(o + size_t(c->n_scopes) * cap * 4);
  d.merge_cos = o;  o = align_up(o + size_t(c->n_scopes) * d.merge_splits * 8);
  d.merge_slot = o; o = align_up(o + size_t(c->n_scopes) * d.merge_splits * 8);
  d.n_score_chunks = ceil_div(c->capacity, kScoreChunkMin);
  d.cand_key = o;   o = align_up(o + size_t(c->n_scopes) * d.n_score_chunks * 8);
  d.cand_slot = o;  o = align_up(o + size_t(c->n_scopes) * d.n_score_chunks * 4);
  d.cand_pos = o;   o = align_up(o + size_t(c->n_scopes) * d.n_score_chunks * 4);
  d.bulk_state = o; o = align_up(o + size_t(c->n_scopes) * sizeof(kvc::BulkScope));
  d.steplen = o;    o = align_up(o + size_t(c->n_scopes) * 4);
  d.bulk_cnt = o;   o = align_up(o + size_t(c->n_scopes) * d.bulk_chunks * 8);
  d.bulk_hist = o;  o = align_up(o + size_t(c->n_scopes) * d.bulk_chunks * 256 * 4);
  d.fpart = o;
  if (d.fold_splits > 1) o = align_up(o + size_t(units_total) * d.fold_splits * kvc::bulk_part_floats() * 4);
  d.total = o;
  return d;
}

template <typename P>
P *at(void *ws, size_t off) { return reinterpret_cast<P *>(static_cast<char *>(ws) + off); }

kvc::CacheArgs cache_args(const kvc_cache *c) {
  kvc::CacheArgs a{};
  a.k = static_cast<char *>(c->k);
  a.v = static_cast<char *>(c->v);
  a.votes = c->votes;
  a.pos = c->pos;
  a.m = c->m;
  a.len = c->len;
  a.scope_stride = c->scope_stride;
  a.unit_stride = c->unit_stride;
  a.dtype = c->dtype;
  a.capacity = c->capacity;
  a.n_scopes = c->n_scopes;
  a.units = c->units_per_scope;
  return a;
}

// The kernels a decode call runs (max_len already resolved, > 0): the per-scope
// kernel for steady steps of single-unit scopes whose per-token state fits in
// LDS, once there are enough scopes to spread over the CUs or each scope's rows
// are few; otherwise split-K attention with the score/finish kernels, plus the
// bulk kernels when a step without merge may evict more than one entry per
// scope (mode: 0 attend and score, 1 step, 2 step with merge).
int decode_plan(const kvc_cache *c, int G, int mode, int budget, int max_len) {
  const bool steady = mode == 0 || int64_t(max_len) <= int64_t(budget) + 1;
  const int64_t scope_bytes = 2 * int64_t(max_len) * kHD * (c->dtype == KVC_BF16 ? 2 : 4);
  if (c->units_per_scope == 1 && steady &&
      (c->n_scopes >= kUnitMinScopes || scope_bytes <= kUnitFewScopesMaxBytes) &&
      kvc::decode_unit_lds_bytes(c->dtype, G, max_len, c->votes != nullptr) <= device_lds_per_block())
    return KVC_PLAN_ONE_LAUNCH;
  return (mode == 1 && !steady) ? KVC_PLAN_SPLIT_BULK : KVC_PLAN_SPLIT;
}

int run_decode(const kvc_cache *c, const void *k_new, const void *v_new, int32_t t, const void *q,
               int32_t G, float scale, int mode, int rule, float alpha, int budget, int refresh,
               float *out, float *lse, float *s, const kvc_moments *mom, const kvc_merge *merge,
               uint8_t *evict_out, int attn_unit0, int attn_units, int32_t max_len, void *ws,
               size_t ws_bytes, void *stream, int32_t *status_out = nullptr) {
  int st = validate_cache(c);
  if (st) return st;
  if (!valid_G(G)) return KVC_ERR_UNSUPPORTED;
  if (!q || !out || !lse) return KVC_ERR_ARG;
  if ((k_new == nullptr) != (v_new == nullptr)) return KVC_ERR_ARG;
  if (!aligned16(q) || (k_new && (!aligned16(k_new) || !aligned16(v_new)))) return KVC_ERR_ALIGN;
  if (attn_units <= 0) {
    attn_unit0 = 0;
    attn_units = c->units_per_scope;
  }
  if (attn_unit0 < 0 || attn_unit0 + attn_units > c->units_per_scope) return KVC_ERR_ARG;
  if (attn_units * G > 64) return KVC_ERR_UNSUPPORTED;
  if (max_len > c->capacity) return KVC_ERR_CAPACITY;
  if (max_len <= 0) max_len = c->capacity;
  if (mode != 0) {
    if (!c->m) return KVC_ERR_ARG;
    if (budget < 0) return KVC_ERR_CAPACITY;
    if (rule < KVC_RULE_SINGLE || rule > KVC_RULE_EMA) return KVC_ERR_ARG;
    if (mom && (!mom->n || !mom->sk || !mom->sv || !mom->S)) return KVC_ERR_ARG;
    if (merge) {
      if (!merge->q || !aligned16(merge->q) || !valid_G(merge->G) || !c->votes) return KVC_ERR_ARG;
      if (c->units_per_scope != 1 || mom) return KVC_ERR_UNSUPPORTED;
    }
  } else if (!c->m && k_new) {
    return KVC_ERR_ARG;
  }
  if (!ws) return KVC_ERR_WORKSPACE;
  const DecodeLayout d = decode_layout(c, G, attn_units);
  if (ws_bytes < d.total) return KVC_ERR_WORKSPACE;

  kvc::StepArgs a{};
  a.k = static_cast<char *>(c->k);
  a.v = static_cast<char *>(c->v);
  a.votes = c->votes;
  a.pos = c->pos;
  a.m = c->m;
  a.len = c->len;
  a.scope_stride = c->scope_stride;
  a.unit_stride = c->unit_stride;
  a.capacity = c->capacity;
  a.n_scopes = c->n_scopes;
  a.units = c->units_per_scope;
  a.attn_unit0 = attn_unit0;
  a.attn_units = attn_units;
  a.k_new = static_cast<const char *>(k_new);
  a.v_new = static_cast<const char *>(v_new);
  a.t = t;
  a.append = k_new ? 1 : 0;
  a.q = static_cast<const char *>(q);
  a.scale = double(scale);
  a.out = out;
  a.lse = lse;
  a.s = s;
  a.mode = (mode != 0 && merge) ? 2 : mode;
  a.rule = rule;
  a.budget = budget;
  a.refresh = mode == 0 ? 1 : (refresh ? 1 : 0);
  a.alpha = alpha;
  if (mom) {
    a.mom_n = mom->n;
    a.mom_sk = mom->sk;
    a.mom_sv = mom->sv;
    a.mom_S = mom->S;
  }
  a.evict_out = evict_out;
  a.status = status_out ? status_out : at<int32_t>(ws, d.status);
  a.partM = at<double>(ws, d.partM);
  a.partZ = at<double>(ws, d.partZ);
  a.partO = at<float>(ws, d.partO);
  a.fac = at<float>(ws, d.fac);
  a.subM = at<double>(ws, d.subM);
  a.ews = at<float>(ws, d.ews);
  a.ewsh = at<uint8_t>(ws, d.ewsh);
  a.m64 = at<double>(ws, d.m64);
  a.flags = at<uint8_t>(ws, d.flags);
  a.list = at<int32_t>(ws, d.list);
  a.list2 = at<int32_t>(ws, d.list2);
  a.nsub_cap = d.nsub_cap;
  a.row_bytes = kHD * (c->dtype == KVC_BF16 ? 2 : 4);
  a.max_len = max_len;
  a.n_score_chunks = d.n_score_chunks;
  a.cand_key = at<uint64_t>(ws, d.cand_key);
  a.cand_slot = at<int32_t>(ws, d.cand_slot);
  a.cand_pos = at<int32_t>(ws, d.cand_pos);
  // multi-unit scopes without moments: the hole fill's rows over up to 16 finish
  // workgroups per scope (16 units each at least), with the score kernel's length copy
  a.steplen = at<int32_t>(ws, d.steplen);
  a.fin_blocks = (c->units_per_scope > 1 && !mom) ? std::max(1, std::min(16, c->units_per_scope / 16)) : 1;
  {
    const int heads = attn_units * G;   // <= 64
    const int chunk = std::max(kScoreChunkMin, kScoreWork / heads);
    a.score_chunk = chunk / kScoreChunkMin * kScoreChunkMin;
  }
  const int CH = kvc::decode_chunk_tokens(c->dtype);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int plan = decode_plan(c, G, a.mode, budget, max_len);
  // split path, merge mode, no flags or moments out: the merge kernels select the entry
  a.merge_select = plan != KVC_PLAN_ONE_LAUNCH && a.mode == 2 && !evict_out && !mom ? 1 : 0;
  if (plan == KVC_PLAN_ONE_LAUNCH) {
    a.n_splits = 1;
    a.lds_len = max_len;
    if (kvc::launch_decode_unit(a, c->dtype, G, hs) != hipSuccess) return KVC_ERR_DEVICE;
  } else {
    // a step that may evict more than one entry per scope hands those scopes to
    // the device-wide bulk kernels
    const bool bulk = plan == KVC_PLAN_SPLIT_BULK;
    if (bulk) a.bulk = at<kvc::BulkScope>(ws, d.bulk_state);
    a.n_splits = split_count(c->n_scopes * attn_units, ceil_div(max_len, CH));
    if (kvc::launch_decode(a, c->dtype, G, hs) != hipSuccess) return KVC_ERR_DEVICE;
    if (bulk) {
      kvc::BulkArgs b{};
      b.st = a.bulk;
      b.cnt = at<int32_t>(ws, d.bulk_cnt);
      b.hpart = at<uint32_t>(ws, d.bulk_hist);
      b.fpart = at<float>(ws, d.fpart);
      b.key = c->m;
      b.key64 = a.m64;   // the step ranks float64 utilities
      b.pos = c->pos;
      b.flags = a.flags;
      b.flags2 = evict_out;
      b.list = a.list;
      b.list2 = a.list2;
      b.cap = c->capacity;
      b.n_scopes = c->n_scopes;
      b.n_chunks = d.bulk_chunks;
      b.chunk = d.bulk_chunk;
      b.fold_splits = d.fold_splits;
      b.move_blocks = d.move_blocks;
      if (kvc::launch_bulk(a, b, c->dtype, hs) != hipSuccess) return KVC_ERR_DEVICE;
    }
  }
  if (a.mode == 2) {
    kvc::MergeArgs mg{};
    mg.q = static_cast<const char *>(merge->q);
    mg.G = merge->G;
    mg.scale = double(merge->scale);
    mg.eps = merge->eps;
    mg.n_splits = d.merge_splits;
    mg.e_slot = a.list;               // the epilogue's choice, list[0] of each scope
    mg.e_stride = c->capacity;
    mg.part_cos = at<double>(ws, d.merge_cos);
    mg.part_slot = at<int32_t>(ws, d.merge_slot);
    if (a.merge_select) {
      mg.cand_key = a.cand_key;
      mg.cand_slot = a.cand_slot;
      mg.cand_pos = a.cand_pos;
      mg.n_score_chunks = a.n_score_chunks;
      mg.score_chunk = a.score_chunk;
      mg.append = a.append;
      mg.budget = budget;
      mg.status = a.status;
      mg.cand_max = ceil_div(max_len, a.score_chunk);
    }
    if (kvc::launch_merge(cache_args(c), a.flags, mg, hs) != hipSuccess) return KVC_ERR_DEVICE;
  }
  return KVC_OK;
}

// ------------------------------------------------------------ compact workspace
struct CompactLayout {
  int merge_splits;
  size_t status, list, list2, cos, slot, total;
  SelectLayout sel;
};

CompactLayout compact_layout(const kvc_cache *c) {
  CompactLayout l{};
  l.merge_splits = std::max(1, std::min(kMergeSplitsMax, ceil_div(kMergeWorkgroups, c->n_scopes)));
  size_t o = 0;
  l.status = o;   o = align_up(o + 256);
  l.list = o;     o = align_up(o + size_t(c->n_scopes) * c->capacity * 4);
  l.list2 = o;    o = align_up(o + size_t(c->n_scopes) * c->capacity * 4);
  l.cos = o;      o = align_up(o + size_t(c->n_scopes) * l.merge_splits * 8);
  l.slot = o;     o = align_up(o + size_t(c->n_scopes) * l.merge_splits * 8);
  l.sel = select_layout(c->n_scopes, c->capacity, o);
  l.total = l.sel.total;
  return l;
}

// ------------------------------------------------------- moment-informed eviction
// Candidates per (scope, chunk of at least kMomentTile tokens), after the status word.
constexpr int kMomentTile = 64;
constexpr int kMomentWorkgroups = 256;   // one 128 KB-LDS workgroup per CU

struct MomentEvictLayout {
  size_t status, score, pos, slot, total;
  int n_chunks;
};

MomentEvictLayout moment_evict_layout(int n_scopes, int cap) {
  MomentEvictLayout l{};
  l.n_chunks = ceil_div(cap, kMomentTile);
  size_t o = 0;
  l.status = o; o = align_up(o + 256);
  l.score = o;  o = align_up(o + size_t(n_scopes) * l.n_chunks * 8);
  l.pos = o;    o = align_up(o + size_t(n_scopes) * l.n_chunks * 4);
  l.slot = o;   o = align_up(o + size_t(n_scopes) * l.n_chunks * 4);
  l.total = o;
  return l;
}

// ------------------------------------------------------- KeepKV prefill merging
struct PrefillLayout {
  size_t status, meta, rec, sum, total;
};

PrefillLayout prefill_layout(int n_scopes, int cap) {
  PrefillLayout l{};
  const size_t n = size_t(n_scopes) * cap;
  size_t o = 0;
  l.status = o; o = align_up(o + 256);
  l.meta = o;   o = align_up(o + n * 16);
  l.rec = o;    o = align_up(o + n * 64);
  l.sum = o;    o = align_up(o + n * 32);
  l.total = o;
  return l;
}

// ------------------------------------------------------- allocation-free decode step
// The workspace of kvc_decode_step_noalloc: one array per GPU, part of the loaded
// code object (each device holds its own copy for the life of the process). Host
// code never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, once per device, and is kept in scratch_ptr.
constexpr size_t kScratchBytes = size_t(128) << 20;
__device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
void *scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

// Device address of the current device's scratch array (looked up on the device's first call).
int current_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVC_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KVC_ERR_DEVICE;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return KVC_OK;
}

// kvc_select_evict with an optional protection bound (defined below the C entry points).
int32_t select_evict(const float *key, const int32_t *pos, const int32_t *len, int32_t n_scopes, int32_t capacity,
                     int32_t budget, bool protect, int32_t protect_from, uint8_t *evict, int32_t *n_evict, void *ws,
                     size_t ws_bytes, void *stream);

}  // namespace

extern "C" {

int32_t kvc_version(void) { return KVC_VERSION; }

int32_t kvc_check(void *stream) {
  if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return KVC_ERR_DEVICE;
  return hipGetLastError() == hipSuccess ? KVC_OK : KVC_ERR_DEVICE;
}

const char *kvc_status_string(int32_t s) {
  switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_ARG: return "invalid argument";
    case KVC_ERR_DTYPE: return "unsupported dtype";
    case KVC_ERR_UNSUPPORTED: return "unsupported shape";
    case KVC_ERR_CAPACITY: return "capacity exceeded";
    case KVC_ERR_ALIGN: return "pointer not 16-byte aligned";
    case KVC_ERR_WORKSPACE: return "workspace missing or too small";
    case KVC_ERR_DEVICE: return "device launch failure";
    default: return "unknown status";
  }
}

size_t kvc_decode_workspace_size(const kvc_cache *cache, int32_t G, int32_t max_len) {
  (void)max_len;
  if (validate_cache(cache) || !valid_G(G)) return 0;
  return decode_layout(cache, G, cache->units_per_scope).total;
}

size_t kvc_select_workspace_size(int32_t n_scopes, int32_t capacity) {
  if (n_scopes <= 0 || capacity <= 0) return 0;
  return std::max(align_up(kvc::wide_state_bytes()), select_layout(n_scopes, capacity).total);
}

size_t kvc_compact_workspace_size(const kvc_cache *cache) {
  if (validate_cache(cache)) return 0;
  return compact_layout(cache).total;
}

int32_t kvc_workspace_status(void *ws, void *stream) {
  if (!ws) return KVC_ERR_ARG;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(hs) != hipSuccess) return KVC_ERR_DEVICE;
  int32_t v = 0;
  if (hipMemcpy(&v, ws, 4, hipMemcpyDeviceToHost) != hipSuccess) return KVC_ERR_DEVICE;
  if (v != 0) {
    const int32_t zero = 0;
    if (hipMemcpy(ws, &zero, 4, hipMemcpyHostToDevice) != hipSuccess) return KVC_ERR_DEVICE;
  }
  return v;
}

int32_t kvc_decode_attn_score(const kvc_cache *cache, const void *k_new, const void *v_new, int32_t t,
                              const void *q, int32_t G, float scale, float *out, float *lse, float *s,
                              int32_t max_len, void *ws, size_t ws_bytes, void *stream) {
  return run_decode(cache, k_new, v_new, t, q, G, scale, 0, 0, 0.f, 0, 1, out, lse, s, nullptr, nullptr,
                    nullptr, 0, 0, max_len, ws, ws_bytes, stream);
}

int32_t kvc_decode_step(const kvc_cache *cache, const void *k_new, const void *v_new, int32_t t,
                        const void *q, int32_t G, float scale, int32_t rule, float alpha,
                        int32_t budget, int32_t refresh, float *out, float *lse, float *s,
                        const kvc_moments *mom, const kvc_merge *merge, uint8_t *evict_out,
                        int32_t attn_unit0, int32_t attn_units, int32_t max_len, void *ws,
                        size_t ws_bytes, void *stream) {
  return run_decode(cache, k_new, v_new, t, q, G, scale, 1, rule, alpha, budget, refresh, out, lse, s,
                    mom, merge, evict_out, attn_unit0, attn_units, max_len, ws, ws_bytes, stream);
}

int32_t kvc_decode_groups(const kvc_cache *cache, const void *q, int32_t G, float scale, int32_t rule,
                          float alpha, int32_t refresh, int32_t unit0, int32_t n_groups, int32_t group_units,
                          float *out, float *lse, float *s, int32_t max_len, void *ws, size_t ws_bytes,
                          void *stream) {
  const kvc_cache *c = cache;
  const int st = validate_cache(c);
  if (st) return st;
  if (!valid_G(G)) return KVC_ERR_UNSUPPORTED;
  if (!q || !out || !lse) return KVC_ERR_ARG;
  if (!aligned16(q)) return KVC_ERR_ALIGN;
  if (n_groups <= 0 || group_units <= 0 || unit0 < 0) return KVC_ERR_ARG;
  const int64_t units64 = int64_t(n_groups) * group_units;
  if (unit0 + units64 > c->units_per_scope) return KVC_ERR_ARG;
  if (group_units * G > 64) return KVC_ERR_UNSUPPORTED;
  const int units = int(units64);
  if (rule < KVC_RULE_SINGLE || rule > KVC_RULE_EMA) return KVC_ERR_ARG;
  if (refresh && !c->m) return KVC_ERR_ARG;
  if (max_len > c->capacity) return KVC_ERR_CAPACITY;
  if (max_len <= 0) max_len = c->capacity;
  if (kvc::groups_score_lds_bytes(c->dtype, G, units) > (64u << 10)) return KVC_ERR_UNSUPPORTED;
  if (!ws) return KVC_ERR_WORKSPACE;
  const DecodeLayout d = decode_layout(c, G, units);
  if (ws_bytes < d.total) return KVC_ERR_WORKSPACE;

  kvc::StepArgs a{};
  a.k = static_cast<char *>(c->k);
  a.v = static_cast<char *>(c->v);
  a.votes = c->votes;
  a.pos = c->pos;
  a.m = c->m;
  a.len = c->len;
  a.scope_stride = c->scope_stride;
  a.unit_stride = c->unit_stride;
  a.capacity = c->capacity;
  a.n_scopes = c->n_scopes;
  a.units = c->units_per_scope;
  a.attn_unit0 = unit0;
  a.attn_units = units;
  a.append = 0;
  a.t = 0;
  a.q = static_cast<const char *>(q);
  a.scale = double(scale);
  a.out = out;
  a.lse = lse;
  a.status = at<int32_t>(ws, d.status);
  a.partM = at<double>(ws, d.partM);
  a.partZ = at<double>(ws, d.partZ);
  a.partO = at<float>(ws, d.partO);
  a.fac = at<float>(ws, d.fac);
  a.subM = at<double>(ws, d.subM);
  a.ews = at<float>(ws, d.ews);
  a.ewsh = at<uint8_t>(ws, d.ewsh);
  a.nsub_cap = d.nsub_cap;
  a.row_bytes = kHD * (c->dtype == KVC_BF16 ? 2 : 4);
  a.max_len = max_len;
  // splits sized for the live-length bound, within what the workspace holds
  const int CH = kvc::decode_chunk_tokens(c->dtype);
  a.n_splits = std::min({split_count(c->n_scopes * units, ceil_div(max_len, CH)), d.n_splits, 64});

  kvc::GroupsArgs g{};
  g.n_scopes = c->n_scopes;
  g.units = units;
  g.group_units = group_units;
  g.n_groups = n_groups;
  g.capacity = c->capacity;
  g.n_splits = a.n_splits;
  g.nsub_cap = d.nsub_cap;
  g.max_len = max_len;
  g.len = c->len;
  g.votes = c->votes;
  g.m = c->m;
  g.s = s;
  g.out = out;
  g.lse = lse;
  g.partM = a.partM;
  g.partZ = a.partZ;
  g.partO = a.partO;
  g.subM = a.subM;
  g.ews = a.ews;
  g.ewsh = a.ewsh;
  g.rule = rule;
  g.alpha = double(alpha);

  hipStream_t hs = static_cast<hipStream_t>(stream);
  // One workgroup per unit (the per-scope kernel's streaming, weights kept in LDS) when a
  // unit's per-token state for max_len tokens fits in LDS and the per-token weight sums
  // fit where the split path keeps its per-token weights; otherwise split-K attention.
  const int64_t wstride = (int64_t(max_len) + 31) / 32 * 32;
  const bool per_unit =
      kvc::decode_unit_groups_lds_bytes(c->dtype, G, max_len, c->votes != nullptr) <= device_lds_per_block() &&
      size_t(c->n_scopes) * units * wstride * sizeof(double) <= d.m64 - d.ews;
  if (per_unit) {
    a.mode = 0;
    a.refresh = refresh ? 1 : 0;
    a.n_splits = 1;
    a.lds_len = max_len;
    a.wsum = at<double>(ws, d.ews);
    a.wsum_stride = int32_t(wstride);
    g.wsum = a.wsum;
    g.wsum_stride = a.wsum_stride;
    if (kvc::launch_decode_unit_groups(a, c->dtype, G, hs) != hipSuccess) return KVC_ERR_DEVICE;
    if (refresh && kvc::launch_groups_wscore(g, G, hs) != hipSuccess) return KVC_ERR_DEVICE;
    return KVC_OK;
  }
  if (kvc::launch_decode_attention(a, c->dtype, G, hs) != hipSuccess) return KVC_ERR_DEVICE;
  if (kvc::launch_groups_epilogue(g, c->dtype, G, refresh != 0, hs) != hipSuccess) return KVC_ERR_DEVICE;
  return KVC_OK;
}

int32_t kvc_decode_plan(const kvc_cache *cache, int32_t G, int32_t step, int32_t merge, int32_t budget,
                        int32_t max_len) {
  const int st = validate_cache(cache);
  if (st) return st;
  if (!valid_G(G)) return KVC_ERR_UNSUPPORTED;
  if (max_len > cache->capacity) return KVC_ERR_CAPACITY;
  if (max_len <= 0) max_len = cache->capacity;
  if (step && budget < 0) return KVC_ERR_CAPACITY;
  return decode_plan(cache, G, step ? (merge ? 2 : 1) : 0, budget, max_len);
}

int32_t kvc_decode_step_noalloc(const kvc_cache *cache, const void *k_new, const void *v_new, int32_t t,
                                const void *q, int32_t G, float scale, int32_t rule, float alpha, int32_t budget,
                                int32_t refresh, float *out, float *lse, float *s, const kvc_moments *mom,
                                const kvc_merge *merge, uint8_t *evict_out, int32_t attn_unit0,
                                int32_t attn_units, int32_t max_len, int32_t *status, void *stream) {
  const int st = validate_cache(cache);
  if (st) return st;
  if (!valid_G(G)) return KVC_ERR_UNSUPPORTED;
  const int au = attn_units > 0 ? attn_units : cache->units_per_scope;
  if (decode_layout(cache, G, au).total > kScratchBytes) return KVC_ERR_WORKSPACE;
  void *ws = nullptr;
  const int sst = current_scratch(&ws);
  if (sst) return sst;
  return run_decode(cache, k_new, v_new, t, q, G, scale, 1, rule, alpha, budget, refresh, out, lse, s, mom, merge,
                    evict_out, attn_unit0, attn_units, max_len, ws, kScratchBytes, stream, status);
}

int32_t kvc_ema_update(float *m, const float *s, const int32_t *len, int32_t n_scopes, int32_t capacity,
                       int32_t rule, float alpha, void *stream) {
  if (!m || !s || !len || n_scopes <= 0 || capacity <= 0) return KVC_ERR_ARG;
  if (rule < KVC_RULE_SINGLE || rule > KVC_RULE_EMA) return KVC_ERR_ARG;
  if (kvc::launch_ema_update(m, s, len, n_scopes, capacity, rule, alpha, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return KVC_ERR_DEVICE;
  return KVC_OK;
}

int32_t kvc_select_evict(const float *key, const int32_t *pos, const int32_t *len, int32_t n_scopes,
                         int32_t capacity, int32_t budget, uint8_t *evict, int32_t *n_evict, void *ws,
                         size_t ws_bytes, void *stream) {
  return select_evict(key, pos, len, n_scopes, capacity, budget, false, 0, evict, n_evict, ws, ws_bytes, stream);
}

int32_t kvc_ema_predict(const float *m, const int32_t *len, int32_t n_scopes, int32_t capacity, float alpha,
                        int32_t t, float *out, void *stream) {
  if (!m || !out || n_scopes <= 0 || capacity <= 0 || t < 1) return KVC_ERR_ARG;
  if (!(alpha > 0.f && alpha < 1.f)) return KVC_ERR_ARG;
  if (kvc::launch_ema_predict(m, len, n_scopes, capacity, alpha, t, out, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return KVC_ERR_DEVICE;
  return KVC_OK;
}

int32_t kvc_read_probe(const void *buf, size_t bytes, int32_t workgroups, int32_t reverse, uint32_t *sink,
                       void *stream) {
  if (!buf || !sink || workgroups <= 0 || bytes < 16) return KVC_ERR_ARG;
  if (!aligned16(buf)) return KVC_ERR_ALIGN;
  if (kvc::launch_read_probe(buf, bytes, workgroups, reverse, sink, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KVC_ERR_DEVICE;
  return KVC_OK;
}

int32_t kvc_keep_jaccard(const uint8_t *keep_a, const uint8_t *keep_b, const int32_t *len, int32_t n_scopes,
                         int32_t capacity, float *out, void *stream) {
  if (!keep_a || !keep_b || !out || n_scopes <= 0 || capacity <= 0) return KVC_ERR_ARG;
  if (kvc::launch_jaccard(keep_a, keep_b, len, n_scopes, capacity, out, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return KVC_ERR_DEVICE;
  return KVC_OK;
}

int32_t kvc_select_evict_protected(const float *key, const int32_t *pos, const int32_t *len, int32_t n_scopes,
                                   int32_t capacity, int32_t budget, int32_t protect_from, uint8_t *evict,
                                   int32_t *n_evict, void *ws, size_t ws_bytes, void *stream) {
  if (n_scopes == 1 && len == nullptr && capacity > (1 << 20)) return KVC_ERR_UNSUPPORTED;
  return select_evict(key, pos, len, n_scopes, capacity, budget, true, protect_from, evict, n_evict, ws, ws_bytes,
                      stream);
}

}  // extern "C"

namespace {

int32_t select_evict(const float *key, const int32_t *pos, const int32_t *len, int32_t n_scopes, int32_t capacity,
                     int32_t budget, bool protect, int32_t protect_from, uint8_t *evict, int32_t *n_evict, void *ws,
                     size_t ws_bytes, void *stream) {
  if (!key || !evict || n_scopes <= 0 || capacity <= 0) return KVC_ERR_ARG;
  if (budget < 0) return KVC_ERR_CAPACITY;
  if (!ws || ws_bytes < kvc_select_workspace_size(n_scopes, capacity)) return KVC_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (n_scopes == 1 && len == nullptr && capacity > (1 << 20)) {   // one model-wide Top-K
    if (kvc::launch_select_wide(key, pos, capacity, budget, evict, n_evict, ws, hs) != hipSuccess)
      return KVC_ERR_DEVICE;
    return KVC_OK;
  }
  const SelectLayout l = select_layout(n_scopes, capacity);
  kvc::BulkArgs b{};
  b.st = at<kvc::BulkScope>(ws, l.state);
  b.hpart = at<uint32_t>(ws, l.hist);
  b.cnt = at<int32_t>(ws, l.cnt);
  b.key = key;
  b.pos = pos;
  b.flags = evict;
  b.len = len;
  b.n_evict = n_evict;
  b.cap = capacity;
  b.budget = budget;
  b.n_scopes = n_scopes;
  b.n_chunks = l.n_chunks;
  b.chunk = l.chunk;
  b.protect = protect ? 1 : 0;
  b.protect_from = protect_from;
  if (kvc::launch_bulk_select(b, hs) != hipSuccess) return KVC_ERR_DEVICE;
  return KVC_OK;
}

}  // namespace

extern "C" {

int32_t kvc_moment_update(const kvc_cache *cache, const uint8_t *evict, const kvc_moments *mom,
                          void *stream) {
  int st = validate_cache(cache);
  if (st) return st;
  if (!evict || !mom || !mom->n || !mom->sk || !mom->sv || !mom->S) return KVC_ERR_ARG;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const hipError_t e = cache->dtype == KVC_BF16
                           ? kvc::launch_moment_update_mfma(cache_args(cache), evict, mom->n, mom->sk, mom->sv, mom->S, hs)
                           : kvc::launch_moment_update(cache_args(cache), evict, mom->n, mom->sk, mom->sv, mom->S, hs);
  if (e != hipSuccess) return KVC_ERR_DEVICE;
  return KVC_OK;
}

int32_t kvc_moment_correct(const kvc_moments *mom, int32_t n_units, const void *q, int32_t dtype, int32_t G,
                           float scale, const float *f_R, const float *lse_R, float *out, void *stream) {
  if (!mom || !mom->n || !mom->sk || !mom->sv || !mom->S || !q || !f_R || !lse_R || !out) return KVC_ERR_ARG;
  if (n_units <= 0) return KVC_ERR_ARG;
  if (dtype != KVC_BF16 && dtype != KVC_F32) return KVC_ERR_DTYPE;
  if (!valid_G(G)) return KVC_ERR_UNSUPPORTED;
  if (!aligned16(mom->S)) return KVC_ERR_ALIGN;
  kvc::MomentArgs m{mom->n, mom->sk, mom->sv, mom->S};
  if (kvc::launch_moment_correct(m, n_units, q, dtype, G, double(scale), f_R, lse_R, out,
                                 static_cast<hipStream_t>(stream)) != hipSuccess)
    return KVC_ERR_DEVICE;
  return KVC_OK;
}

size_t kvc_moment_evict_workspace_size(const kvc_cache *cache) {
  if (validate_cache(cache)) return 0;
  return moment_evict_layout(cache->n_scopes, cache->capacity).total;
}

int32_t kvc_moment_evict(const kvc_cache *cache, const kvc_moments *mom, const float *alpha, float scale,
                         int32_t budget, int32_t max_len, uint8_t *evict, int32_t *order, float *score_out,
                         int32_t *n_evict, void *ws, size_t ws_bytes, void *stream) {
  int st = validate_cache(cache);
  if (st) return st;
  if (cache->units_per_scope != 1) return KVC_ERR_UNSUPPORTED;
  if (!mom || !mom->n || !mom->sk || !mom->sv || !mom->S || !alpha || !evict || !ws) return KVC_ERR_ARG;
  if (!aligned16(mom->S) || !aligned16(mom->sk)) return KVC_ERR_ALIGN;
  if (budget < 0 || max_len > cache->capacity) return KVC_ERR_CAPACITY;
  const MomentEvictLayout l = moment_evict_layout(cache->n_scopes, cache->capacity);
  if (ws_bytes < l.total) return KVC_ERR_WORKSPACE;
  const int ml = max_len > 0 ? max_len : cache->capacity;
  kvc::MomentEvictArgs p{};
  p.k = static_cast<const char *>(cache->k);
  p.v = static_cast<const char *>(cache->v);
  p.scope_stride = cache->scope_stride;
  p.pos = cache->pos;
  p.len = cache->len;
  p.mom_n = mom->n;
  p.sk = mom->sk;
  p.sv = mom->sv;
  p.S = mom->S;
  p.alpha = alpha;
  p.scale = double(scale);
  p.capacity = cache->capacity;
  p.n_scopes = cache->n_scopes;
  p.budget = budget;
  p.rounds = std::max(1, ml - budget);
  // chunks of whole 64-token tiles, about kMomentWorkgroups workgroups over the scopes
  const int tiles = ceil_div(ml, kMomentTile);
  const int per_scope = std::max(1, std::min(tiles, ceil_div(kMomentWorkgroups, cache->n_scopes)));
  p.chunk = kMomentTile * ceil_div(tiles, per_scope);
  p.n_chunks = l.n_chunks;
  p.n_chunks_used = ceil_div(cache->capacity, p.chunk);   // chunks past a scope's live length exit at once
  p.fused_pick = p.chunk >= cache->capacity;
  p.evict = evict;
  p.order = order;
  p.n_evict = n_evict;
  p.score_out = score_out;
  p.cand_score = at<double>(ws, l.score);
  p.cand_pos = at<int32_t>(ws, l.pos);
  p.cand_slot = at<int32_t>(ws, l.slot);
  p.status = at<int32_t>(ws, l.status);
  if (kvc::launch_moment_evict(p, cache->dtype, p.rounds, static_cast<hipStream_t>(stream)) != hipSuccess)
    return KVC_ERR_DEVICE;
  return KVC_OK;
}

size_t kvc_keepkv_prefill_workspace_size(const kvc_cache *cache) {
  if (validate_cache(cache)) return 0;
  return prefill_layout(cache->n_scopes, cache->capacity).total;
}

int32_t kvc_keepkv_prefill_merge(const kvc_cache *cache, const kvc_merge *merge, int32_t budget,
                                 int32_t protect_from, uint8_t *evict, int32_t *pairs, int32_t *n_merged,
                                 void *ws, size_t ws_bytes, void *stream) {
  return kvc_keepkv_prefill_merge_marked(cache, merge, budget, protect_from, evict, pairs, n_merged, ws, ws_bytes,
                                         stream, nullptr, 0);
}

int32_t kvc_keepkv_prefill_merge_marked(const kvc_cache *cache, const kvc_merge *merge, int32_t budget,
                                        int32_t protect_from, uint8_t *evict, int32_t *pairs, int32_t *n_merged,
                                        void *ws, size_t ws_bytes, void *stream, void *const *events,
                                        int32_t n_events) {
  if (events && n_events != 4) return KVC_ERR_ARG;
  int st = validate_cache(cache);
  if (st) return st;
  if (cache->units_per_scope != 1 || cache->capacity > kvc::PREFILL_MAX_ROWS) return KVC_ERR_UNSUPPORTED;
  if (!cache->votes || !merge || !merge->q || !evict || !ws) return KVC_ERR_ARG;
  if (!valid_G(merge->G)) return KVC_ERR_UNSUPPORTED;
  if (!aligned16(merge->q)) return KVC_ERR_ALIGN;
  if (budget < 0) return KVC_ERR_CAPACITY;
  const PrefillLayout l = prefill_layout(cache->n_scopes, cache->capacity);
  if (ws_bytes < l.total) return KVC_ERR_WORKSPACE;
  kvc::PrefillMergeArgs p{};
  p.k = static_cast<char *>(cache->k);
  p.v = static_cast<char *>(cache->v);
  p.scope_stride = cache->scope_stride;
  p.votes = cache->votes;
  p.pos = cache->pos;
  p.len = cache->len;
  p.m = cache->m;
  p.q = static_cast<const char *>(merge->q);
  p.G = merge->G;
  p.scale = double(merge->scale);
  p.eps = merge->eps;
  p.capacity = cache->capacity;
  p.n_scopes = cache->n_scopes;
  p.budget = budget;
  p.protect_from = protect_from;
  p.evict = evict;
  p.pairs = pairs;
  p.n_merged = n_merged;
  p.meta = at<char>(ws, l.meta);
  p.rec = at<char>(ws, l.rec);
  p.sum = at<char>(ws, l.sum);
  p.status = at<int32_t>(ws, l.status);
  hipEvent_t *marks = events ? reinterpret_cast<hipEvent_t *>(const_cast<void **>(events)) : nullptr;
  if (kvc::launch_prefill_merge(p, cache->dtype, static_cast<hipStream_t>(stream), marks) != hipSuccess)
    return KVC_ERR_DEVICE;
  return KVC_OK;
}

int32_t kvc_compact(const kvc_cache *cache, const uint8_t *evict, const kvc_merge *merge, void *ws,
                    size_t ws_bytes, void *stream) {
  int st = validate_cache(cache);
  if (st) return st;
  if (!evict) return KVC_ERR_ARG;
  if (!ws) return KVC_ERR_WORKSPACE;
  const CompactLayout l = compact_layout(cache);
  if (ws_bytes < l.total) return KVC_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if (merge) {
    if (!merge->q || !aligned16(merge->q) || !valid_G(merge->G) || !cache->votes) return KVC_ERR_ARG;
    if (cache->units_per_scope != 1) return KVC_ERR_UNSUPPORTED;
    kvc::MergeArgs mg{};
    mg.status = at<int32_t>(ws, l.status);
    mg.q = static_cast<const char *>(merge->q);
    mg.G = merge->G;
    mg.scale = double(merge->scale);
    mg.eps = merge->eps;
    mg.n_splits = l.merge_splits;
    mg.part_cos = at<double>(ws, l.cos);
    mg.part_slot = at<int32_t>(ws, l.slot);
    if (kvc::launch_merge(cache_args(cache), evict, mg, hs) != hipSuccess) return KVC_ERR_DEVICE;
    return KVC_OK;
  }
  kvc::StepArgs a{};
  a.k = static_cast<char *>(cache->k);
  a.v = static_cast<char *>(cache->v);
  a.votes = cache->votes;
  a.pos = cache->pos;
  a.m = cache->m;
  a.len = cache->len;
  a.scope_stride = cache->scope_stride;
  a.unit_stride = cache->unit_stride;
  a.capacity = cache->capacity;
  a.n_scopes = cache->n_scopes;
  a.units = cache->units_per_scope;
  kvc::BulkArgs b{};
  b.st = at<kvc::BulkScope>(ws, l.sel.state);
  b.cnt = at<int32_t>(ws, l.sel.cnt);
  b.flags = const_cast<uint8_t *>(evict);   // read only on this path
  b.list = at<int32_t>(ws, l.list);
  b.list2 = at<int32_t>(ws, l.list2);
  b.len = cache->len;
  b.cap = cache->capacity;
  b.n_scopes = cache->n_scopes;
  b.n_chunks = l.sel.n_chunks;
  b.chunk = l.sel.chunk;
  b.move_blocks = std::max(1, std::min(64, ceil_div(kTargetWorkgroups, cache->n_scopes)));
  if (kvc::launch_bulk_compact(a, b, cache->dtype, hs) != hipSuccess) return KVC_ERR_DEVICE;
  return KVC_OK;
}

size_t kvc_keepkv_ema_init_workspace_size(const kvc_cache *cache, int32_t G, int32_t n_win, int32_t n_tokens) {
  if (validate_cache(cache) || !valid_G(G) || n_win <= 0 || n_tokens < n_win || n_tokens > cache->capacity)
    return 0;
  return kvc::ema_window_workspace_bytes(cache->n_scopes, G, n_tokens, n_win);
}

int32_t kvc_keepkv_ema_init(const kvc_cache *cache, const void *q_win, int32_t G, int32_t n_win, int32_t n_tokens,
                            float scale, float alpha, void *ws, size_t ws_bytes, void *stream) {
  return kvc_keepkv_ema_init_marked(cache, q_win, G, n_win, n_tokens, scale, alpha, ws, ws_bytes, stream, nullptr,
                                    0);
}

int32_t kvc_keepkv_ema_init_marked(const kvc_cache *cache, const void *q_win, int32_t G, int32_t n_win,
                                   int32_t n_tokens, float scale, float alpha, void *ws, size_t ws_bytes,
                                   void *stream, void *const *events, int32_t n_events) {
  if (events && n_events != kvc::kEmaStages + 1) return KVC_ERR_ARG;
  int st = validate_cache(cache);
  if (st) return st;
  if (cache->units_per_scope != 1 || !valid_G(G)) return KVC_ERR_UNSUPPORTED;
  if (cache->dtype != KVC_BF16) return KVC_ERR_DTYPE;
  if (!q_win || !cache->m || !(alpha > 0.f && alpha < 1.f)) return KVC_ERR_ARG;
  if (n_win <= 0 || n_tokens < n_win || n_tokens > cache->capacity) return KVC_ERR_CAPACITY;
  if (!aligned16(q_win)) return KVC_ERR_ALIGN;
  if (!ws || ws_bytes < kvc::ema_window_workspace_bytes(cache->n_scopes, G, n_tokens, n_win)) return KVC_ERR_WORKSPACE;
  hipEvent_t *marks = events ? reinterpret_cast<hipEvent_t *>(const_cast<void **>(events)) : nullptr;
  if (kvc::launch_ema_window(q_win, cache->k, cache->scope_stride, cache->n_scopes, G, n_win, n_tokens, double(scale),
                             double(alpha), cache->m, cache->capacity, ws, static_cast<hipStream_t>(stream),
                             marks) != hipSuccess)
    return KVC_ERR_DEVICE;
  return KVC_OK;
}

// ------------------------------------------------------- KeepKV periodic refresh
// The prefill merging's workspace first (its status word is the refresh's), then
// the EMA window initialisation's, the compaction's, and the merge flags.
struct RefreshLayout {
  size_t prefill, ema, compact, evict, total;
};

RefreshLayout refresh_layout(const kvc_cache *c, int G, int n_win, int n_tokens) {
  RefreshLayout l{};
  size_t o = 0;
  l.prefill = o; o = align_up(o + prefill_layout(c->n_scopes, c->capacity).total);
  l.ema = o;     o = align_up(o + kvc::ema_window_workspace_bytes(c->n_scopes, G, n_tokens, n_win));
  l.compact = o; o = align_up(o + compact_layout(c).total);
  l.evict = o;   o = align_up(o + size_t(c->n_scopes) * c->capacity);
  l.total = o;
  return l;
}

size_t kvc_keepkv_refresh_workspace_size(const kvc_cache *cache, int32_t G, int32_t n_win, int32_t n_tokens) {
  if (validate_cache(cache) || !valid_G(G) || n_win <= 0 || n_tokens < n_win || n_tokens > cache->capacity)
    return 0;
  return refresh_layout(cache, G, n_win, n_tokens).total;
}

int32_t kvc_keepkv_refresh(const kvc_cache *cache, const void *host_k, const void *host_v, const int32_t *host_pos,
                           int32_t n_tokens, const void *q_win, int32_t n_win, const kvc_merge *merge, float alpha,
                           int32_t budget, int32_t protect_from, int32_t *pairs, int32_t *n_merged, void *ws,
                           size_t ws_bytes, void *stream) {
  return kvc_keepkv_refresh_marked(cache, host_k, host_v, host_pos, n_tokens, q_win, n_win, merge, alpha, budget,
                                   protect_from, pairs, n_merged, ws, ws_bytes, stream, nullptr, 0);
}

int32_t kvc_keepkv_refresh_marked(const kvc_cache *cache, const void *host_k, const void *host_v,
                                  const int32_t *host_pos, int32_t n_tokens, const void *q_win, int32_t n_win,
                                  const kvc_merge *merge, float alpha, int32_t budget, int32_t protect_from,
                                  int32_t *pairs, int32_t *n_merged, void *ws, size_t ws_bytes, void *stream,
                                  void *const *events, int32_t n_events) {
  if (events && n_events != 5) return KVC_ERR_ARG;
  const int st = validate_cache(cache);
  if (st) return st;
  const kvc_cache *c = cache;
  if (c->units_per_scope != 1 || c->capacity > kvc::PREFILL_MAX_ROWS) return KVC_ERR_UNSUPPORTED;
  if (c->dtype != KVC_BF16) return KVC_ERR_DTYPE;
  if (!host_k || !host_v || !host_pos || !q_win || !merge || !merge->q || !c->votes || !c->m) return KVC_ERR_ARG;
  if (!valid_G(merge->G)) return KVC_ERR_UNSUPPORTED;
  if (!aligned16(q_win) || !aligned16(merge->q)) return KVC_ERR_ALIGN;
  if (!(alpha > 0.f && alpha < 1.f)) return KVC_ERR_ARG;
  if (n_win <= 0 || n_tokens < n_win || n_tokens > c->capacity || budget < 0) return KVC_ERR_CAPACITY;
  if (!ws) return KVC_ERR_WORKSPACE;
  const int G = merge->G;
  const RefreshLayout l = refresh_layout(c, G, n_win, n_tokens);
  if (ws_bytes < l.total) return KVC_ERR_WORKSPACE;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipEvent_t *marks = events ? reinterpret_cast<hipEvent_t *>(const_cast<void **>(events)) : nullptr;
  auto mark = [&](int i) { return marks ? hipEventRecord(marks[i], hs) : hipSuccess; };
  const size_t rb = size_t(kHD) * 2;   // bf16 row
  const size_t width = size_t(n_tokens) * rb, dpitch = size_t(c->scope_stride) * rb;

  // reload: rows and positions of the full KV into slots [0, n_tokens), votes 1, length n_tokens
  if (mark(0) != hipSuccess) return KVC_ERR_DEVICE;
  if (hipMemcpy2DAsync(c->k, dpitch, host_k, width, width, c->n_scopes, hipMemcpyHostToDevice, hs) != hipSuccess ||
      hipMemcpy2DAsync(c->v, dpitch, host_v, width, width, c->n_scopes, hipMemcpyHostToDevice, hs) != hipSuccess ||
      hipMemcpy2DAsync(c->pos, size_t(c->capacity) * 4, host_pos, size_t(n_tokens) * 4, size_t(n_tokens) * 4,
                       c->n_scopes, hipMemcpyHostToDevice, hs) != hipSuccess)
    return KVC_ERR_DEVICE;
  if (kvc::launch_reload_slots(c->votes, c->len, c->n_scopes, n_tokens, c->capacity, hs) != hipSuccess)
    return KVC_ERR_DEVICE;
  if (mark(1) != hipSuccess) return KVC_ERR_DEVICE;

  // the EMA state of every reloaded token: eq. (15)'s window form over the last n_win queries
  if (kvc::launch_ema_window(q_win, c->k, c->scope_stride, c->n_scopes, G, n_win, n_tokens, double(merge->scale),
                             double(alpha), c->m, c->capacity, at<char>(ws, l.ema), hs, nullptr) != hipSuccess)
    return KVC_ERR_DEVICE;
  if (mark(2) != hipSuccess) return KVC_ERR_DEVICE;

  // greedy ZIP merging with the current query's exact group-mean logits
  const PrefillLayout pl = prefill_layout(c->n_scopes, c->capacity);
  uint8_t *evict = at<uint8_t>(ws, l.evict);
  kvc::PrefillMergeArgs p{};
  p.k = static_cast<char *>(c->k);
  p.v = static_cast<char *>(c->v);
  p.scope_stride = c->scope_stride;
  p.votes = c->votes;
  p.pos = c->pos;
  p.len = c->len;
  p.m = c->m;
  p.q = static_cast<const char *>(merge->q);
  p.G = G;
  p.scale = double(merge->scale);
  p.eps = merge->eps;
  p.capacity = c->capacity;
  p.n_scopes = c->n_scopes;
  p.budget = budget;
  p.protect_from = protect_from;
  p.evict = evict;
  p.pairs = pairs;
  p.n_merged = n_merged;
  p.meta = at<char>(ws, l.prefill + pl.meta);
  p.rec = at<char>(ws, l.prefill + pl.rec);
  p.sum = at<char>(ws, l.prefill + pl.sum);
  p.status = at<int32_t>(ws, l.prefill + pl.status);
  if (kvc::launch_prefill_merge(p, c->dtype, hs, nullptr) != hipSuccess) return KVC_ERR_DEVICE;
  if (mark(3) != hipSuccess) return KVC_ERR_DEVICE;

  // the merged-away slots out
  const CompactLayout cl = compact_layout(c);
  char *cws = at<char>(ws, l.compact);
  kvc::StepArgs a{};
  a.k = static_cast<char *>(c->k);
  a.v = static_cast<char *>(c->v);
  a.votes = c->votes;
  a.pos = c->pos;
  a.m = c->m;
  a.len = c->len;
  a.scope_stride = c->scope_stride;
  a.unit_stride = c->unit_stride;
  a.capacity = c->capacity;
  a.n_scopes = c->n_scopes;
  a.units = c->units_per_scope;
  kvc::BulkArgs b{};
  b.st = reinterpret_cast<kvc::BulkScope *>(cws + cl.sel.state);
  b.cnt = reinterpret_cast<int32_t *>(cws + cl.sel.cnt);
  b.flags = evict;
  b.list = reinterpret_cast<int32_t *>(cws + cl.list);
  b.list2 = reinterpret_cast<int32_t *>(cws + cl.list2);
  b.len = c->len;
  b.cap = c->capacity;
  b.n_scopes = c->n_scopes;
  b.n_chunks = cl.sel.n_chunks;
  b.chunk = cl.sel.chunk;
  b.move_blocks = std::max(1, std::min(64, ceil_div(kTargetWorkgroups, c->n_scopes)));
  if (kvc::launch_bulk_compact(a, b, c->dtype, hs) != hipSuccess) return KVC_ERR_DEVICE;
  if (mark(4) != hipSuccess) return KVC_ERR_DEVICE;
  return KVC_OK;
}

size_t kvc_laprox_workspace_size(int32_t n_layers, int32_t H, int32_t n_kv, int32_t N, int32_t w, int32_t d,
                                 int32_t D) {
  return kvc::laprox_workspace_bytes(n_layers, H, n_kv, N, w, d, D);
}

int32_t kvc_laprox_score(const void *q_win, const void *k, const void *v, const void *w_o, int32_t n_layers,
                         int32_t H, int32_t n_kv, int32_t N, int32_t w, int32_t d, int32_t D, float scale,
                         float *score, void *ws, size_t ws_bytes, void *stream) {
  return kvc_laprox_score_marked(q_win, k, v, w_o, n_layers, H, n_kv, N, w, d, D, scale, score, ws, ws_bytes,
                                 stream, nullptr, 0);
}

int32_t kvc_laprox_score_marked(const void *q_win, const void *k, const void *v, const void *w_o,
                                int32_t n_layers, int32_t H, int32_t n_kv, int32_t N, int32_t w, int32_t d,
                                int32_t D, float scale, float *score, void *ws, size_t ws_bytes, void *stream,
                                void *const *events, int32_t n_events) {
  if (events && n_events != kvc::kLaproxStages + 1) return KVC_ERR_ARG;
  if (!q_win || !k || !v || !w_o || !score) return KVC_ERR_ARG;
  if (n_layers <= 0 || H <= 0 || n_kv <= 0 || N <= 0 || w <= 0 || D <= 0) return KVC_ERR_ARG;
  if (d != kHD || !kvc::laprox_shape_supported(H, n_kv, N, w, D)) return KVC_ERR_UNSUPPORTED;
  if (!aligned16(q_win) || !aligned16(k) || !aligned16(v) || !aligned16(w_o)) return KVC_ERR_ALIGN;
  if (!ws || ws_bytes < kvc::laprox_workspace_bytes(n_layers, H, n_kv, N, w, d, D)) return KVC_ERR_WORKSPACE;
  hipEvent_t *marks = events ? reinterpret_cast<hipEvent_t *>(const_cast<void **>(events)) : nullptr;
  if (kvc::launch_laprox(q_win, k, v, w_o, n_layers, H, n_kv, N, w, D, double(scale), score, ws,
                         static_cast<hipStream_t>(stream), marks) != hipSuccess)
    return KVC_ERR_DEVICE;
  return KVC_OK;
}

}  // extern "C"
