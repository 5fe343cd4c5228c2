// Expert-slot cache: host-side LRU over a fixed HBM pool of expert records,
// refilled from a pinned host bank (FreeToken guide, "expert bank & LRU slot
// cache", "MoE strategies" offload, "minimum cache constraint").
//
// The handle owns host metadata only: slot owners, last-active steps, the
// step clock and a small ring of pinned slot-table rows used as sources of
// the host->device slot-table updates (a row is never rewritten while an
// earlier copy from it may still be pending).
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "moe_internal.h"

namespace {

constexpr int kRing = 8;
constexpr int kMaxGroups = 16;  // fill groups of expert_cache_fill_groups

struct Cache {
  int L = 0, E = 0, S = 0;
  int64_t slot_bytes = 0;
  uint8_t* pool = nullptr;
  const uint8_t* bank = nullptr;
  int32_t* table_dev = nullptr;
  std::vector<int64_t> owner;    // per slot: layer*E + expert, or -1
  std::vector<int64_t> recency;  // per slot: last active step
  std::vector<int32_t> where;    // per (layer, expert): slot or -1
  int64_t clock = 0;
  int64_t st_steps = 0, st_hits = 0, st_misses = 0, st_bytes = 0;
  int32_t* ring = nullptr;  // pinned [kRing][E]
  hipEvent_t ring_done[kRing] = {};
  bool ring_used[kRing] = {};
  int ring_next = 0;
  hipEvent_t compute_mark = nullptr, side_done = nullptr;
  hipEvent_t group_done[kMaxGroups] = {};
};

}  // namespace

struct moe_cache : Cache {};

using moe::set_error;

extern "C" int moe_cache_create(moe_cache_t* out, int32_t n_layers, int32_t E, int32_t S,
                                int64_t slot_bytes, void* pool_dev, const void* bank_host,
                                int32_t* slot_table_dev) {
  if (!out) return set_error(MOE_ERR_INVALID_ARG, "moe_cache_create: out is NULL");
  *out = nullptr;
  if (n_layers < 1 || E < 1 || E > moe::kMaxE || S < 1 || slot_bytes <= 0 || slot_bytes % 256)
    return set_error(MOE_ERR_INVALID_ARG,
                     "moe_cache_create: need n_layers>=1, 1<=E<=%d, S>=1, slot_bytes>0 and a "
                     "multiple of 256", moe::kMaxE);
  moe_cache* c = new (std::nothrow) moe_cache();
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "moe_cache_create: out of host memory");
  c->L = n_layers; c->E = E; c->S = S; c->slot_bytes = slot_bytes;
  c->pool = static_cast<uint8_t*>(pool_dev);
  c->bank = static_cast<const uint8_t*>(bank_host);
  c->table_dev = slot_table_dev;
  c->owner.assign(S, -1);
  c->recency.assign(S, -1);
  c->where.assign((size_t)n_layers * E, -1);
  // Device-side pieces are only needed by expert_cache_fill; a handle without
  // them still runs the policy (expert_cache_lookup is host-only).
  if (pool_dev && bank_host && slot_table_dev) {
    if (hipHostMalloc((void**)&c->ring, sizeof(int32_t) * kRing * E, hipHostMallocDefault) !=
        hipSuccess) {
      delete c;
      return set_error(MOE_ERR_HIP, "moe_cache_create: hipHostMalloc failed");
    }
    bool ok = hipEventCreateWithFlags(&c->compute_mark, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&c->side_done, hipEventDisableTiming) == hipSuccess;
    for (int i = 0; ok && i < kRing; ++i)
      ok = hipEventCreateWithFlags(&c->ring_done[i], hipEventDisableTiming) == hipSuccess;
    for (int i = 0; ok && i < kMaxGroups; ++i)
      ok = hipEventCreateWithFlags(&c->group_done[i], hipEventDisableTiming) == hipSuccess;
    if (!ok) {
      moe_cache_destroy(c);
      return set_error(MOE_ERR_HIP, "moe_cache_create: hipEventCreate failed");
    }
  }
  *out = c;
  return MOE_OK;
}

extern "C" void moe_cache_destroy(moe_cache_t c) {
  if (!c) return;
  for (int i = 0; i < kRing; ++i)
    if (c->ring_done[i]) {
      if (c->ring_used[i]) (void)hipEventSynchronize(c->ring_done[i]);
      (void)hipEventDestroy(c->ring_done[i]);
    }
  for (int i = 0; i < kMaxGroups; ++i)
    if (c->group_done[i]) (void)hipEventDestroy(c->group_done[i]);
  if (c->compute_mark) (void)hipEventDestroy(c->compute_mark);
  if (c->side_done) (void)hipEventDestroy(c->side_done);
  if (c->ring) (void)hipHostFree(c->ring);
  delete c;
}

extern "C" int expert_cache_lookup(moe_cache_t c, int32_t layer, const int32_t* counts_host,
                                   int32_t* miss_expert, int32_t* miss_slot, int32_t* n_miss,
                                   int32_t* n_hit, int32_t* slot_row_host) {
  if (!c || !counts_host || !miss_expert || !miss_slot || !n_miss || !n_hit)
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_lookup: null argument");
  if (layer < 0 || layer >= c->L)
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_lookup: layer %d of %d", layer, c->L);
  const int E = c->E, S = c->S;
  std::vector<int> needed;
  needed.reserve(E);
  for (int e = 0; e < E; ++e) {
    if (counts_host[e] < 0)
      return set_error(MOE_ERR_INVALID_ARG, "expert_cache_lookup: counts[%d] < 0", e);
    if (counts_host[e] > 0) needed.push_back(e);
  }
  if ((int)needed.size() > S)
    return set_error(MOE_ERR_CAPACITY,
                     "expert_cache_lookup: layer %d needs %d distinct experts, pool has %d slots",
                     layer, (int)needed.size(), S);
  const int64_t key0 = (int64_t)layer * E;
  std::vector<char> is_needed_slot(S, 0);
  for (int e : needed) {
    const int s = c->where[key0 + e];
    if (s >= 0) is_needed_slot[s] = 1;
  }
  int nm = 0;
  int next_empty = 0;
  for (int e : needed) {
    if (c->where[key0 + e] >= 0) continue;
    int s = -1;
    while (next_empty < S && c->owner[next_empty] >= 0) ++next_empty;
    if (next_empty < S) {
      s = next_empty;
    } else {
      int64_t best_r = 0;
      for (int q = 0; q < S; ++q) {
        if (is_needed_slot[q]) continue;
        if (s < 0 || c->recency[q] < best_r) { s = q; best_r = c->recency[q]; }
      }
      // |needed| <= S guarantees a candidate; evict its owner
      const int64_t old = c->owner[s];
      c->where[old] = -1;
    }
    c->owner[s] = key0 + e;
    c->where[key0 + e] = s;
    is_needed_slot[s] = 1;
    miss_expert[nm] = e;
    miss_slot[nm] = s;
    ++nm;
  }
  for (int e : needed) c->recency[c->where[key0 + e]] = c->clock;
  c->clock += 1;
  *n_miss = nm;
  *n_hit = (int)needed.size() - nm;
  if (slot_row_host)
    for (int e = 0; e < E; ++e) slot_row_host[e] = c->where[key0 + e];
  c->st_steps += 1;
  c->st_hits += *n_hit;
  c->st_misses += nm;
  return MOE_OK;
}

extern "C" int expert_cache_row(moe_cache_t c, int32_t layer, int32_t* slot_row_host) {
  if (!c || !slot_row_host) return set_error(MOE_ERR_INVALID_ARG, "expert_cache_row: null argument");
  if (layer < 0 || layer >= c->L)
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_row: layer %d of %d", layer, c->L);
  const int64_t key0 = (int64_t)layer * c->E;
  for (int e = 0; e < c->E; ++e) slot_row_host[e] = c->where[key0 + e];
  return MOE_OK;
}

extern "C" int expert_cache_fill(moe_cache_t c, int32_t layer, const int32_t* miss_expert,
                                 const int32_t* miss_slot, int32_t n_miss, moe_stream_t side,
                                 moe_stream_t compute) {
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "expert_cache_fill: null handle");
  if (!c->pool || !c->bank || !c->table_dev || !c->ring)
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_fill: handle has no pool/bank/table");
  if (layer < 0 || layer >= c->L || n_miss < 0 || n_miss > c->E ||
      (n_miss > 0 && (!miss_expert || !miss_slot)))
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_fill: bad layer or miss list");
  for (int i = 0; i < n_miss; ++i) {
    const int e = miss_expert[i], s = miss_slot[i];
    if (e < 0 || e >= c->E || s < 0 || s >= c->S ||
        c->owner[s] != (int64_t)layer * c->E + e)
      return set_error(MOE_ERR_INVALID_ARG,
                       "expert_cache_fill: miss %d (expert %d -> slot %d) is not a pending fill "
                       "of layer %d", i, e, s, layer);
  }
  hipStream_t sd = reinterpret_cast<hipStream_t>(side);
  hipStream_t cp = reinterpret_cast<hipStream_t>(compute);
  const int r = c->ring_next;
  c->ring_next = (r + 1) % kRing;
  if (c->ring_used[r] && hipEventSynchronize(c->ring_done[r]) != hipSuccess)
    return set_error(MOE_ERR_HIP, "expert_cache_fill: ring wait failed");
  int32_t* row = c->ring + (size_t)r * c->E;
  const int64_t key0 = (int64_t)layer * c->E;
  for (int e = 0; e < c->E; ++e) row[e] = c->where[key0 + e];

  hipError_t err = hipEventRecord(c->compute_mark, cp);
  if (err == hipSuccess) err = hipStreamWaitEvent(sd, c->compute_mark, 0);
  for (int i = 0; err == hipSuccess && i < n_miss; ++i) {
    const int e = miss_expert[i], s = miss_slot[i];
    err = hipMemcpyAsync(c->pool + (size_t)s * c->slot_bytes,
                         c->bank + ((size_t)layer * c->E + e) * c->slot_bytes, c->slot_bytes,
                         hipMemcpyHostToDevice, sd);
  }
  if (err == hipSuccess)
    err = hipMemcpyAsync(c->table_dev + key0, row, sizeof(int32_t) * c->E, hipMemcpyHostToDevice,
                         sd);
  if (err == hipSuccess) err = hipEventRecord(c->ring_done[r], sd);
  if (err == hipSuccess) c->ring_used[r] = true;
  if (err == hipSuccess) err = hipEventRecord(c->side_done, sd);
  if (err == hipSuccess) err = hipStreamWaitEvent(cp, c->side_done, 0);
  if (err != hipSuccess)
    return set_error(MOE_ERR_HIP, "expert_cache_fill: %s", hipGetErrorString(err));
  c->st_bytes += (int64_t)n_miss * c->slot_bytes;
  return MOE_OK;
}

// The fills of one lookup as groups the caller can compute behind: the slot
// table row is published on `compute` first (hit entries are unchanged; miss
// entries name slots whose bytes land with their group), `side` waits for
// everything already enqueued on `compute` (no victim slot is overwritten
// while an earlier FFN still reads it), then copies the misses group by group
// and marks each group's end; `compute` is not made to wait.
extern "C" int expert_cache_fill_groups(moe_cache_t c, int32_t layer, const int32_t* miss_expert,
                                        const int32_t* miss_slot, int32_t n_miss,
                                        int32_t n_groups, moe_stream_t side,
                                        moe_stream_t compute) {
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "expert_cache_fill_groups: null handle");
  if (!c->pool || !c->bank || !c->table_dev || !c->ring)
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_fill_groups: handle has no pool/bank/table");
  if (layer < 0 || layer >= c->L || n_miss < 0 || n_miss > c->E ||
      (n_miss > 0 && (!miss_expert || !miss_slot)))
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_fill_groups: bad layer or miss list");
  if (n_groups < (n_miss > 0 ? 1 : 0) || n_groups > kMaxGroups || n_groups > (n_miss > 0 ? n_miss : 0))
    return set_error(MOE_ERR_INVALID_ARG,
                     "expert_cache_fill_groups: n_groups %d must be in [1, min(%d, n_miss=%d)] "
                     "(0 when there are no misses)", n_groups, kMaxGroups, n_miss);
  for (int i = 0; i < n_miss; ++i) {
    const int e = miss_expert[i], s = miss_slot[i];
    if (e < 0 || e >= c->E || s < 0 || s >= c->S || c->owner[s] != (int64_t)layer * c->E + e)
      return set_error(MOE_ERR_INVALID_ARG,
                       "expert_cache_fill_groups: miss %d (expert %d -> slot %d) is not a pending "
                       "fill of layer %d", i, e, s, layer);
  }
  hipStream_t sd = reinterpret_cast<hipStream_t>(side);
  hipStream_t cp = reinterpret_cast<hipStream_t>(compute);
  const int r = c->ring_next;
  c->ring_next = (r + 1) % kRing;
  if (c->ring_used[r] && hipEventSynchronize(c->ring_done[r]) != hipSuccess)
    return set_error(MOE_ERR_HIP, "expert_cache_fill_groups: ring wait failed");
  int32_t* row = c->ring + (size_t)r * c->E;
  const int64_t key0 = (int64_t)layer * c->E;
  for (int e = 0; e < c->E; ++e) row[e] = c->where[key0 + e];

  hipError_t err = hipMemcpyAsync(c->table_dev + key0, row, sizeof(int32_t) * c->E,
                                  hipMemcpyHostToDevice, cp);
  if (err == hipSuccess) err = hipEventRecord(c->ring_done[r], cp);
  if (err == hipSuccess) c->ring_used[r] = true;
  if (err == hipSuccess) err = hipEventRecord(c->compute_mark, cp);
  if (err == hipSuccess) err = hipStreamWaitEvent(sd, c->compute_mark, 0);
  for (int gi = 0; err == hipSuccess && gi < n_groups; ++gi) {
    const int i0 = (int)((int64_t)n_miss * gi / n_groups);
    const int i1 = (int)((int64_t)n_miss * (gi + 1) / n_groups);
    for (int i = i0; err == hipSuccess && i < i1; ++i) {
      const int e = miss_expert[i], s = miss_slot[i];
      err = hipMemcpyAsync(c->pool + (size_t)s * c->slot_bytes,
                           c->bank + ((size_t)layer * c->E + e) * c->slot_bytes, c->slot_bytes,
                           hipMemcpyHostToDevice, sd);
    }
    if (err == hipSuccess) err = hipEventRecord(c->group_done[gi], sd);
  }
  if (err != hipSuccess)
    return set_error(MOE_ERR_HIP, "expert_cache_fill_groups: %s", hipGetErrorString(err));
  c->st_bytes += (int64_t)n_miss * c->slot_bytes;
  return MOE_OK;
}

extern "C" int expert_cache_wait_group(moe_cache_t c, int32_t group, moe_stream_t compute) {
  if (!c || !c->ring)
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_wait_group: handle has no device side");
  if (group < 0 || group >= kMaxGroups)
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_wait_group: group %d of %d", group,
                     kMaxGroups);
  if (hipStreamWaitEvent(reinterpret_cast<hipStream_t>(compute), c->group_done[group], 0) !=
      hipSuccess)
    return set_error(MOE_ERR_HIP, "expert_cache_wait_group: hipStreamWaitEvent failed");
  return MOE_OK;
}

// Elastic pool size: keep the residents used most recently (ties: lower slot),
// as many as the new size allows, pack them in their old slot order into the
// lowest slots, drop the rest.  Packing in ascending order only ever moves a
// record down to a slot that is free or already vacated, so in-place moves on
// one stream never overwrite a record that is still to be moved.
extern "C" int moe_cache_resize(moe_cache_t c, int32_t new_S, void* new_pool_dev,
                                int32_t* move_from, int32_t* move_to, int32_t* n_moves,
                                moe_stream_t side, moe_stream_t compute) {
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "moe_cache_resize: null handle");
  if (new_S < 1) return set_error(MOE_ERR_INVALID_ARG, "moe_cache_resize: new_S %d < 1", new_S);
  const bool dev = c->pool && c->bank && c->table_dev && c->ring;
  if (!dev && new_pool_dev)
    return set_error(MOE_ERR_INVALID_ARG, "moe_cache_resize: handle has no device pool to move");
  const int S = c->S;
  std::vector<int> res;
  for (int s = 0; s < S; ++s)
    if (c->owner[s] >= 0) res.push_back(s);
  // most recent first, lower slot first among equals
  std::vector<int> order(res);
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    return c->recency[a] != c->recency[b] ? c->recency[a] > c->recency[b] : a < b;
  });
  const int n_keep = (int)order.size() < new_S ? (int)order.size() : new_S;
  std::vector<char> keep(S, 0);
  for (int i = 0; i < n_keep; ++i) keep[order[i]] = 1;
  std::vector<int> from;
  for (int s : res)
    if (keep[s]) from.push_back(s);  // ascending old slot

  uint8_t* dst_pool = new_pool_dev ? static_cast<uint8_t*>(new_pool_dev) : c->pool;
  std::vector<int64_t> owner(new_S, -1), recency(new_S, -1);
  for (int p = 0; p < n_keep; ++p) {
    owner[p] = c->owner[from[p]];
    recency[p] = c->recency[from[p]];
  }
  std::vector<int32_t> where((size_t)c->L * c->E, -1);
  for (int p = 0; p < n_keep; ++p) where[owner[p]] = p;

  if (dev) {
    hipStream_t sd = reinterpret_cast<hipStream_t>(side);
    hipStream_t cp = reinterpret_cast<hipStream_t>(compute);
    // every fill already issued on `side` lands before anything moves
    hipError_t err = hipEventRecord(c->side_done, sd);
    if (err == hipSuccess) err = hipStreamWaitEvent(cp, c->side_done, 0);
    for (int p = 0; err == hipSuccess && p < n_keep; ++p) {
      if (dst_pool == c->pool && from[p] == p) continue;
      err = hipMemcpyAsync(dst_pool + (size_t)p * c->slot_bytes,
                           c->pool + (size_t)from[p] * c->slot_bytes, c->slot_bytes,
                           hipMemcpyDeviceToDevice, cp);
    }
    if (err == hipSuccess)
      err = hipMemcpyAsync(c->table_dev, where.data(), sizeof(int32_t) * where.size(),
                           hipMemcpyHostToDevice, cp);
    if (err == hipSuccess) err = hipStreamSynchronize(cp);
    if (err != hipSuccess)
      return set_error(MOE_ERR_HIP, "moe_cache_resize: %s", hipGetErrorString(err));
  }
  c->pool = dst_pool;
  c->S = new_S;
  c->owner.swap(owner);
  c->recency.swap(recency);
  c->where.swap(where);
  for (int p = 0; p < n_keep; ++p) {
    if (move_from) move_from[p] = from[p];
    if (move_to) move_to[p] = p;
  }
  if (n_moves) *n_moves = n_keep;
  return MOE_OK;
}

extern "C" int moe_cache_stats(moe_cache_t c, int64_t* steps, int64_t* hits, int64_t* misses,
                               int64_t* bytes_filled) {
  if (!c) return set_error(MOE_ERR_INVALID_ARG, "moe_cache_stats: null handle");
  if (steps) *steps = c->st_steps;
  if (hits) *hits = c->st_hits;
  if (misses) *misses = c->st_misses;
  if (bytes_filled) *bytes_filled = c->st_bytes;
  return MOE_OK;
}
