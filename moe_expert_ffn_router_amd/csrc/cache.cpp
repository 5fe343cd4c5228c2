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
constexpr int kWaveRing = 16;   // pinned per-wave records of moe_expert_ffn_streamed

struct Cache {
  int L = 0, E = 0, S = 0;
  int64_t slot_bytes = 0;
  uint8_t* pool = nullptr;
  const uint8_t* bank = nullptr;
  int32_t* table_dev = nullptr;
  std::vector<int64_t> owner;    // per slot: layer*E + expert, or -1
  std::vector<int64_t> recency;  // per slot: last active step
  std::vector<int32_t> where;    // per (layer, expert): slot or -1
  std::vector<int64_t> last_active;  // per (layer, expert): last step it was needed, or -1
  int64_t clock = 0;
  int64_t st_steps = 0, st_hits = 0, st_misses = 0, st_bytes = 0;
  int32_t* ring = nullptr;  // pinned [kRing][E]
  hipEvent_t ring_done[kRing] = {};
  bool ring_used[kRing] = {};
  int ring_next = 0;
  hipEvent_t compute_mark = nullptr, side_done = nullptr;
  hipEvent_t group_done[kMaxGroups] = {};
  // streamed steps: pinned per-wave records [kWaveRing][(2 + kMaxGroups) * E]
  // (the wave's slot-table row, then the masked counts of its hit set and of
  // each fill group), the events that free them, and the end of each wave's
  // expert FFN work on the compute stream (two: waves w-1 and w-2)
  int32_t* wave_rec = nullptr;
  hipEvent_t wave_rec_done[kWaveRing] = {};
  bool wave_rec_used[kWaveRing] = {};
  int wave_rec_next = 0;
  hipEvent_t ffn_done[2] = {};
  // hybrid steps: the host staging (x, offsets, sorted_idx copied down) has
  // landed; the CPU experts' rows have been copied up (the staging is free)
  hipEvent_t stage_in = nullptr, cpu_rows_done = nullptr;
  bool cpu_rows_used = false;
  // host scratch of one planned step (kept across calls)
  std::vector<int32_t> plan_wave_of, plan_fill_e, plan_fill_s, plan_wave_end, plan_rows;
  std::vector<int32_t> plan_order, plan_wave_start;
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
  c->last_active.assign((size_t)n_layers * E, -1);
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
    for (int i = 0; ok && i < kWaveRing; ++i)
      ok = hipEventCreateWithFlags(&c->wave_rec_done[i], hipEventDisableTiming) == hipSuccess;
    for (int i = 0; ok && i < 2; ++i)
      ok = hipEventCreateWithFlags(&c->ffn_done[i], hipEventDisableTiming) == hipSuccess;
    ok = ok && hipEventCreateWithFlags(&c->stage_in, hipEventDisableTiming) == hipSuccess &&
         hipEventCreateWithFlags(&c->cpu_rows_done, hipEventDisableTiming) == hipSuccess;
    ok = ok && hipHostMalloc((void**)&c->wave_rec,
                             sizeof(int32_t) * kWaveRing * (2 + kMaxGroups) * E,
                             hipHostMallocDefault) == hipSuccess;
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
  for (int i = 0; i < kWaveRing; ++i)
    if (c->wave_rec_done[i]) {
      if (c->wave_rec_used[i]) (void)hipEventSynchronize(c->wave_rec_done[i]);
      (void)hipEventDestroy(c->wave_rec_done[i]);
    }
  for (int i = 0; i < 2; ++i)
    if (c->ffn_done[i]) (void)hipEventDestroy(c->ffn_done[i]);
  if (c->cpu_rows_done) {
    if (c->cpu_rows_used) (void)hipEventSynchronize(c->cpu_rows_done);
    (void)hipEventDestroy(c->cpu_rows_done);
  }
  if (c->stage_in) (void)hipEventDestroy(c->stage_in);
  if (c->wave_rec) (void)hipHostFree(c->wave_rec);
  if (c->compute_mark) (void)hipEventDestroy(c->compute_mark);
  if (c->side_done) (void)hipEventDestroy(c->side_done);
  if (c->ring) (void)hipHostFree(c->ring);
  delete c;
}

// One step of the policy over `needed` (ascending experts of `layer`, at most
// S of them): misses take the lowest empty slot, else the slot not needed now
// with the smallest (last-active step, slot index); every needed slot's
// last-active step becomes the clock; the clock advances.  Returns the number
// of misses, written in order to miss_expert / miss_slot.
static int lookup_core(Cache* c, int layer, const int* needed, int n_needed, int32_t* miss_expert,
                       int32_t* miss_slot) {
  const int E = c->E, S = c->S;
  const int64_t key0 = (int64_t)layer * E;
  std::vector<char> is_needed_slot(S, 0);
  for (int i = 0; i < n_needed; ++i) {
    const int s = c->where[key0 + needed[i]];
    if (s >= 0) is_needed_slot[s] = 1;
  }
  int nm = 0;
  int next_empty = 0;
  for (int i = 0; i < n_needed; ++i) {
    const int e = needed[i];
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
      // n_needed <= S guarantees a candidate; evict its owner
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
  for (int i = 0; i < n_needed; ++i) {
    c->recency[c->where[key0 + needed[i]]] = c->clock;
    c->last_active[key0 + needed[i]] = c->clock;
  }
  c->clock += 1;
  c->st_steps += 1;
  c->st_hits += n_needed - nm;
  c->st_misses += nm;
  return nm;
}

static int check_counts(const Cache* c, const int32_t* counts_host, std::vector<int>& needed,
                        const char* who) {
  needed.clear();
  for (int e = 0; e < c->E; ++e) {
    if (counts_host[e] < 0)
      return set_error(MOE_ERR_INVALID_ARG, "%s: counts[%d] < 0", who, e);
    if (counts_host[e] > 0) needed.push_back(e);
  }
  return MOE_OK;
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
  if (int st = check_counts(c, counts_host, needed, "expert_cache_lookup")) return st;
  if ((int)needed.size() > S)
    return set_error(MOE_ERR_CAPACITY,
                     "expert_cache_lookup: layer %d needs %d distinct experts, pool has %d slots",
                     layer, (int)needed.size(), S);
  const int nm = lookup_core(c, layer, needed.data(), (int)needed.size(), miss_expert, miss_slot);
  *n_miss = nm;
  *n_hit = (int)needed.size() - nm;
  if (slot_row_host)
    for (int e = 0; e < E; ++e) slot_row_host[e] = c->where[(int64_t)layer * E + e];
  return MOE_OK;
}

// The policy for one step in waves (see expert_cache_plan in the header):
// the step's experts in waves of at most S (one wave) or floor(S/2) (several;
// resident experts first, then the others, each ascending), one lookup per
// wave.  Fills go to c->plan_fill_e / plan_fill_s in order, wave w's fills
// end at c->plan_wave_end[w], its experts are plan_order[plan_wave_start[w]
// .. plan_wave_start[w+1]), and the layer's slot-table row after wave w is
// c->plan_rows[w * E ..].  Returns the number of waves.
static int plan_step(Cache* c, int layer, const std::vector<int>& needed) {
  const int E = c->E, S = c->S, n = (int)needed.size();
  const int64_t key0 = (int64_t)layer * E;
  c->plan_order.clear();
  if (n <= S) {
    c->plan_order.assign(needed.begin(), needed.end());
  } else {
    for (int e : needed)
      if (c->where[key0 + e] >= 0) c->plan_order.push_back(e);
    for (int e : needed)
      if (c->where[key0 + e] < 0) c->plan_order.push_back(e);
  }
  const int size = n <= S ? (n > 0 ? n : 1) : (S / 2 > 0 ? S / 2 : 1);
  const int n_waves = (n + size - 1) / size;
  c->plan_fill_e.resize(n > 0 ? n : 1);
  c->plan_fill_s.resize(n > 0 ? n : 1);
  c->plan_wave_end.resize(n_waves > 0 ? n_waves : 1);
  c->plan_wave_start.resize(n_waves + 1);
  c->plan_rows.resize((size_t)(n_waves > 0 ? n_waves : 1) * E);
  std::vector<int> wave;
  int nf = 0;
  for (int w = 0; w < n_waves; ++w) {
    const int i0 = w * size, i1 = i0 + size < n ? i0 + size : n;
    c->plan_wave_start[w] = i0;
    wave.assign(c->plan_order.begin() + i0, c->plan_order.begin() + i1);
    std::sort(wave.begin(), wave.end());
    nf += lookup_core(c, layer, wave.data(), (int)wave.size(), c->plan_fill_e.data() + nf,
                      c->plan_fill_s.data() + nf);
    c->plan_wave_end[w] = nf;
    for (int e = 0; e < E; ++e) c->plan_rows[(size_t)w * E + e] = c->where[key0 + e];
  }
  c->plan_wave_start[n_waves] = n;
  return n_waves;
}

extern "C" int expert_cache_plan(moe_cache_t c, int32_t layer, const int32_t* counts_host,
                                 int32_t* wave_of_expert, int32_t* fill_expert,
                                 int32_t* fill_slot, int32_t* wave_fill_end, int32_t* n_waves,
                                 int32_t* n_hit) {
  if (!c || !counts_host || !n_waves)
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_plan: null argument");
  if (layer < 0 || layer >= c->L)
    return set_error(MOE_ERR_INVALID_ARG, "expert_cache_plan: layer %d of %d", layer, c->L);
  std::vector<int> needed;
  if (int st = check_counts(c, counts_host, needed, "expert_cache_plan")) return st;
  const int nw = plan_step(c, layer, needed);
  const int nf = nw > 0 ? c->plan_wave_end[nw - 1] : 0;
  if (wave_of_expert) {
    for (int e = 0; e < c->E; ++e) wave_of_expert[e] = -1;
    for (int w = 0; w < nw; ++w)
      for (int i = c->plan_wave_start[w]; i < c->plan_wave_start[w + 1]; ++i)
        wave_of_expert[c->plan_order[i]] = w;
  }
  for (int i = 0; i < nf; ++i) {
    if (fill_expert) fill_expert[i] = c->plan_fill_e[i];
    if (fill_slot) fill_slot[i] = c->plan_fill_s[i];
  }
  if (wave_fill_end)
    for (int w = 0; w < nw; ++w) wave_fill_end[w] = c->plan_wave_end[w];
  *n_waves = nw;
  if (n_hit) *n_hit = (int)needed.size() - nf;
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

// ---------------------------------------------------------------------------
// One (layer-)step of the expert FFN through the slot pool, streamed: the
// policy in waves (plan_step), each wave's misses copied on `side` in groups,
// the FFN over the wave's hit experts at once and over each group once it has
// landed.  Two staging sets: wave w's copies wait only for the FFN work of
// wave w-2 (all of it, and all work enqueued before the call), unless one of
// its victims is a slot wave w-1 reads (only with S = 1), then for wave w-1.
// Every FFN call is moe_expert_ffn with the counts of the experts outside its
// set zeroed, so the tiles and results equal those of one call over all.
// ---------------------------------------------------------------------------
extern "C" size_t moe_expert_ffn_streamed_workspace(const moe_experts* W, int32_t T, int32_t k) {
  if (!W) return 0;
  const size_t ffn = moe_expert_ffn_workspace(W, T, k);
  const size_t masks = (size_t)(1 + kMaxGroups) * W->E * sizeof(int32_t);
  return (ffn + 255) / 256 * 256 + (masks + 255) / 256 * 256;
}

// Plans `needed` (ascending) as plan_step does and enqueues the grouped fills
// and the FFN launches; gpu_counts (host [E]) holds the counts of the experts
// the GPU computes (others zero).  Returns the number of waves in *n_waves.
static int streamed_core(Cache* c, int layer, const moe_experts* pool_W, const uint16_t* x,
                         int T, int k, const int32_t* gpu_counts, const std::vector<int>& needed,
                         const int32_t* offsets, const int32_t* sorted_idx, uint16_t* y_perm,
                         int n_groups, void* ws, moe_stream_t side, moe_stream_t compute,
                         int* n_waves) {
  const char* who = "moe_expert_ffn_streamed";
  const int32_t* counts_host = gpu_counts;
  const int E = c->E;
  const size_t ffn_ws = (moe_expert_ffn_workspace(pool_W, T, k) + 255) / 256 * 256;
  int32_t* masks_dev = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + ffn_ws);
  int32_t* row_dev = c->table_dev + (int64_t)layer * E;
  hipStream_t sd = reinterpret_cast<hipStream_t>(side);
  hipStream_t cp = reinterpret_cast<hipStream_t>(compute);

  const int nw = plan_step(c, layer, needed);
  hipError_t err = hipEventRecord(c->compute_mark, cp);  // all work enqueued before the call
  int st = MOE_OK;
  for (int w = 0; w < nw && err == hipSuccess && st == MOE_OK; ++w) {
    const int f0 = w ? c->plan_wave_end[w - 1] : 0, f1 = c->plan_wave_end[w];
    const int nm = f1 - f0;
    const int G = nm < n_groups ? nm : n_groups;
    // the wave's record: slot-table row, masked counts of its hits and groups
    const int r = c->wave_rec_next;
    c->wave_rec_next = (r + 1) % kWaveRing;
    if (c->wave_rec_used[r] && hipEventSynchronize(c->wave_rec_done[r]) != hipSuccess)
      return set_error(MOE_ERR_HIP, "%s: record wait failed", who);
    int32_t* rec = c->wave_rec + (size_t)r * (2 + kMaxGroups) * E;
    int32_t* row = rec;
    int32_t* masks = rec + E;
    memcpy(row, c->plan_rows.data() + (size_t)w * E, sizeof(int32_t) * E);
    memset(masks, 0, sizeof(int32_t) * (size_t)(1 + G) * E);
    std::vector<char> is_miss(E, 0);
    for (int i = f0; i < f1; ++i) is_miss[c->plan_fill_e[i]] = 1;
    int n_hit = 0;
    for (int i = c->plan_wave_start[w]; i < c->plan_wave_start[w + 1]; ++i) {
      const int e = c->plan_order[i];
      if (!is_miss[e]) {
        masks[e] = counts_host[e];
        ++n_hit;
      }
    }
    for (int g = 0; g < G; ++g) {
      const int i0 = f0 + (int)((int64_t)nm * g / G), i1 = f0 + (int)((int64_t)nm * (g + 1) / G);
      for (int i = i0; i < i1; ++i) {
        const int e = c->plan_fill_e[i];
        masks[(size_t)(1 + g) * E + e] = counts_host[e];
      }
    }
    err = hipMemcpyAsync(row_dev, row, sizeof(int32_t) * E, hipMemcpyHostToDevice, cp);
    if (err == hipSuccess)
      err = hipMemcpyAsync(masks_dev, masks, sizeof(int32_t) * (size_t)(1 + G) * E,
                           hipMemcpyHostToDevice, cp);
    if (err == hipSuccess) err = hipEventRecord(c->wave_rec_done[r], cp);
    if (err != hipSuccess) break;
    c->wave_rec_used[r] = true;
    // copies: wait for the FFN work whose slots they may overwrite
    if (nm > 0) {
      bool hits_prev = false;
      if (w > 0) {
        const int32_t* prow = c->plan_rows.data() + (size_t)(w - 1) * E;
        for (int i = c->plan_wave_start[w - 1]; i < c->plan_wave_start[w] && !hits_prev; ++i) {
          const int ps = prow[c->plan_order[i]];
          for (int j = f0; j < f1; ++j)
            if (c->plan_fill_s[j] == ps) { hits_prev = true; break; }
        }
      }
      hipEvent_t dep = hits_prev ? c->ffn_done[(w - 1) & 1]
                       : (w >= 2 ? c->ffn_done[w & 1] : c->compute_mark);
      err = hipStreamWaitEvent(sd, dep, 0);
      for (int g = 0; err == hipSuccess && g < G; ++g) {
        const int i0 = f0 + (int)((int64_t)nm * g / G), i1 = f0 + (int)((int64_t)nm * (g + 1) / G);
        for (int i = i0; err == hipSuccess && i < i1; ++i) {
          const int e = c->plan_fill_e[i], s = c->plan_fill_s[i];
          err = hipMemcpyAsync(c->pool + (size_t)s * c->slot_bytes,
                               c->bank + ((size_t)layer * E + e) * c->slot_bytes, c->slot_bytes,
                               hipMemcpyHostToDevice, sd);
        }
        if (err == hipSuccess) err = hipEventRecord(c->group_done[g], sd);
      }
      if (err != hipSuccess) break;
      c->st_bytes += (int64_t)nm * c->slot_bytes;
    }
    // expert FFN: the hits now, each group once it has landed
    if (n_hit > 0)
      st = moe_expert_ffn(pool_W, row_dev, x, T, k, masks_dev, offsets, sorted_idx, y_perm, 0, ws,
                          ffn_ws, compute);
    for (int g = 0; g < G && st == MOE_OK && err == hipSuccess; ++g) {
      err = hipStreamWaitEvent(cp, c->group_done[g], 0);
      if (err == hipSuccess)
        st = moe_expert_ffn(pool_W, row_dev, x, T, k, masks_dev + (size_t)(1 + g) * E, offsets,
                            sorted_idx, y_perm, 0, ws, ffn_ws, compute);
    }
    if (err == hipSuccess && st == MOE_OK) err = hipEventRecord(c->ffn_done[w & 1], cp);
  }
  *n_waves = nw;
  if (st != MOE_OK) return st;
  if (err != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", who, hipGetErrorString(err));
  return MOE_OK;
}

static void plan_outputs(const Cache* c, int nw, int32_t* fill_expert, int32_t* fill_slot,
                         int32_t* wave_fill_end) {
  const int nf = nw > 0 ? c->plan_wave_end[nw - 1] : 0;
  for (int i = 0; i < nf; ++i) {
    if (fill_expert) fill_expert[i] = c->plan_fill_e[i];
    if (fill_slot) fill_slot[i] = c->plan_fill_s[i];
  }
  if (wave_fill_end)
    for (int w = 0; w < nw; ++w) wave_fill_end[w] = c->plan_wave_end[w];
}

static int check_stream_args(const Cache* c, int layer, const moe_experts* pool_W, int T, int k,
                             int n_groups, void* ws, size_t ws_bytes, const char* who) {
  if (!c->pool || !c->bank || !c->table_dev || !c->ring || !c->wave_rec)
    return set_error(MOE_ERR_INVALID_ARG, "%s: handle has no pool/bank/table", who);
  if (layer < 0 || layer >= c->L)
    return set_error(MOE_ERR_INVALID_ARG, "%s: layer %d of %d", who, layer, c->L);
  if (pool_W->E != c->E || pool_W->base != c->pool || pool_W->stride != c->slot_bytes)
    return set_error(MOE_ERR_INVALID_ARG,
                     "%s: pool_W must describe the cache's pool (E, base, stride)", who);
  if (n_groups < 1 || n_groups > kMaxGroups)
    return set_error(MOE_ERR_INVALID_ARG, "%s: n_groups %d not in [1, %d]", who, n_groups,
                     kMaxGroups);
  if (!ws || ws_bytes < moe_expert_ffn_streamed_workspace(pool_W, T, k))
    return set_error(MOE_ERR_WORKSPACE, "%s: workspace too small", who);
  return MOE_OK;
}

extern "C" int moe_expert_ffn_streamed(moe_cache_t c, int32_t layer, const moe_experts* pool_W,
                                       const uint16_t* x, int32_t T, int32_t k,
                                       const int32_t* counts_host, const int32_t* offsets,
                                       const int32_t* sorted_idx, uint16_t* y_perm,
                                       int32_t n_groups, void* ws, size_t ws_bytes,
                                       moe_stream_t side, moe_stream_t compute,
                                       int32_t* fill_expert, int32_t* fill_slot,
                                       int32_t* wave_fill_end, int32_t* n_waves_out,
                                       int32_t* n_hit_out) {
  const char* who = "moe_expert_ffn_streamed";
  if (!c || !pool_W || !counts_host)
    return set_error(MOE_ERR_INVALID_ARG, "%s: null argument", who);
  if (int st = check_stream_args(c, layer, pool_W, T, k, n_groups, ws, ws_bytes, who)) return st;
  std::vector<int> needed;
  if (int st = check_counts(c, counts_host, needed, who)) return st;
  int nw = 0;
  if (int st = streamed_core(c, layer, pool_W, x, T, k, counts_host, needed, offsets, sorted_idx,
                             y_perm, n_groups, ws, side, compute, &nw))
    return st;
  plan_outputs(c, nw, fill_expert, fill_slot, wave_fill_end);
  const int nf = nw > 0 ? c->plan_wave_end[nw - 1] : 0;
  if (n_waves_out) *n_waves_out = nw;
  if (n_hit_out) *n_hit_out = (int)needed.size() - nf;
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// Hybrid steps: n_fetch = ceil(q * misses) (at most max_fetch when >= 0) of
// the step's misses are fetched — the most recently active first (never
// active last, ties lower expert) — and the rest run on the CPU from the
// bank, taking no slot; the fetched misses and the hits are the GPU step
// (waves as in plan_step; with no GPU expert the clock still ticks).  CPU
// experts' last active step becomes the step's clock.
// ---------------------------------------------------------------------------
static int split_hybrid(Cache* c, int layer, const std::vector<int>& needed, double q,
                        int max_fetch, std::vector<int>& gpu, std::vector<int>& cpu) {
  const int64_t key0 = (int64_t)layer * c->E;
  std::vector<int> misses;
  for (int e : needed)
    if (c->where[key0 + e] < 0) misses.push_back(e);
  std::stable_sort(misses.begin(), misses.end(), [&](int a, int b) {
    return c->last_active[key0 + a] > c->last_active[key0 + b];  // ascending e among equals
  });
  int n_fetch = (int)ceil(q * (double)misses.size());
  if (max_fetch >= 0 && n_fetch > max_fetch) n_fetch = max_fetch;
  if (n_fetch > (int)misses.size()) n_fetch = (int)misses.size();
  if (n_fetch < 0) n_fetch = 0;
  std::vector<char> on_cpu(c->E, 0);
  cpu.assign(misses.begin() + n_fetch, misses.end());
  std::sort(cpu.begin(), cpu.end());
  for (int e : cpu) on_cpu[e] = 1;
  gpu.clear();
  for (int e : needed)
    if (!on_cpu[e]) gpu.push_back(e);
  return n_fetch;
}

static void finish_hybrid_clock(Cache* c, int layer, bool gpu_empty, const std::vector<int>& cpu) {
  if (gpu_empty) {  // a step with no GPU expert still advances the clock
    c->clock += 1;
    c->st_steps += 1;
  }
  const int64_t key0 = (int64_t)layer * c->E;
  for (int e : cpu) c->last_active[key0 + e] = c->clock - 1;
}

extern "C" int expert_cache_plan_hybrid(moe_cache_t c, int32_t layer, const int32_t* counts_host,
                                        double fetch_fraction, int32_t max_fetch,
                                        int32_t* cpu_expert, int32_t* n_cpu,
                                        int32_t* fill_expert, int32_t* fill_slot,
                                        int32_t* wave_fill_end, int32_t* n_waves,
                                        int32_t* n_hit) {
  const char* who = "expert_cache_plan_hybrid";
  if (!c || !counts_host || !n_waves || !n_cpu)
    return set_error(MOE_ERR_INVALID_ARG, "%s: null argument", who);
  if (layer < 0 || layer >= c->L)
    return set_error(MOE_ERR_INVALID_ARG, "%s: layer %d of %d", who, layer, c->L);
  if (!(fetch_fraction >= 0.0 && fetch_fraction <= 1.0))
    return set_error(MOE_ERR_INVALID_ARG, "%s: fetch_fraction must lie in [0, 1]", who);
  std::vector<int> needed, gpu, cpu;
  if (int st = check_counts(c, counts_host, needed, who)) return st;
  split_hybrid(c, layer, needed, fetch_fraction, max_fetch, gpu, cpu);
  const int nw = plan_step(c, layer, gpu);
  finish_hybrid_clock(c, layer, gpu.empty(), cpu);
  plan_outputs(c, nw, fill_expert, fill_slot, wave_fill_end);
  for (size_t i = 0; i < cpu.size(); ++i)
    if (cpu_expert) cpu_expert[i] = cpu[i];
  *n_cpu = (int)cpu.size();
  *n_waves = nw;
  const int nf = nw > 0 ? c->plan_wave_end[nw - 1] : 0;
  if (n_hit) *n_hit = (int)gpu.size() - nf;
  return MOE_OK;
}

static size_t al256(size_t v) { return (v + 255) / 256 * 256; }

extern "C" size_t moe_expert_ffn_hybrid_host_bytes(const moe_experts* pool_W, int32_t T,
                                                   int32_t k) {
  if (!pool_W || T < 0 || k < 1) return 0;
  const size_t A = (size_t)T * k;
  return al256((size_t)T * pool_W->H * 2) + al256(((size_t)pool_W->E + 1) * 4) + al256(A * 4) +
         al256(A * pool_W->H * 2);
}

extern "C" int moe_expert_ffn_hybrid(moe_cache_t c, int32_t layer, const moe_experts* pool_W,
                                     moe_cpu_pool_t cpu_pool, const uint16_t* x, int32_t T,
                                     int32_t k, const int32_t* counts_host,
                                     const int32_t* offsets, const int32_t* sorted_idx,
                                     uint16_t* y_perm, double fetch_fraction, int32_t max_fetch,
                                     int32_t n_groups, void* ws, size_t ws_bytes,
                                     void* host_stage, size_t host_bytes, moe_stream_t side,
                                     moe_stream_t compute, int32_t* cpu_expert, int32_t* n_cpu,
                                     int32_t* fill_expert, int32_t* fill_slot,
                                     int32_t* wave_fill_end, int32_t* n_waves, int32_t* n_hit) {
  const char* who = "moe_expert_ffn_hybrid";
  if (!c || !pool_W || !counts_host || !cpu_pool)
    return set_error(MOE_ERR_INVALID_ARG, "%s: null argument", who);
  if (int st = check_stream_args(c, layer, pool_W, T, k, n_groups, ws, ws_bytes, who)) return st;
  if (!(fetch_fraction >= 0.0 && fetch_fraction <= 1.0))
    return set_error(MOE_ERR_INVALID_ARG, "%s: fetch_fraction must lie in [0, 1]", who);
  if (!host_stage || host_bytes < moe_expert_ffn_hybrid_host_bytes(pool_W, T, k))
    return set_error(MOE_ERR_WORKSPACE, "%s: host staging too small", who);
  if (T > 0 && (!x || !offsets || !sorted_idx || !y_perm))
    return set_error(MOE_ERR_INVALID_ARG, "%s: null device pointer", who);
  std::vector<int> needed, gpu, cpu;
  if (int st = check_counts(c, counts_host, needed, who)) return st;
  const int E = c->E, H = pool_W->H;
  const size_t A = (size_t)T * k;
  uint8_t* hs = static_cast<uint8_t*>(host_stage);
  uint16_t* x_h = reinterpret_cast<uint16_t*>(hs);
  int32_t* off_h = reinterpret_cast<int32_t*>(hs + al256((size_t)T * H * 2));
  int32_t* sidx_h = reinterpret_cast<int32_t*>(hs + al256((size_t)T * H * 2) + al256(((size_t)E + 1) * 4));
  uint16_t* y_h = reinterpret_cast<uint16_t*>(hs + al256((size_t)T * H * 2) +
                                              al256(((size_t)E + 1) * 4) + al256(A * 4));
  hipStream_t cp = reinterpret_cast<hipStream_t>(compute);
  // the staging of the previous hybrid step is free once its rows went up
  if (c->cpu_rows_used && hipEventSynchronize(c->cpu_rows_done) != hipSuccess)
    return set_error(MOE_ERR_HIP, "%s: staging wait failed", who);
  split_hybrid(c, layer, needed, fetch_fraction, max_fetch, gpu, cpu);
  hipError_t err = hipSuccess;
  if (!cpu.empty()) {  // the CPU experts' inputs, down before the GPU work is queued
    err = hipMemcpyAsync(x_h, x, (size_t)T * H * 2, hipMemcpyDeviceToHost, cp);
    if (err == hipSuccess)
      err = hipMemcpyAsync(off_h, offsets, ((size_t)E + 1) * 4, hipMemcpyDeviceToHost, cp);
    if (err == hipSuccess) err = hipMemcpyAsync(sidx_h, sorted_idx, A * 4, hipMemcpyDeviceToHost, cp);
    if (err == hipSuccess) err = hipEventRecord(c->stage_in, cp);
    if (err != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", who, hipGetErrorString(err));
  }
  std::vector<int32_t> gpu_counts(counts_host, counts_host + E);
  for (int e : cpu) gpu_counts[e] = 0;
  int nw = 0;
  if (int st = streamed_core(c, layer, pool_W, x, T, k, gpu_counts.data(), gpu, offsets,
                             sorted_idx, y_perm, n_groups, ws, side, compute, &nw))
    return st;
  finish_hybrid_clock(c, layer, gpu.empty(), cpu);
  if (!cpu.empty()) {
    // the CPU's share runs now, while the GPU streams and computes its own
    if (hipEventSynchronize(c->stage_in) != hipSuccess)
      return set_error(MOE_ERR_HIP, "%s: staging copy failed", who);
    moe_experts bank_W = *pool_W;
    bank_W.base = c->bank + (size_t)layer * E * c->slot_bytes;
    if (int st = moe_cpu_expert_ffn(cpu_pool, &bank_W, cpu.data(), (int)cpu.size(), x_h, T, k,
                                    off_h, sidx_h, y_h))
      return st;
    for (size_t i = 0; err == hipSuccess && i < cpu.size(); ++i) {
      const int e = cpu[i], p0 = off_h[e], n = off_h[e + 1] - p0;
      if (n > 0)
        err = hipMemcpyAsync(y_perm + (size_t)p0 * H, y_h + (size_t)p0 * H, (size_t)n * H * 2,
                             hipMemcpyHostToDevice, cp);
    }
    if (err == hipSuccess) err = hipEventRecord(c->cpu_rows_done, cp);
    if (err != hipSuccess) return set_error(MOE_ERR_HIP, "%s: %s", who, hipGetErrorString(err));
    c->cpu_rows_used = true;
  }
  plan_outputs(c, nw, fill_expert, fill_slot, wave_fill_end);
  for (size_t i = 0; i < cpu.size(); ++i)
    if (cpu_expert) cpu_expert[i] = cpu[i];
  if (n_cpu) *n_cpu = (int)cpu.size();
  if (n_waves) *n_waves = nw;
  const int nf = nw > 0 ? c->plan_wave_end[nw - 1] : 0;
  if (n_hit) *n_hit = (int)gpu.size() - nf;
  return MOE_OK;
}
