// Fixed-slot expert arena: host-side slot policy and asynchronous fills.
//
// One arena per layer ("Strata on a Mac", Status: an expert cache of 64 slots).
// The policy is a deterministic LRU ("Strata" README, Architecture: routed
// experts leased into device memory per decode step through an LRU cache);
// see moe.h for the exact rule. Misses are filled with one asynchronous copy
// per expert from a pinned host source (one contiguous read per expert,
// "Strata on a Mac", What you need), on a caller-chosen side stream. Read-ahead
// (arena_prefetch) maps predicted experts with the same eviction rule; it
// changes which bytes are in the slots early, never what a later call computes.
#include <new>
#include <vector>

#include "arena_internal.h"

extern "C" int arena_create(int E, int S, size_t blob_bytes, size_t stride, void* slots_dev,
                            int32_t* slot_table_dev, const void* host_src, moe_arena** out) {
  if (!out || E <= 0 || S <= 0 || E > (1 << 24) || S > (1 << 24) || blob_bytes == 0 || stride < blob_bytes)
    return MOE_EINVAL;
  moe_arena* a = new (std::nothrow) moe_arena;
  if (!a) return MOE_EINVAL;
  a->E = E;
  a->S = S;
  a->blob_bytes = blob_bytes;
  a->stride = stride;
  a->slots_dev = static_cast<uint8_t*>(slots_dev);
  a->table_dev = slot_table_dev;
  a->host_src = static_cast<const uint8_t*>(host_src);
  a->slot_of.assign(E, -1);
  a->expert_in.assign(S, -1);
  a->stamp.assign(S, 0);
  a->prefetched.assign(S, 0);
  a->req_mark.assign(E, 0);
  *out = a;
  return MOE_OK;
}

extern "C" void arena_destroy(moe_arena* a) {
  if (a && a->fill_event) (void)hipEventDestroy(a->fill_event);
  delete a;
}

extern "C" int arena_reset(moe_arena* a) {
  if (!a) return MOE_EINVAL;
  a->slot_of.assign(a->E, -1);
  a->expert_in.assign(a->S, -1);
  a->stamp.assign(a->S, 0);
  a->prefetched.assign(a->S, 0);
  a->calls = 0;
  a->stats = moe_arena_stats{};
  a->last_fills.clear();
  a->last_evicted.clear();
  return MOE_OK;
}

extern "C" int arena_stats(const moe_arena* a, moe_arena_stats* out) {
  if (!a || !out) return MOE_EINVAL;
  *out = a->stats;
  return MOE_OK;
}

extern "C" int arena_slot_table(const moe_arena* a, int32_t* slot_of) {
  if (!a || !slot_of) return MOE_EINVAL;
  for (int e = 0; e < a->E; ++e) slot_of[e] = a->slot_of[e];
  return MOE_OK;
}

extern "C" int arena_place(moe_arena* a, int expert, int slot) {
  if (!a || expert < 0 || expert >= a->E || slot < 0 || slot >= a->S) return MOE_EINVAL;
  const int old = a->expert_in[slot];
  if (old >= 0) a->slot_of[old] = -1;
  const int prev = a->slot_of[expert];
  if (prev >= 0) a->expert_in[prev] = -1;
  a->expert_in[slot] = expert;
  a->slot_of[expert] = slot;
  a->stamp[slot] = 0;
  a->prefetched[slot] = 0;
  return MOE_OK;
}

namespace {

// Checks the ids and de-duplicates them in first-occurrence order; the experts
// of this call are marked in req_mark. MOE_ENOSLOT leaves the arena as it was
// (but for the marks, which only ever compare equal to the current call's).
int distinct_ids(moe_arena* a, const int32_t* ids, int n, std::vector<int32_t>& distinct) {
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= a->E) return MOE_EINVAL;
  const uint64_t mark = ++a->marker;
  distinct.clear();
  distinct.reserve(n);
  for (int i = 0; i < n; ++i) {
    if (a->req_mark[ids[i]] != mark) {
      a->req_mark[ids[i]] = mark;
      distinct.push_back(ids[i]);
    }
  }
  return (int)distinct.size() > a->S ? MOE_ENOSLOT : MOE_OK;
}

// Places expert e (not resident) with stamp now: the lowest empty slot, else the
// slot of the oldest expert not marked in this call (ties to the lower slot).
// Records the fill and what it evicted.
void place_miss(moe_arena* a, int e, uint64_t now, bool by_prefetch) {
  int victim_slot = -1;
  for (int s = 0; s < a->S; ++s)
    if (a->expert_in[s] < 0) {
      victim_slot = s;
      break;
    }
  int evicted = -1;
  if (victim_slot < 0) {
    for (int s = 0; s < a->S; ++s) {
      const int r = a->expert_in[s];
      if (a->req_mark[r] == a->marker) continue;  // named in this call: protected
      if (victim_slot < 0 || a->stamp[s] < a->stamp[victim_slot]) victim_slot = s;
    }
    evicted = a->expert_in[victim_slot];
    a->slot_of[evicted] = -1;
    a->stats.evictions++;
  }
  a->expert_in[victim_slot] = e;
  a->slot_of[e] = victim_slot;
  a->stamp[victim_slot] = now;
  a->prefetched[victim_slot] = by_prefetch ? 1 : 0;
  a->last_fills.push_back(moe_fill{e, victim_slot});
  a->last_evicted.push_back(evicted);
  a->stats.fills++;
  a->stats.h2d_bytes += a->blob_bytes;
}

void copy_fills(const moe_arena* a, moe_fill* fills, int* n_fills) {
  for (size_t i = 0; i < a->last_fills.size(); ++i) fills[i] = a->last_fills[i];
  *n_fills = (int)a->last_fills.size();
}

}  // namespace

extern "C" int arena_map_slots(moe_arena* a, const int32_t* ids, int n, int32_t* slots, moe_fill* fills,
                               int* n_fills) {
  if (!a || n < 0 || (n > 0 && (!ids || !slots || !fills)) || !n_fills) return MOE_EINVAL;
  std::vector<int32_t> distinct;
  const int rc = distinct_ids(a, ids, n, distinct);
  if (rc != MOE_OK) return rc;
  const uint64_t now = ++a->calls;
  std::vector<int32_t> misses;
  for (int e : distinct) {
    const int s = a->slot_of[e];
    if (s >= 0) {
      a->stamp[s] = now;
      a->stats.hits++;
      if (a->prefetched[s]) {
        a->stats.prefetch_hits++;
        a->prefetched[s] = 0;
      }
    } else {
      misses.push_back(e);
    }
  }
  a->last_fills.clear();
  a->last_evicted.clear();
  for (int e : misses) {
    place_miss(a, e, now, false);
    a->stats.misses++;
  }
  for (int i = 0; i < n; ++i) slots[i] = a->slot_of[ids[i]];
  copy_fills(a, fills, n_fills);
  return MOE_OK;
}

extern "C" int arena_prefetch(moe_arena* a, const int32_t* ids, int n, moe_fill* fills, int* n_fills) {
  if (!a || n < 0 || (n > 0 && (!ids || !fills)) || !n_fills) return MOE_EINVAL;
  std::vector<int32_t> distinct;
  const int rc = distinct_ids(a, ids, n, distinct);
  if (rc != MOE_OK) return rc;
  const uint64_t now = ++a->calls;
  a->last_fills.clear();
  a->last_evicted.clear();
  for (int e : distinct)
    if (a->slot_of[e] < 0) {  // a resident prediction is left as it is
      place_miss(a, e, now, true);
      a->stats.prefetch_fills++;
    }
  copy_fills(a, fills, n_fills);
  return MOE_OK;
}

extern "C" int arena_fill_async(moe_arena* a, const moe_fill* fills, int n_fills, moe_stream_t side,
                                moe_event_t done) {
  if (!a || n_fills < 0 || (n_fills > 0 && !fills)) return MOE_EINVAL;
  if (!a->slots_dev || !a->table_dev || !a->host_src) return MOE_EINVAL;
  if ((size_t)n_fills != a->last_fills.size()) return MOE_EINVAL;
  for (int i = 0; i < n_fills; ++i)
    if (fills[i].expert != a->last_fills[i].expert || fills[i].slot != a->last_fills[i].slot) return MOE_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(side);
  std::vector<int32_t> idx, val;
  for (int i = 0; i < n_fills; ++i) {
    const moe_fill f = fills[i];
    if (hipMemcpyAsync(a->slots_dev + (size_t)f.slot * a->stride, a->host_src + (size_t)f.expert * a->stride,
                       a->blob_bytes, hipMemcpyHostToDevice, s) != hipSuccess)
      return MOE_EHIP;
    if (a->last_evicted[i] >= 0) {
      idx.push_back(a->last_evicted[i]);
      val.push_back(-1);
    }
  }
  for (int i = 0; i < n_fills; ++i) {
    idx.push_back(fills[i].expert);
    val.push_back(fills[i].slot);
  }
  if (!idx.empty() && moe::launch_table_update(a->table_dev, idx.data(), val.data(), (int)idx.size(), s) != hipSuccess)
    return MOE_EHIP;
  a->last_fills.clear();
  a->last_evicted.clear();
  if (n_fills > 0) {
    if (!a->fill_event && hipEventCreateWithFlags(&a->fill_event, hipEventDisableTiming) != hipSuccess) {
      a->fill_event = nullptr;
      return MOE_EHIP;
    }
    if (hipEventRecord(a->fill_event, s) != hipSuccess) return MOE_EHIP;
  }
  if (done && hipEventRecord(static_cast<hipEvent_t>(done), s) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

// Chunked paged runs: the distinct experts of a chunk, resident ones first, cut
// into passes that each fit the arena (each pass then maps, fills and computes
// its experts; the chunk's outputs are combined after the last pass).
extern "C" int arena_chunk_passes(const moe_arena* a, const int32_t* ids, int n, int max_per_pass,
                                  int32_t* experts, int32_t* pass_end, int* n_distinct, int* n_passes) {
  if (!a || n < 0 || (n > 0 && (!ids || !experts || !pass_end)) || !n_distinct || !n_passes) return MOE_EINVAL;
  if (max_per_pass < 1 || max_per_pass > a->S) return MOE_EINVAL;
  for (int i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= a->E) return MOE_EINVAL;
  std::vector<uint8_t> used(a->E, 0);
  for (int i = 0; i < n; ++i) used[ids[i]] = 1;
  int m = 0;
  for (int e = 0; e < a->E; ++e)
    if (used[e] && a->slot_of[e] >= 0) experts[m++] = e;
  for (int e = 0; e < a->E; ++e)
    if (used[e] && a->slot_of[e] < 0) experts[m++] = e;
  int p = 0;
  for (int end = 0; end < m;) {
    end = end + max_per_pass < m ? end + max_per_pass : m;
    pass_end[p++] = end;
  }
  *n_distinct = m;
  *n_passes = p;
  return MOE_OK;
}
