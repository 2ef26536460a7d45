// Host metadata of a fixed-slot expert arena (arena.cpp owns the policy; the
// paged decode sequencer reads the device buffers and the fill event).
#pragma once
#include <vector>

#include "moe_internal.h"

struct moe_arena {
  int E = 0, S = 0;
  size_t blob_bytes = 0, stride = 0;
  uint8_t* slots_dev = nullptr;
  int32_t* table_dev = nullptr;
  const uint8_t* host_src = nullptr;
  std::vector<int32_t> slot_of;    // expert -> slot, -1 absent
  std::vector<int32_t> expert_in;  // slot -> expert, -1 empty
  std::vector<uint64_t> stamp;     // slot -> call number of last use
  std::vector<uint8_t> prefetched; // slot -> filled by arena_prefetch, not requested since
  std::vector<uint64_t> req_mark;  // expert -> call number that requested it
  uint64_t calls = 0;
  uint64_t marker = 0;             // distinct value per map call (also failed ones)
  moe_arena_stats stats{};
  std::vector<moe_fill> last_fills;
  std::vector<int32_t> last_evicted;  // per last fill: evicted expert or -1
  hipEvent_t fill_event = nullptr;     // recorded on the side stream after the last fills into this arena
};

// The last fills of this arena enqueued on the side stream are complete once
// this event has completed; nullptr while no fill was ever enqueued.
inline hipEvent_t arena_fill_event(const moe_arena* a) { return a->fill_event; }
