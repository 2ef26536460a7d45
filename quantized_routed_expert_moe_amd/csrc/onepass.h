// One-pass routing of one token: the router GEMV and the top-k selection in one
// dispatch ("Strata on a Mac", Switches: the Metal build can fuse the router
// GEMV and moe_route into one dispatch; the same page reports that handing the
// logits to the last threadgroup with relaxed atomics alone gave it stale logits).
//
// Hand-off without fences or shared counters: every value another workgroup
// needs travels in its own 64-bit word (epoch << 32 | value), written with a
// device-scope relaxed store and read with device-scope relaxed loads (on
// gfx950 these bypass the per-XCD L2: global_store/global_load ... sc1). A word
// is fresh when its epoch equals this call's, so no ordering between words is
// needed and no L2 writeback or invalidation is issued. The calls on one
// workspace number themselves: word 0 holds the number of the last completed
// call, each call uses epoch = word 0 + 1, and word 0 is advanced only once
// every workgroup of the call has read it. A workspace region starts at zero
// (the caller zeroes it once), so no stale word can carry the current epoch.
//
// Region (64-bit words): [0] epoch of the last call; [1 + e] logit of expert e;
// [onepass_slot_word(E, k, c)] copy c of the slot of the expert of rank k
// (moe_layer's one-pass path).
#pragma once

#include "moe_internal.h"
#include "wave_ops.h"

namespace moe {

constexpr int kOnepassSpinLimit = 1 << 21;  // polls (each one memory round trip) before giving up

__device__ inline uint64_t ll_load(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ inline void ll_store(uint64_t* p, uint32_t epoch, uint32_t value) {
  __hip_atomic_store(p, ((uint64_t)epoch << 32) | value, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// This call's epoch (the same on every workgroup of the call).
__device__ inline uint32_t onepass_epoch(const uint64_t* words) { return (uint32_t)ll_load(words) + 1u; }

// Workgroup e of the GEMV part: logit e into its word.
__device__ inline void onepass_publish_logit(const uint16_t* x, const float* wr, int H, int e, uint64_t* words,
                                             uint32_t ep, double* part) {
  const double s = router_row_sum(x, wr + (size_t)e * H, H, part);
  if (threadIdx.x == 0) ll_store(words + 1 + e, ep, __float_as_uint((float)s));
}

// The selector (one wave, lanes 0..63): waits until all E logit words carry
// this epoch; lane l gets lg[i] = logit of expert l * EPL + i (0 past E), the
// blocked layout of wave_topk. Every poll
// issues all of its loads before it waits (one round trip per poll). Returns
// false when the words did not arrive within the spin limit (status set).
template <int EPL>
__device__ inline bool onepass_wait_logits(const uint64_t* words, int E, uint32_t ep, int32_t* status,
                                           float (&lg)[EPL]) {
  const int lane = threadIdx.x & 63;
  for (int spins = 0;; ++spins) {
    uint64_t v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      v[i] = ll_load(words + 1 + (e < E ? e : E - 1));
    }
    bool fresh = true;
#pragma unroll
    for (int i = 0; i < EPL; ++i) fresh = fresh && (uint32_t)(v[i] >> 32) == ep;
    if (__ballot(!fresh) == 0) {
#pragma unroll
      for (int i = 0; i < EPL; ++i) lg[i] = lane * EPL + i < E ? __uint_as_float((uint32_t)v[i]) : 0.0f;
      return true;
    }
    if (spins >= kOnepassSpinLimit) {
      if (lane == 0) *status = MOE_EHIP;
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// Lane l writes the logits of experts l * EPL + i (stores are issued after the
// selection and the hand-off, so that no wait for them lands on the critical path).
template <int EPL>
__device__ inline void onepass_store_logits(const float (&lg)[EPL], int E, float* logits) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane * EPL + i < E) logits[lane * EPL + i] = lg[i];
}

// Wait for copy `copy` of rank k's slot word of this epoch (moe_layer's one-pass
// path); every lane of the calling wave gets the slot, or INT32_MIN after the
// spin limit.
__device__ inline int32_t onepass_wait_slot(const uint64_t* words, int E, int k, uint32_t ep, int copy) {
  for (int spins = 0; spins < kOnepassSpinLimit; ++spins) {
    const uint64_t v = ll_load(words + onepass_slot_word(E, k, copy));
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    if (hi == ep) return (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    __builtin_amdgcn_s_sleep(2);
  }
  return INT32_MIN;
}

}  // namespace moe
