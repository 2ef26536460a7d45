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
// [1 + E + k] slot of the expert of rank k (moe_layer's one-pass path).
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

// The selector (one wave, lanes 0..63): waits for all E logit words of this
// epoch, writes the fp32 logits, and selects as moe_route does. Returns false
// when the words did not arrive within the spin limit (status set; id = -1).
template <int EPL>
__device__ inline bool onepass_select(const uint64_t* words, int E, int K, unsigned flags, uint32_t ep,
                                      float* logits, int32_t* status, int32_t& id, float& wt) {
  const int lane = threadIdx.x & 63;
  float lg[EPL];
  uint32_t got = 0;  // bit i: word of expert lane + 64 i is fresh
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + 64 * i >= E) got |= 1u << i;
  for (int spins = 0;; ++spins) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (!(got & (1u << i))) {
        const uint64_t v = ll_load(words + 1 + lane + 64 * i);
        if ((uint32_t)(v >> 32) == ep) {
          lg[i] = __uint_as_float((uint32_t)v);
          got |= 1u << i;
        }
      }
    }
    if (__ballot(got != (1u << EPL) - 1u) == 0) break;
    if (spins >= kOnepassSpinLimit) {
      if (lane == 0) *status = MOE_EHIP;
      id = -1;
      wt = 0.0f;
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e < E) logits[e] = lg[i];
    else lg[i] = 0.0f;
  }
  wave_select_values<EPL>(lg, E, K, flags, lane, id, wt);
  return true;
}

// Wait for word k (rank k's slot in moe_layer's one-pass path) of this epoch;
// every lane of the calling wave gets the slot, or INT32_MIN after the spin limit.
__device__ inline int32_t onepass_wait_slot(const uint64_t* words, int E, int k, uint32_t ep) {
  for (int spins = 0; spins < kOnepassSpinLimit; ++spins) {
    const uint64_t v = ll_load(words + 1 + E + k);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    if (hi == ep) return (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    __builtin_amdgcn_s_sleep(1);
  }
  return INT32_MIN;
}

}  // namespace moe
