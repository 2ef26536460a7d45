// Per-workgroup stamps of the instrumented build (include/moe_timeline.h for
// the row format). Without MOE_TIMELINE every function here is an empty inline
// and a kernel's code is unchanged.
//
// A translation unit that stamps kernels names its kernels' id range once, at
// namespace scope inside moe: MOE_TL_UNIT(name, first id, count). In the
// instrumented build that defines the unit's row buffer (a file-scope device
// array) and the host functions tl_read_<name> / tl_clear_<name>, which
// resolve the array's device address with hipGetSymbolAddress; api.cpp routes
// moe_timeline_read / moe_timeline_clear to them. Rows are written with
// ordinary vector stores (thread 0) and vector atomics (each wave's end).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_timeline.h"

namespace moe {

#ifdef MOE_TIMELINE

struct TlRow {
  uint64_t* row;  // nullptr past MOE_TL_MAX_BLOCKS
  uint64_t t0;
};

__device__ inline uint64_t tl_now() { return __builtin_amdgcn_s_memrealtime(); }

__device__ inline void tl_mark(const TlRow& r, int i) {
  if (r.row && threadIdx.x == 0) r.row[2 + i] = tl_now();
}

// Called by every wave when it finishes (waves of a workgroup need not finish
// together): the first active lane of each wave raises the end word to its
// clock with an atomic maximum, so the row ends with the workgroup's last wave
// (the clock only grows, so an older dispatch's end never wins); thread 0 also
// writes the start and the hardware ids.
__device__ inline void tl_end(const TlRow& r) {
  if (!r.row) return;
  const uint64_t t = tl_now();
  const int lane = threadIdx.x & 63;
  if (lane == (int)__builtin_ctzll(__ballot(1)))
    __hip_atomic_fetch_max(r.row + MOE_TL_WORDS - 1, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (threadIdx.x == 0) {
    uint32_t hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    r.row[0] = ((uint64_t)xcc << 32) | hw;
    r.row[1] = r.t0;
  }
}

#define MOE_TL_UNIT(NAME, FIRST, COUNT)                                                                   \
  static __device__ uint64_t tl_rows_##NAME[(COUNT) * MOE_TL_MAX_BLOCKS * MOE_TL_WORDS];                 \
  static __device__ inline TlRow tl_begin(int kernel) {                                                  \
    TlRow r;                                                                                             \
    r.t0 = tl_now();                                                                                     \
    r.row = blockIdx.x < MOE_TL_MAX_BLOCKS                                                               \
                ? tl_rows_##NAME + ((size_t)(kernel - (FIRST)) * MOE_TL_MAX_BLOCKS + blockIdx.x) * MOE_TL_WORDS \
                : nullptr;                                                                               \
    return r;                                                                                            \
  }                                                                                                      \
  static uint64_t* tl_addr_##NAME() {                                                                    \
    void* p = nullptr;                                                                                   \
    return hipGetSymbolAddress(&p, HIP_SYMBOL(tl_rows_##NAME)) == hipSuccess ? (uint64_t*)p : nullptr;  \
  }                                                                                                      \
  bool tl_owns_##NAME(int kernel) { return kernel >= (FIRST) && kernel < (FIRST) + (COUNT); }           \
  hipError_t tl_read_##NAME(int kernel, uint64_t* host, int blocks) {                                    \
    uint64_t* d = tl_addr_##NAME();                                                                      \
    if (!d) return hipErrorInvalidSymbol;                                                                \
    return hipMemcpy(host, d + (size_t)(kernel - (FIRST)) * MOE_TL_MAX_BLOCKS * MOE_TL_WORDS,            \
                     (size_t)blocks * MOE_TL_WORDS * 8, hipMemcpyDeviceToHost);                          \
  }                                                                                                      \
  hipError_t tl_clear_##NAME() {                                                                         \
    uint64_t* d = tl_addr_##NAME();                                                                      \
    if (!d) return hipErrorInvalidSymbol;                                                                \
    return hipMemset(d, 0, sizeof(tl_rows_##NAME));                                                      \
  }

#else

struct TlRow {};
__device__ inline void tl_mark(const TlRow&, int) {}
__device__ inline void tl_end(const TlRow&) {}
#define MOE_TL_UNIT(NAME, FIRST, COUNT) \
  static __device__ inline TlRow tl_begin(int) { return TlRow{}; }

#endif

}  // namespace moe
