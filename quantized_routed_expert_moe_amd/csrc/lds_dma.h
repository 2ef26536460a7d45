// Loads from global memory straight into LDS, for kernels that stage operands
// without holding them in registers.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// Loads straight into LDS (gfx950 buffer_load ... lds): lane l's n bytes (n = 4
// or 16) from base + voffset + soffset land at lds + n l; lds must be the same on
// every lane of the wave (an instruction offset would move the LDS address too,
// so none is used). The buffer form rather than the global one: the
// compiler treats a pending global (FLAT) load into LDS as an out-of-order LDS
// access and then waits for every LDS read at once, instead of only for the one
// an MFMA needs. A read past the descriptor's byte range returns zeros.
__device__ inline __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ inline void ld16_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}
__device__ inline void ld4_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
}

// Copy n16 16-byte chunks from offset off of buffer r to LDS at dst, one wave
// instruction (64 chunks, 1 KB) at a time; instruction k is issued by wave
// k % nw, so each wave's share is a fixed set of instructions.
__device__ inline void stage_lds(__amdgpu_buffer_rsrc_t r, uint32_t off, int n16, unsigned char* dst, int wave,
                                 int lane, int nw) {
  for (int k = wave; k * 64 < n16; k += nw) {
    const int c = k * 64 + lane;
    if (c < n16) ld16_lds(r, off + (uint32_t)c * 16, 0, dst + (size_t)k * 1024);
  }
}

// s_waitcnt immediate (gfx9 encoding) that waits until at most vm vector-memory
// operations of this wave are outstanding; LDS and export counters are not waited for.
__host__ __device__ constexpr int vmcnt_imm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8); }

}  // namespace moe
