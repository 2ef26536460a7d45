// Wave-level helpers shared by the routing and FFN kernels: cross-lane sums
// and maxima, and the top-k selection of one token.
//
// Cross-lane moves avoid the LDS crossbar: DPP rotations inside a row of 16
// lanes and the gfx950 permlane swaps between rows. Every helper is a fixed
// instruction sequence, so its result depends only on the data.
#pragma once

#include "moe_internal.h"

namespace moe {

template <int ROR>  // the value of the lane ROR places over in this lane's row of 16
__device__ inline uint32_t ror_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + ROR, 0xF, 0xF, false);
}
template <int ROR>
__device__ inline uint64_t ror_u64(uint64_t v) {
  return ((uint64_t)ror_u32<ROR>((uint32_t)(v >> 32)) << 32) | ror_u32<ROR>((uint32_t)v);
}
// (this lane's v, v of lane ^ 16) and (v, v of lane ^ 32), in some order per lane
__device__ inline void swap16_u64(uint64_t v, uint64_t& a, uint64_t& b) {
  const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
  a = ((uint64_t)hi[0] << 32) | lo[0];
  b = ((uint64_t)hi[1] << 32) | lo[1];
}
__device__ inline void swap32_u64(uint64_t v, uint64_t& a, uint64_t& b) {
  const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(v >> 32), (uint32_t)(v >> 32), false, false);
  a = ((uint64_t)hi[0] << 32) | lo[0];
  b = ((uint64_t)hi[1] << 32) | lo[1];
}
__device__ inline double as_f64(uint64_t v) { return __builtin_bit_cast(double, v); }
__device__ inline uint64_t as_u64(double v) { return __builtin_bit_cast(uint64_t, v); }

// Sum over the 64 lanes in a fixed sequence of additions; lane 0's result is the one to use.
__device__ inline double wave_sum_f64(double a) {
  a += as_f64(ror_u64<1>(as_u64(a)));
  a += as_f64(ror_u64<2>(as_u64(a)));
  a += as_f64(ror_u64<4>(as_u64(a)));
  a += as_f64(ror_u64<8>(as_u64(a)));
  uint64_t x, y;
  swap16_u64(as_u64(a), x, y);
  a = as_f64(x) + as_f64(y);
  swap32_u64(as_u64(a), x, y);
  return as_f64(x) + as_f64(y);
}

// Sum over the 64 lanes in a fixed sequence of additions, lane 0's bits on every lane.
__device__ inline float wave_sum_f32(float a) {
  a += __uint_as_float(ror_u32<1>(__float_as_uint(a)));
  a += __uint_as_float(ror_u32<2>(__float_as_uint(a)));
  a += __uint_as_float(ror_u32<4>(__float_as_uint(a)));
  a += __uint_as_float(ror_u32<8>(__float_as_uint(a)));
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  a = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  a = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
  return __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane(__float_as_uint(a)));
}

// The maximum over the 64 lanes, on every lane.
__device__ inline uint64_t wave_max_u64(uint64_t v) {
  uint64_t o = ror_u64<1>(v);
  v = o > v ? o : v;
  o = ror_u64<2>(v);
  v = o > v ? o : v;
  o = ror_u64<4>(v);
  v = o > v ? o : v;
  o = ror_u64<8>(v);
  v = o > v ? o : v;
  uint64_t x, y;
  swap16_u64(v, x, y);
  v = x > y ? x : y;
  swap32_u64(v, x, y);
  return x > y ? x : y;
}

// t + t of the lane ROR places over in its row of 16 (lanes may differ in association order)
template <int ROR>
__device__ inline float dpp_add(float t) {
  return t + __uint_as_float(ror_u32<ROR>(__float_as_uint(t)));
}
// t + t of lane ^ X (X = 1 or 2): the same bits on both lanes
template <int X>
__device__ inline float quad_xor_add(float t) {
  constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
  return t + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(t), ctrl, 0xF, 0xF, false));
}
// t summed over lanes l, l ^ 16, l ^ 32, l ^ 48: the same bits on all four
__device__ inline float sum_rows(float t) {
  const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  t = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
}

// Total order key of (logit, expert): larger key = higher logit, then lower id.
// -0.0 is folded into +0.0. Every real key is > 0.
__device__ inline uint64_t route_key(float l, int e) {
  const uint32_t u = __float_as_uint(l + 0.0f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ inline float key_logit(uint64_t k) {
  const uint32_t ord = (uint32_t)(k >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}
__device__ inline int32_t key_id(uint64_t k) { return (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu)); }

// The maximum over the 64 lanes, on every lane.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  v = max(v, ror_u32<1>(v));
  v = max(v, ror_u32<2>(v));
  v = max(v, ror_u32<4>(v));
  v = max(v, ror_u32<8>(v));
  const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)s16[0], (uint32_t)s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)s32[0], (uint32_t)s32[1]);
}

// Softmax top-k of one token's E logits l[0..E) by one whole wave (E <= 64 * EPL,
// K <= 64). Lane k < K gets rank k: its expert id and its weight
// softmax(l)[id] (divided by the sum of the K weights with MOE_ROUTE_RENORM).
// Lane l holds the keys of experts l, l+64, ... sorted descending in
// registers; each of K rounds takes the wave-wide maximum of the lanes' first
// keys (on the 32-bit logit image; among equal images the full key, i.e. the
// lowest id, decides) and pops it from its owner lane.
// The K largest keys of the wave (lane l holds the keys of experts l, l + 64, ...;
// 0 marks an absent expert): lane k < K returns the key of rank k, the others 0.
template <int EPL>
__device__ inline uint64_t wave_topk(uint64_t (&key)[EPL], int K, int lane) {
  // local descending sort (odd-even transposition)
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
#pragma unroll
    for (int i = (r & 1); i + 1 < EPL; i += 2) {
      const uint64_t a = key[i], b = key[i + 1];
      key[i] = a > b ? a : b;
      key[i + 1] = a > b ? b : a;
    }
  }
  uint64_t mine = 0;  // lane k keeps the winner of rank k
  for (int k = 0; k < K; ++k) {
    const uint32_t hi = (uint32_t)(key[0] >> 32);
    const uint32_t m = wave_max_u32(hi);
    uint64_t owners = __ballot(hi == m);
    if (__builtin_popcountll(owners) > 1) {  // equal values: the highest full key (lowest id) wins
      const uint64_t best = wave_max_u64(hi == m ? key[0] : 0ull);
      owners = __ballot(key[0] == best);
    }
    const int src = (int)__builtin_ctzll(owners);
    const uint64_t best = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)(key[0] >> 32), src) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((uint32_t)key[0], src);
    if (lane == src) {
#pragma unroll
      for (int i = 0; i + 1 < EPL; ++i) key[i] = key[i + 1];
      key[EPL - 1] = 0;
    }
    if (lane == k) mine = best;
  }
  return mine;
}

// Softmax + top-k of one token's logits l[0..E): lane k < K gets the expert of
// rank k and its weight (the softmax probability over all E, with
// MOE_ROUTE_RENORM divided by the sum over the K selected).
template <int EPL>
__device__ inline void wave_select(const float* __restrict__ l, int E, int K, unsigned flags, int lane, int32_t& id,
                                   float& wt) {
  uint64_t key[EPL];
  float lg[EPL];
  // every load unconditional (a clamped index past E), so that all of them are in
  // flight at once: a load under a branch is waited for before the branch joins
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    lg[i] = l[e < E ? e : E - 1];
  }
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    if (e >= E) lg[i] = 0.0f;
    key[i] = e < E ? route_key(lg[i], e) : 0ull;  // real keys are > 0
  }
  const uint64_t mine = wave_topk<EPL>(key, K, lane);
  const uint32_t top_hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(mine >> 32));
  const uint32_t top_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)mine);
  const float m = key_logit(((uint64_t)top_hi << 32) | top_lo);  // the largest logit (rank 0, lane 0)
  float part = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + 64 * i < E) part += expf(lg[i] - m);
  part = wave_sum_f32(part);
  float w = 0.0f;
  if (lane < K) w = expf(key_logit(mine) - m) / part;
  if (flags & MOE_ROUTE_RENORM) w = w / wave_sum_f32(lane < K ? w : 0.0f);
  id = key_id(mine);
  wt = w;
}

// ------------------------------------------------------------------ int4 codes x fp16 activations
// A code dword w holds 8 offset-binary nibbles u = q + 8 (see the blob layout);
// its four fp16 pairs, one AND-OR each (two also need w >> 8), are exact:
//   A pairs (nibbles at bits 0..3 / 16..19 of w or w >> 8): 0x6400 | u  = 1024 + u = q + 1032
//   B pairs (nibbles at bits 4..7 / 20..23):                 0x5400 | 16u = 64 + u  = q + 72
// Pair k of dword d covers columns 8d + 2k and 8d + 2k + 1 (A: k = 0, 2; B: k = 1, 3).
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ inline float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// d + the 8 codes of w times the activation pairs x0..x3 of the same columns.
__device__ inline float code_dot(uint32_t w, uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, float d) {
  const uint32_t w8 = w >> 8;
  d = dot2h((w & 0x000F000Fu) | 0x64006400u, x0, d);   // columns +0, +1
  d = dot2h((w & 0x00F000F0u) | 0x54005400u, x1, d);   // +2, +3
  d = dot2h((w8 & 0x000F000Fu) | 0x64006400u, x2, d);  // +4, +5
  d = dot2h((w8 & 0x00F000F0u) | 0x54005400u, x3, d);  // +6, +7
  return d;
}

// The 16 pairs of a 16-byte code chunk (32 columns), pair k for activation dword k.
__device__ inline void code_pairs(const uint4& c, uint32_t (&out)[16]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t w8 = w[d] >> 8;
    out[4 * d + 0] = (w[d] & 0x000F000Fu) | 0x64006400u;
    out[4 * d + 1] = (w[d] & 0x00F000F0u) | 0x54005400u;
    out[4 * d + 2] = (w8 & 0x000F000Fu) | 0x64006400u;
    out[4 * d + 3] = (w8 & 0x00F000F0u) | 0x54005400u;
  }
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// fp16 bits of the fp32 value v (round to nearest even); *bad set when it overflows.
__device__ inline uint32_t to_f16_bits(float v, bool* bad) {
  const _Float16 h = (_Float16)v;
  const uint32_t b = __builtin_bit_cast(uint16_t, h);
  if ((b & 0x7FFFu) == 0x7C00u) *bad = true;
  return b;
}

__device__ inline float f16_lo(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu)); }
__device__ inline float f16_hi(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

}  // namespace moe
