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

// Top-k of one token's E experts by one whole wave (E <= 64 * EPL, K <= 64), in
// the blocked layout: lane l holds experts l * EPL + i, i = 0 .. EPL-1, so a
// lower lane holds only lower ids. The order is the logit (its 32-bit order
// image, sel_image), then the lower id. Each lane sorts its EPL entries (a
// stable odd-even transposition sort: equal images keep id order); each of K
// rounds takes the wave maximum of the lanes' first images, and the lowest lane
// holding it wins, which is the lowest id among equal logits, without a
// tie-break pass. The winner pops its entry; a payload value per entry (a slot,
// or nothing) travels with it.
// Out: lane k < K gets img_out = the image and id_out = the expert of rank k.
// A rank hook is called as hook(k, id, payload) once per rank k = 0 .. K-1 as
// soon as that rank is known (wave-uniform arguments); the default does nothing.
struct NoRankHook {
  __device__ void operator()(int, int32_t, int32_t) const {}
};

// Order image of a logit: larger image = higher logit, -0.0 folded into +0.0.
// Image 0 marks an absent expert; the one logit that would map to it (the NaN
// with every bit set) maps to 1 instead.
__device__ inline uint32_t sel_image(float l) {
  const uint32_t u = __float_as_uint(l + 0.0f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ord > 1u ? ord : 1u;
}
__device__ inline float image_logit(uint32_t ord) {
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

template <int EPL, typename Hook = NoRankHook>
__device__ inline void wave_topk(uint32_t (&img)[EPL], int32_t (&idv)[EPL], int32_t (&pay)[EPL], int K, int lane,
                                 uint32_t& img_out, int32_t& id_out, const Hook& hook = Hook{}) {
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
#pragma unroll
    for (int i = (r & 1); i + 1 < EPL; i += 2) {
      const bool sw = img[i + 1] > img[i];
      const uint32_t a = img[i], b = img[i + 1];
      const int32_t ia = idv[i], ib = idv[i + 1], pa = pay[i], pb = pay[i + 1];
      img[i] = sw ? b : a;
      img[i + 1] = sw ? a : b;
      idv[i] = sw ? ib : ia;
      idv[i + 1] = sw ? ia : ib;
      pay[i] = sw ? pb : pa;
      pay[i + 1] = sw ? pa : pb;
    }
  }
  img_out = 0u;
  id_out = 0;
  for (int k = 0; k < K; ++k) {
    const uint32_t m = wave_max_u32(img[0]);
    const int src = (int)__builtin_ctzll(__ballot(img[0] == m));
    const int32_t idk = __builtin_amdgcn_readlane(idv[0], src);
    const int32_t pk = __builtin_amdgcn_readlane(pay[0], src);
    if (lane == src) {
#pragma unroll
      for (int i = 0; i + 1 < EPL; ++i) {
        img[i] = img[i + 1];
        idv[i] = idv[i + 1];
        pay[i] = pay[i + 1];
      }
      img[EPL - 1] = 0u;
    }
    if (lane == k) {
      img_out = m;
      id_out = idk;
    }
    hook(k, idk, pk);
  }
}

// The same selection as wave_topk by a wave-wide bitonic sort of all 64 * EPL
// full keys (route_key: logit image, then the lower id; EPL a power of two),
// descending: element i is key[i / 64] of lane i % 64 (the order the keys come in
// does not matter, they carry their ids), so rank k ends in key[0] of lane k. A
// compare-exchange at distance j < 64 pairs lanes (shuffle), at j >= 64
// registers of one lane. The keys are distinct, so the K selected and their
// order equal wave_topk's. The rank hook gets payload 0.
__device__ inline uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
template <int EPL, typename Hook = NoRankHook>
__device__ inline uint64_t wave_topk_bitonic(uint64_t (&key)[EPL], int K, int lane, const Hook& hook = Hook{}) {
  constexpr int N = 64 * EPL;
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int j = size >> 1; j > 0; j >>= 1) {
      if (j < 64) {
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
          const bool desc = ((r * 64 + lane) & size) == 0;  // block sorted descending
          const uint64_t a = key[r], b = shfl_xor_u64(a, j);
          const bool take_max = ((lane & j) == 0) == desc;
          key[r] = take_max ? (a > b ? a : b) : (a > b ? b : a);
        }
      } else {
        const int jr = j / 64;
#pragma unroll
        for (int r = 0; r < EPL; ++r) {
          if ((r & jr) == 0) {
            const bool desc = ((r * 64) & size) == 0;
            const uint64_t a = key[r], b = key[r | jr];
            const uint64_t hi = a > b ? a : b, lo = a > b ? b : a;
            key[r] = desc ? hi : lo;
            key[r | jr] = desc ? lo : hi;
          }
        }
      }
    }
  }
  for (int k = 0; k < K; ++k) hook(k, key_id(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((uint32_t)(key[0] >> 32), k) << 32) |
                                        (uint32_t)__builtin_amdgcn_readlane((uint32_t)key[0], k)), 0);
  return lane < K ? key[0] : 0ull;
}

// Softmax + top-k of one token's logits held in registers in the blocked layout
// (lane l holds lg[i] = logit of expert l * EPL + i; entries past E ignored):
// lane k < K gets the expert of rank k and its weight (the softmax probability
// over all E, with MOE_ROUTE_RENORM divided by the sum over the K selected).
// pay[i] is a payload per expert (e.g. its slot) handed to the rank hook.
template <int EPL, bool BITONIC = false, typename Hook = NoRankHook>
__device__ inline void wave_select_values(float (&lg)[EPL], int32_t (&pay)[EPL], int E, int K, unsigned flags,
                                          int lane, int32_t& id, float& wt, const Hook& hook = Hook{}) {
  float top;  // this lane's rank's logit (lanes < K)
  if constexpr (BITONIC) {
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      if (e >= E) lg[i] = 0.0f;
      key[i] = e < E ? route_key(lg[i], e) : 0ull;  // real keys are > 0
    }
    const uint64_t mine = wave_topk_bitonic<EPL>(key, K, lane, hook);
    top = key_logit(mine);
    id = key_id(mine);
  } else {
    uint32_t img[EPL];
    int32_t idv[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      if (e >= E) lg[i] = 0.0f;
      img[i] = e < E ? sel_image(lg[i]) : 0u;
      idv[i] = e;
    }
    uint32_t mine;
    wave_topk<EPL>(img, idv, pay, K, lane, mine, id, hook);
    top = image_logit(mine);
  }
  const float m = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane(__float_as_uint(top)));  // rank 0's
  float part = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane * EPL + i < E) part += expf(lg[i] - m);
  part = wave_sum_f32(part);
  float w = 0.0f;
  if (lane < K) w = expf(top - m) / part;
  if (flags & MOE_ROUTE_RENORM) w = w / wave_sum_f32(lane < K ? w : 0.0f);
  wt = w;
}
template <int EPL, bool BITONIC = false>
__device__ inline void wave_select_values(float (&lg)[EPL], int E, int K, unsigned flags, int lane, int32_t& id,
                                          float& wt) {
  int32_t pay[EPL] = {};
  wave_select_values<EPL, BITONIC>(lg, pay, E, K, flags, lane, id, wt);
}

template <int EPL, bool BITONIC = false>
__device__ inline void wave_select(const float* __restrict__ l, int E, int K, unsigned flags, int lane, int32_t& id,
                                   float& wt) {
  float lg[EPL];
  // every load unconditional (a clamped index past E), so that all of them are in
  // flight at once: a load under a branch is waited for before the branch joins
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    lg[i] = l[e < E ? e : E - 1];
  }
  wave_select_values<EPL, BITONIC>(lg, E, K, flags, lane, id, wt);
}

// ------------------------------------------------------------------ router GEMV of one token
// l = sum_h x[h] * w[h] over one router row, by a workgroup of 256 threads (4
// waves): thread t covers the 16 columns 16 (t + 256 j) for j = 0, 1 (H <= 8192)
// with four independent fp64 accumulators (one per float4 of the row; bf16 x
// fp32 products are exact in fp64), added in a fixed order, then the lanes
// (wave_sum_f64) and the four waves in order. Every workgroup-wide path through
// here gives the same bits. part: 4 doubles of LDS. Thread 0 returns the sum.
__device__ inline double router_row_sum(const uint16_t* __restrict__ x, const float* __restrict__ w, int H,
                                        double* part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float4 wv[2][4];
  uint4 xv[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = 16 * (tid + 256 * j);
    const bool ok = c < H;
    const int cc = ok ? c : 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) wv[j][q] = reinterpret_cast<const float4*>(w + cc)[q];
#pragma unroll
    for (int q = 0; q < 2; ++q) xv[j][q] = reinterpret_cast<const uint4*>(x + cc)[q];
    if (!ok) {
#pragma unroll
      for (int q = 0; q < 2; ++q) xv[j][q] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t x01 = q & 1 ? (q & 2 ? xv[j][1].z : xv[j][0].z) : (q & 2 ? xv[j][1].x : xv[j][0].x);
      const uint32_t x23 = q & 1 ? (q & 2 ? xv[j][1].w : xv[j][0].w) : (q & 2 ? xv[j][1].y : xv[j][0].y);
      acc[q] = fma((double)__uint_as_float(x01 << 16), (double)wv[j][q].x, acc[q]);
      acc[q] = fma((double)__uint_as_float(x01 & 0xFFFF0000u), (double)wv[j][q].y, acc[q]);
      acc[q] = fma((double)__uint_as_float(x23 << 16), (double)wv[j][q].z, acc[q]);
      acc[q] = fma((double)__uint_as_float(x23 & 0xFFFF0000u), (double)wv[j][q].w, acc[q]);
    }
  }
  double a = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  a = wave_sum_f64(a);
  if (lane == 0) part[wave] = a;
  __syncthreads();
  return ((part[0] + part[1]) + part[2]) + part[3];
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
