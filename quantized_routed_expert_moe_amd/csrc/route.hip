// Routing kernels: router GEMV (fp64 accumulation) and per-token softmax + top-k.
//
// "Strata on a Mac", Switches: the router is a GEMV giving one logit per
// expert, and a separate routing dispatch (moe_route) picks the top experts.
// Softmax and the tie rule (equal logits -> lower id) follow the plain reading
// of a softmax top-k router.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterTok = 4;  // tokens per router wave (one router row is read once for them)

__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// One wave per (expert, block of kRouterTok tokens). Each lane accumulates its
// columns h = 4*lane + 256*i in order in fp64 (the bf16 x fp32 products are
// exact in fp64), then a fixed butterfly sums the 64 lanes; one rounding to
// fp32 at the end. The reduction order is fixed, so the bits are reproducible.
__global__ void __launch_bounds__(64) router_gemv_kernel(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                         float* __restrict__ logits, int T, int H, int E) {
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kRouterTok;
  const int lane = threadIdx.x;
  const float* w = wr + (size_t)e * H;
  double acc[kRouterTok];
#pragma unroll
  for (int i = 0; i < kRouterTok; ++i) acc[i] = 0.0;
  for (int h = 4 * lane; h < H; h += 256) {
    const float4 wv = *reinterpret_cast<const float4*>(w + h);
#pragma unroll
    for (int i = 0; i < kRouterTok; ++i) {
      if (t0 + i < T) {
        const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)(t0 + i) * H + h);
        double a = acc[i];
        a = fma((double)bf16_lo(xv.x), (double)wv.x, a);
        a = fma((double)bf16_hi(xv.x), (double)wv.y, a);
        a = fma((double)bf16_lo(xv.y), (double)wv.z, a);
        a = fma((double)bf16_hi(xv.y), (double)wv.w, a);
        acc[i] = a;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRouterTok; ++i) {
    double a = acc[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) a += __shfl_xor(a, off, 64);
    if (lane == 0 && t0 + i < T) logits[(size_t)(t0 + i) * E + e] = (float)a;
  }
}

// Total order key: larger key = higher logit, then lower id. -0.0 is folded into +0.0.
__device__ inline uint64_t route_key(float l, int e) {
  const uint32_t u = __float_as_uint(l + 0.0f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ inline float key_logit(uint64_t k) {
  const uint32_t ord = (uint32_t)(k >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

__device__ inline uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

// One wave per token. Lane l holds the keys of experts l, l+64, ... sorted
// descending in registers; K rounds of a butterfly max across the wave each
// pick the next expert in rank order and pop it from its owner lane.
template <int EPL>
__global__ void __launch_bounds__(64) route_select_kernel(const float* __restrict__ logits, int T, int E, int K,
                                                          unsigned flags, int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* l = logits + (size_t)t * E;
  uint64_t key[EPL];
  float lg[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane + 64 * i;
    lg[i] = e < E ? l[e] : 0.0f;
    key[i] = e < E ? route_key(lg[i], e) : 0ull;  // real keys are > 0
  }
  // local descending sort (odd-even transposition, EPL <= 16)
#pragma unroll
  for (int r = 0; r < EPL; ++r) {
#pragma unroll
    for (int i = (r & 1); i + 1 < EPL; i += 2) {
      const uint64_t a = key[i], b = key[i + 1];
      key[i] = a > b ? a : b;
      key[i + 1] = a > b ? b : a;
    }
  }
  uint64_t mine_best = 0;  // lane k keeps the winner of rank k
  for (int k = 0; k < K; ++k) {
    const uint64_t best = wave_max_u64(key[0]);
    if (key[0] == best) {
#pragma unroll
      for (int i = 0; i + 1 < EPL; ++i) key[i] = key[i + 1];
      key[EPL - 1] = 0;
    }
    if (lane == k) mine_best = best;
  }
  const float m = key_logit(__shfl(mine_best, 0, 64));
  float part = 0.0f;
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    if (lane + 64 * i < E) part += expf(lg[i] - m);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
  float wk = 0.0f;
  if (lane < K) wk = expf(key_logit(mine_best) - m) / part;
  if (flags & MOE_ROUTE_RENORM) {
    float s = lane < K ? wk : 0.0f;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    wk = wk / s;
  }
  if (lane < K) {
    ids[(size_t)t * K + lane] = (int32_t)(0xFFFFFFFFu - (uint32_t)(mine_best & 0xFFFFFFFFu));
    w[(size_t)t * K + lane] = wk;
  }
}

constexpr int kMaxTableUpdates = 64;
struct TableUpdates {
  int32_t idx[kMaxTableUpdates];
  int32_t val[kMaxTableUpdates];
  int n;
};

__global__ void __launch_bounds__(64) table_update_kernel(int32_t* table, TableUpdates u) {
  const int i = threadIdx.x;
  if (i < u.n) table[u.idx[i]] = u.val[i];
}

}  // namespace

hipError_t launch_router_gemv(const uint16_t* x, const float* wr, float* logits, int T, int H, int E,
                              hipStream_t s) {
  dim3 grid(E, (T + kRouterTok - 1) / kRouterTok);
  hipLaunchKernelGGL(router_gemv_kernel, grid, dim3(64), 0, s, x, wr, logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_route_select(const float* logits, int T, int E, int K, unsigned flags, int32_t* ids, float* w,
                               hipStream_t s) {
  const int epl = (E + 63) / 64;
  dim3 grid(T);
  if (epl <= 1)
    hipLaunchKernelGGL(route_select_kernel<1>, grid, dim3(64), 0, s, logits, T, E, K, flags, ids, w);
  else if (epl <= 2)
    hipLaunchKernelGGL(route_select_kernel<2>, grid, dim3(64), 0, s, logits, T, E, K, flags, ids, w);
  else if (epl <= 4)
    hipLaunchKernelGGL(route_select_kernel<4>, grid, dim3(64), 0, s, logits, T, E, K, flags, ids, w);
  else if (epl <= 8)
    hipLaunchKernelGGL(route_select_kernel<8>, grid, dim3(64), 0, s, logits, T, E, K, flags, ids, w);
  else
    hipLaunchKernelGGL(route_select_kernel<16>, grid, dim3(64), 0, s, logits, T, E, K, flags, ids, w);
  return hipGetLastError();
}

hipError_t launch_table_update(int32_t* table, const int32_t* idx, const int32_t* val, int n, hipStream_t s) {
  for (int base = 0; base < n; base += kMaxTableUpdates) {
    TableUpdates u;
    u.n = n - base < kMaxTableUpdates ? n - base : kMaxTableUpdates;
    for (int i = 0; i < u.n; ++i) {
      u.idx[i] = idx[base + i];
      u.val[i] = val[base + i];
    }
    // one thread per entry; entries within a launch touch distinct experts
    hipLaunchKernelGGL(table_update_kernel, dim3(1), dim3(64), 0, s, table, u);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
