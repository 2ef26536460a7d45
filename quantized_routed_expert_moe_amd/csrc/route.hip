// Routing kernels: router GEMV (fp64 accumulation) and per-token softmax + top-k.
//
// "Strata on a Mac", Switches: the router is a GEMV giving one logit per
// expert, and a separate routing dispatch (moe_route) picks the top experts.
// Softmax and the tie rule (equal logits -> lower id) follow the plain reading
// of a softmax top-k router.
#include "moe_internal.h"
#include "onepass.h"
#include "timeline.h"
#include "wave_ops.h"

namespace moe {
MOE_TL_UNIT(route, MOE_TL_ROUTER_GEMV, 2)
namespace {

constexpr int kRouterTok = 4;  // tokens per router wave (one router row is read once for them)

__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// One workgroup (4 waves) per (expert, block of kRouterTok tokens). Wave w
// covers the contiguous quarter [w*H/4, (w+1)*H/4) of the row; lane l takes
// columns 4l + 256i of it, all loads issued before any arithmetic. Each lane
// accumulates its columns in order in fp64 (bf16 x fp32 products are exact in
// fp64), a fixed sequence of DPP and permlane additions sums the lanes, and the
// four wave sums are added in wave order; one rounding to fp32 at the end. The order is fixed, so the bits
// are reproducible.
constexpr int kRouterMaxIt = 8;  // columns per lane = 4 * kRouterMaxIt -> H <= 8192

__global__ void __launch_bounds__(256) router_gemv_kernel(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                          float* __restrict__ logits, int T, int H, int E) {
  __shared__ double part[4][kRouterTok];
  const int e = blockIdx.x;
  const int t0 = blockIdx.y * kRouterTok;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = H / 4;
  const int h0 = wave * q;
  const float* w = wr + (size_t)e * H;
  float4 wv[kRouterMaxIt];
  uint2 xv[kRouterTok][kRouterMaxIt];
#pragma unroll
  for (int i = 0; i < kRouterMaxIt; ++i) {
    const int h = 4 * lane + 256 * i;
    if (h < q) {
      wv[i] = *reinterpret_cast<const float4*>(w + h0 + h);
#pragma unroll
      for (int tt = 0; tt < kRouterTok; ++tt)
        if (t0 + tt < T) xv[tt][i] = *reinterpret_cast<const uint2*>(x + (size_t)(t0 + tt) * H + h0 + h);
    }
  }
#pragma unroll
  for (int tt = 0; tt < kRouterTok; ++tt) {
    double a = 0.0;
#pragma unroll
    for (int i = 0; i < kRouterMaxIt; ++i) {
      if (4 * lane + 256 * i < q && t0 + tt < T) {
        a = fma((double)bf16_lo(xv[tt][i].x), (double)wv[i].x, a);
        a = fma((double)bf16_hi(xv[tt][i].x), (double)wv[i].y, a);
        a = fma((double)bf16_lo(xv[tt][i].y), (double)wv[i].z, a);
        a = fma((double)bf16_hi(xv[tt][i].y), (double)wv[i].w, a);
      }
    }
    a = wave_sum_f64(a);
    if (lane == 0) part[wave][tt] = a;
  }
  __syncthreads();
  if (threadIdx.x < kRouterTok && t0 + (int)threadIdx.x < T) {
    const int tt = threadIdx.x;
    const double s = ((part[0][tt] + part[1][tt]) + part[2][tt]) + part[3][tt];
    logits[(size_t)(t0 + tt) * E + e] = (float)s;
  }
}

// Single token: one workgroup per expert (router_row_sum), one rounding to fp32.
__global__ void __launch_bounds__(256) router_gemv1_kernel(const uint16_t* __restrict__ x,
                                                           const float* __restrict__ wr, float* __restrict__ logits,
                                                           int H, int E) {
  const TlRow tl = tl_begin(MOE_TL_ROUTER_GEMV);
  __shared__ double part[4];
  const int e = blockIdx.x;
  const double s = router_row_sum(x, wr + (size_t)e * H, H, part);
  if (threadIdx.x == 0) logits[e] = (float)s;
  tl_end(tl);
}

// One-pass routing of one token (moe_route_onepass): workgroup e computes
// logit e (router_row_sum, the bits of router_gemv1_kernel) and publishes it;
// the last workgroup's first wave waits for all E words of this call, writes
// the logits, selects (the bits of route_select_kernel) and advances the
// region's call number (every workgroup has read it by then: each published a
// word of this epoch).
template <int EPL>
__global__ void __launch_bounds__(256) route_onepass_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr, float* __restrict__ logits,
                                                            int H, int E, int K, unsigned flags, int32_t* ids, float* w,
                                                            uint64_t* words, int32_t* status) {
  __shared__ double part[4];
  const uint32_t ep = onepass_epoch(words);
  onepass_publish_logit(x, wr, H, blockIdx.x, words, ep, part);
  if ((int)blockIdx.x != E - 1 || threadIdx.x >= 64) return;
  float lg[EPL];
  if (!onepass_wait_logits<EPL>(words, E, ep, status, lg)) return;
  float sel[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) sel[i] = lg[i];
  int32_t id;
  float wt;
  wave_select_values<EPL>(sel, E, K, flags, threadIdx.x, id, wt);
  const int lane = threadIdx.x;
  if (lane < K) {
    ids[lane] = id;
    w[lane] = wt;
  }
  onepass_store_logits<EPL>(lg, E, logits);
  if (lane == 0) __hip_atomic_store(words, (uint64_t)ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One wave per token. The weights are multiplied by scale (1 for moe_route,
// where the product is exact). With slot_table (one token): the table is staged
// in LDS while the logits load, and lane k also writes slots_out[k] =
// slot_table[ids[k]], so the single-token FFN kernels find their blobs with one
// load instead of two.
template <int EPL, bool BITONIC>
__global__ void __launch_bounds__(64) route_select_kernel(const float* __restrict__ logits, int T, int E, int K,
                                                          unsigned flags, float scale, int32_t* __restrict__ ids,
                                                          float* __restrict__ w,
                                                          const int32_t* __restrict__ slot_table,
                                                          int32_t* __restrict__ slots_out) {
  const TlRow tl = tl_begin(MOE_TL_ROUTE_SELECT);
  __shared__ int32_t tbl[64 * EPL];
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  // the table loads go out with the logits loads (clamped index past E); the
  // values reach LDS only after the selection, so no wait comes between the two
  int32_t tv[EPL];
  if (slot_table) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      tv[i] = slot_table[e < E ? e : E - 1];
    }
  }
  int32_t id;
  float wt;
  wave_select<EPL, BITONIC>(logits + (size_t)t * E, E, K, flags, lane, id, wt);
  if (lane < K) {
    ids[(size_t)t * K + lane] = id;
    w[(size_t)t * K + lane] = wt * scale;
  }
  if (slot_table) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) tbl[lane * EPL + i] = tv[i];  // entries past E are never read
    __builtin_amdgcn_wave_barrier();  // one wave: its LDS stores precede its loads
    if (lane < K) slots_out[lane] = tbl[id];
  }
  tl_end(tl);
}

// Score of one logit for the scored router variants ("Strata" README, Models:
// sigmoid and sqrtsoftplus routing): evaluated in fp64 and rounded once to
// fp32, the precision of the selection key. softplus(l) = l + ln(1 + e^-l)
// for l > 0 and ln(1 + e^l) otherwise, so e^l never overflows.
__device__ inline float expert_score(float l, int score) {
  const double x = (double)l;
  if (score == MOE_SCORE_SIGMOID) return (float)(1.0 / (1.0 + exp(-x)));
  const double sp = x > 0.0 ? x + log1p(exp(-x)) : log1p(exp(x));
  return (float)sqrt(sp);
}

// One wave per token: selection on c = fp32(score + bias) with the total order
// of wave_select (c descending, equal values to the lower id); the weight of
// a selected expert is its score (the bias steers selection only), divided by
// the sum over the K selected with MOE_ROUTE_RENORM, then times scale.
template <int EPL>
__global__ void __launch_bounds__(64) route_scored_kernel(const float* __restrict__ logits, int T, int E, int K,
                                                          unsigned flags, int score, const float* __restrict__ bias,
                                                          float scale, int32_t* __restrict__ ids,
                                                          float* __restrict__ w) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const float* l = logits + (size_t)t * E;
  float lv[EPL], bv[EPL];  // loads first, all in flight together (clamped index past E)
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    const int ec = e < E ? e : E - 1;
    lv[i] = l[ec];
    bv[i] = bias ? bias[ec] : 0.0f;
  }
  uint32_t img[EPL];
  int32_t idv[EPL], pay[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    const int e = lane * EPL + i;
    idv[i] = e;
    pay[i] = 0;
    if (e < E) {
      const float s = expert_score(lv[i], score);
      const float c = bias ? s + bv[i] : s;
      img[i] = sel_image(c);
    } else {
      img[i] = 0u;  // absent
    }
  }
  uint32_t mine;
  int32_t id;
  wave_topk<EPL>(img, idv, pay, K, lane, mine, id);
  float wt = 0.0f;
  if (lane < K) wt = expert_score(l[id], score);
  if (flags & MOE_ROUTE_RENORM) wt = wt / wave_sum_f32(lane < K ? wt : 0.0f);
  if (lane < K) {
    ids[(size_t)t * K + lane] = id;
    w[(size_t)t * K + lane] = wt * scale;
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

// The n ids to pinned host memory, then host[n] = seq: one lane stores every id
// at system scope and then the sequence word with a system-scope release, so a
// host that reads seq in host[n] (acquire) also reads the ids of this call.
__global__ void __launch_bounds__(64) publish_ids_kernel(const int32_t* ids, int n, int32_t* host, int32_t seq) {
  if (threadIdx.x != 0) return;
  for (int i = 0; i < n; ++i) __hip_atomic_store(host + i, ids[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __hip_atomic_store(host + n, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// src == nullptr: *dst = 0. Else the first error wins: a non-zero *src is copied
// into *dst when *dst is still 0.
__global__ void __launch_bounds__(64) status_kernel(int32_t* dst, const int32_t* src) {
  if (threadIdx.x != 0) return;
  if (!src) {
    *dst = 0;
    return;
  }
  const int32_t v = *src;
  if (v != 0 && *dst == 0) *dst = v;
}

}  // namespace

hipError_t launch_router_gemv(const uint16_t* x, const float* wr, float* logits, int T, int H, int E,
                              hipStream_t s) {
  if (T == 1) {
    hipLaunchKernelGGL(router_gemv1_kernel, dim3(E), dim3(256), 0, s, x, wr, logits, H, E);
    return hipGetLastError();
  }
  dim3 grid(E, (T + kRouterTok - 1) / kRouterTok);
  hipLaunchKernelGGL(router_gemv_kernel, grid, dim3(256), 0, s, x, wr, logits, T, H, E);
  return hipGetLastError();
}

hipError_t launch_route_select(const float* logits, int T, int E, int K, unsigned flags, int32_t* ids, float* w,
                               hipStream_t s, int score, const float* bias, float scale, const int32_t* slot_table,
                               int32_t* slots_out) {
  if (slot_table && (T != 1 || score != MOE_SCORE_SOFTMAX || !slots_out)) return hipErrorInvalidValue;
  const int epl = (E + 63) / 64;
  dim3 grid(T);
#define SEL(N)                                                                                                    \
  do {                                                                                                            \
    if (score == MOE_SCORE_SOFTMAX && (flags & MOE_ROUTE_BITONIC))                                                \
      hipLaunchKernelGGL((route_select_kernel<N, true>), grid, dim3(64), 0, s, logits, T, E, K, flags, scale, ids, \
                         w, slot_table, slots_out);                                                               \
    else if (score == MOE_SCORE_SOFTMAX)                                                                          \
      hipLaunchKernelGGL((route_select_kernel<N, false>), grid, dim3(64), 0, s, logits, T, E, K, flags, scale, ids, \
                         w, slot_table, slots_out);                                                               \
    else                                                                                                          \
      hipLaunchKernelGGL(route_scored_kernel<N>, grid, dim3(64), 0, s, logits, T, E, K, flags, score, bias, scale, \
                         ids, w);                                                                                 \
  } while (0)
  if (epl <= 1) SEL(1);
  else if (epl <= 2) SEL(2);
  else if (epl <= 4) SEL(4);
  else if (epl <= 8) SEL(8);
  else SEL(16);
#undef SEL
  return hipGetLastError();
}

hipError_t launch_publish_ids(const int32_t* ids, int n, int32_t* host, int32_t seq, hipStream_t s) {
  hipLaunchKernelGGL(publish_ids_kernel, dim3(1), dim3(64), 0, s, ids, n, host, seq);
  return hipGetLastError();
}

hipError_t launch_status(int32_t* dst, const int32_t* src, hipStream_t s) {
  hipLaunchKernelGGL(status_kernel, dim3(1), dim3(64), 0, s, dst, src);
  return hipGetLastError();
}

hipError_t launch_route_onepass(const uint16_t* x, const float* wr, float* logits, int H, int E, int K, unsigned flags,
                                int32_t* ids, float* w, uint64_t* words, int32_t* status, hipStream_t s) {
  const int epl = (E + 63) / 64;
#define OP(N) hipLaunchKernelGGL(route_onepass_kernel<N>, dim3(E), dim3(256), 0, s, x, wr, logits, H, E, K, flags, ids, \
                                 w, words, status)
  if (epl <= 1) OP(1);
  else if (epl <= 2) OP(2);
  else if (epl <= 4) OP(4);
  else if (epl <= 8) OP(8);
  else OP(16);
#undef OP
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
