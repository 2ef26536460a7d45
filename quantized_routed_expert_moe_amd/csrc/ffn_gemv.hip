// Decode expert FFN (GEMV path): int4 group-32 dequant fused into SwiGLU,
// then down projection with the routing-weighted combine.
//
// The experts are W4A16 ("Strata" README, Models: 4-bit grouped integer
// experts with 16-bit activations): codes and fp16 scales stream from HBM once
// per layer call and are dequantised in registers. Work is split into items
// (unit, row block); a unit is one distinct expert (or the always-on shared
// expert) together with every token routed to it, so each expert's bytes are
// read once however many tokens use it.
//
// Kernel 1 (gate/up): item = (unit, 16 rows of I). Thread (row r, slice s)
//   loads the codes of its row for groups s, s+16, ... of gate and up, keeps
//   them in registers, and for each chunk of up to 4 tokens forms
//   D = sum_c bf16(16 + u_c) * x_c with v_dot2 (u = q + 8 is the stored nibble,
//   16 + u is exact in bf16), so sum_c q_c x_c = D - 24 * sum_c x_c; the group
//   result is scaled by its fp16 scale. Slices are summed in a fixed order in
//   LDS and h = silu(g) * u is written in fp32.
// Kernel 2 (down + combine): item = (unit, 32 rows of H). The same scheme in
//   fp32 (h is fp32): P = sum_c u_c h_c, sum_c q_c h_c = P - 8 * sum_c h_c.
//   Each item writes fp32 o rows for its pairs.
// Kernel 3 (combine): y[t] = o_shared[t] + sum_{k=0..K-1} w[t][k] * o[t][k],
//   added in rank order and rounded once to bf16.
// No floating-point atomics: the reduction order depends only on (T, K, E).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kTB = 4;  // tokens per chunk
constexpr int kRowsGU = 16;
constexpr int kSlicesGU = kThreads / kRowsGU;  // 16
constexpr int kRowsDN = 32;
constexpr int kSlicesDN = kThreads / kRowsDN;  // 8
constexpr int kMaxPairs = kGemvMaxT * kMaxK;   // 1024

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ workspace
struct GemvWs {
  size_t h_off, o_off, bytes;
};

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

__host__ __device__ inline GemvWs gemv_ws(int T, int H, int I, int K, int has_shared) {
  const size_t pairs = (size_t)T * K + (has_shared ? T : 0);
  GemvWs w;
  w.h_off = 0;
  w.o_off = align256(w.h_off + pairs * I * sizeof(float));
  w.bytes = align256(w.o_off + pairs * H * sizeof(float));
  return w;
}

// ------------------------------------------------------------------ plan
// LDS plan shared by both kernels: which units exist and which pairs belong to
// each. Pair p = t*K + k for routed pairs; the shared expert's pair for token
// t is T*K + t. Unit 0 is the shared expert when present.
struct PlanLds {
  int n_units;
  int list_n;
  int wcnt[kThreads / 64];
  int unit_expert[kMaxPairs + 1];   // routed expert id, -1 for the shared unit
  int unit_of_pair[kMaxPairs];      // routed pairs only; -1 when the id is invalid
  int first[kMaxE];                 // dedup scratch: lowest pair using expert e
  int uoe[kMaxE];                   // unit of expert e
  int list[kMaxPairs + kGemvMaxT];  // pair list of the current item's unit
};

// Block-wide ordered compaction of the indices i < n with pred(i) into out[];
// returns the count (identical in every thread).
template <typename Pred>
__device__ int block_compact(int n, Pred pred, int* out, int* wcnt) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int running = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tid;
    const bool f = i < n && pred(i);
    const unsigned long long m = __ballot(f);
    if (lane == 0) wcnt[wave] = __popcll(m);
    __syncthreads();
    int off = running, tot = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      if (w < wave) off += wcnt[w];
      tot += wcnt[w];
    }
    if (f) out[off + __popcll(m & ((1ull << lane) - 1ull))] = i;
    __syncthreads();
    running += tot;
  }
  return running;
}

__device__ void build_plan(PlanLds& pl, const int32_t* __restrict__ ids, int T, int K, int E, bool has_shared,
                           int32_t* status) {
  const int tid = threadIdx.x;
  const int P = T * K;
  const int base = has_shared ? 1 : 0;
  if (tid == 0) pl.unit_expert[0] = -1;
  if (T == 1) {
    // one token: its K pairs are the units (ids of one token are distinct when
    // they come from moe_route; duplicates would only cost a second read)
    for (int p = tid; p < P; p += kThreads) {
      const int e = ids[p];
      const bool ok = e >= 0 && e < E;
      if (!ok) *status = MOE_EINVAL;
      pl.unit_expert[base + p] = ok ? e : -2;
      pl.unit_of_pair[p] = base + p;
    }
    if (tid == 0) pl.n_units = base + P;
    __syncthreads();
    return;
  }
  for (int e = tid; e < E; e += kThreads) pl.first[e] = 0x7FFFFFFF;
  __syncthreads();
  for (int p = tid; p < P; p += kThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E)
      atomicMin(&pl.first[e], p);
    else
      *status = MOE_EINVAL;
  }
  __syncthreads();
  // leaders (first pair of each distinct expert) in pair order become units
  const int n_routed = block_compact(
      P,
      [&](int p) {
        const int e = ids[p];
        return e >= 0 && e < E && pl.first[e] == p;
      },
      pl.list, pl.wcnt);
  for (int u = tid; u < n_routed; u += kThreads) {
    const int e = ids[pl.list[u]];
    pl.unit_expert[base + u] = e;
    pl.uoe[e] = base + u;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kThreads) {
    const int e = ids[p];
    pl.unit_of_pair[p] = (e >= 0 && e < E) ? pl.uoe[e] : -1;
  }
  if (tid == 0) pl.n_units = base + n_routed;
  __syncthreads();
}

// Pair list of unit u into pl.list / pl.list_n (all threads must call).
__device__ void unit_pairs(PlanLds& pl, int u, int T, int K, bool has_shared) {
  if (has_shared && u == 0) {
    for (int t = threadIdx.x; t < T; t += kThreads) pl.list[t] = T * K + t;
    if (threadIdx.x == 0) pl.list_n = T;
    __syncthreads();
    return;
  }
  if (T == 1) {
    if (threadIdx.x == 0) {
      pl.list[0] = u - (has_shared ? 1 : 0);
      pl.list_n = 1;
    }
    __syncthreads();
    return;
  }
  const int n = block_compact(T * K, [&](int p) { return pl.unit_of_pair[p] == u; }, pl.list, pl.wcnt);
  if (threadIdx.x == 0) pl.list_n = n;
  __syncthreads();
}

__device__ inline int pair_token(int p, int T, int K) { return p < T * K ? p / K : p - T * K; }

// Blob of unit u or nullptr (status set) when the expert is not resident.
__device__ inline const uint8_t* unit_blob(const FfnArgs& a, int expert) {
  if (expert == -1) return a.shared_blob;
  if (expert < 0) return nullptr;
  const int slot = a.slot_table[expert];
  if (slot < 0) {
    *a.status = MOE_ENOTRES;
    return nullptr;
  }
  return a.slots + (size_t)slot * a.stride;
}

__device__ inline uint32_t nib_pair(uint32_t w, int p) {
  // nibbles p and p+4 of w -> bf16 pair (16 + u_lo, 16 + u_hi)
  const uint32_t sh = p == 0 ? (w << 3) : (w >> (4 * p - 3));
  return (sh & 0x00780078u) | 0x41804180u;
}

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// ------------------------------------------------------------------ gate/up
struct GuLds {
  PlanLds plan;
  float red[kTB][2][kSlicesGU][kRowsGU];
  float gsum[kTB][kRowsGU][2];
  // followed in dynamic memory by: x chunk bf16 [kTB][H], group sums fp32 [kTB][G]
};

template <int GPS, int TBC>
__global__ void __launch_bounds__(kThreads) ffn_gateup_kernel(FfnArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  GuLds& L = *reinterpret_cast<GuLds*>(smem_raw);
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem_raw + align256(sizeof(GuLds)));  // [kTB][H/2]
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const int G = H / kGroup;
  float* xsum = reinterpret_cast<float*>(xs + (size_t)kTB * H / 2);  // [kTB][G]
  const int tid = threadIdx.x;
  const int r = tid % kRowsGU, sl = tid / kRowsGU;
  const bool has_shared = a.shared_blob != nullptr;
  const GemvWs W = gemv_ws(T, H, I, K, has_shared);
  float* hws = reinterpret_cast<float*>(a.ws + W.h_off);
  build_plan(L.plan, a.ids, T, K, a.E, has_shared, a.status);
  const int n_rb = I / kRowsGU;
  const int n_items = L.plan.n_units * n_rb;
  const BlobLayout BL = blob_layout(H, I);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int u = item / n_rb, rb = item % n_rb;
    const int n = rb * kRowsGU + r;
    const uint8_t* blob = unit_blob(a, L.plan.unit_expert[u]);
    unit_pairs(L.plan, u, T, K, has_shared);
    const int npairs = L.plan.list_n;
    if (!blob) {  // expert not resident (status already set): h = 0 for its pairs
      for (int idx = tid; idx < npairs * kRowsGU; idx += kThreads)
        hws[(size_t)L.plan.list[idx / kRowsGU] * I + rb * kRowsGU + idx % kRowsGU] = 0.0f;
      __syncthreads();
      continue;
    }
    uint4 cg[GPS], cu[GPS];
    _Float16 sgh[GPS], suh[GPS];
#pragma unroll
    for (int i = 0; i < GPS; ++i) {
      const int jr = sl + kSlicesGU * i;
      const int j = jr < G ? jr : G - 1;  // out-of-range slices reload the last group, scaled by 0 below
      const size_t co = code_off(n, j, G, kRowBlockGU);
      cg[i] = *reinterpret_cast<const uint4*>(blob + BL.gate_codes + co);
      cu[i] = *reinterpret_cast<const uint4*>(blob + BL.up_codes + co);
      const size_t so = scale_off(n, j, G, kRowBlockGU);
      sgh[i] = *reinterpret_cast<const _Float16*>(blob + BL.gate_scales + so);
      suh[i] = *reinterpret_cast<const _Float16*>(blob + BL.up_scales + so);
    }
    for (int c0 = 0; c0 < npairs; c0 += TBC) {
      const int tc = npairs - c0 < TBC ? npairs - c0 : TBC;
      // The code registers are opaque per chunk, so their dequantised form is
      // recomputed in each chunk instead of being hoisted out (which would
      // hold every group's bf16 pairs in registers at once).
#pragma unroll
      for (int i = 0; i < GPS; ++i)
        asm volatile("" : "+v"(cg[i].x), "+v"(cg[i].y), "+v"(cg[i].z), "+v"(cg[i].w), "+v"(cu[i].x), "+v"(cu[i].y),
                     "+v"(cu[i].z), "+v"(cu[i].w));
      // stage x of the chunk's tokens and their group sums
      for (int idx = tid; idx < tc * (H / 8); idx += kThreads) {
        const int ti = idx / (H / 8), q = idx % (H / 8);
        const int t = pair_token(L.plan.list[c0 + ti], T, K);
        reinterpret_cast<uint4*>(xs + (size_t)ti * H / 2)[q] =
            reinterpret_cast<const uint4*>(a.x + (size_t)t * H)[q];
      }
      __syncthreads();
      for (int idx = tid; idx < tc * G; idx += kThreads) {
        const int ti = idx / G, j = idx % G;
        const uint32_t* xv = xs + (size_t)ti * H / 2 + j * 16;
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          s += __uint_as_float(xv[q] << 16);
          s += __uint_as_float(xv[q] & 0xFFFF0000u);
        }
        xsum[ti * G + j] = s;
      }
      __syncthreads();
      float ag[TBC], au[TBC];
#pragma unroll
      for (int ti = 0; ti < TBC; ++ti) ag[ti] = au[ti] = 0.0f;
#pragma unroll
      for (int i = 0; i < GPS; ++i) {
        const int jr = sl + kSlicesGU * i;
        const int j = jr < G ? jr : G - 1;
        const float sgi = jr < G ? (float)sgh[i] : 0.0f;
        const float sui = jr < G ? (float)suh[i] : 0.0f;
        {
#pragma unroll
          for (int ti = 0; ti < TBC; ++ti) {
            if (ti < tc) {
              const uint4* xq = reinterpret_cast<const uint4*>(xs + (size_t)ti * H / 2 + j * 16);
              const uint4 x0 = xq[0], x1 = xq[1], x2 = xq[2], x3 = xq[3];
              const uint32_t xw[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                       x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
              const uint32_t gw[4] = {cg[i].x, cg[i].y, cg[i].z, cg[i].w};
              const uint32_t uw[4] = {cu[i].x, cu[i].y, cu[i].z, cu[i].w};
              float dg = 0.0f, du = 0.0f;
#pragma unroll
              for (int d = 0; d < 4; ++d) {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                  dg = dot2(nib_pair(gw[d], p), xw[4 * d + p], dg);
                  du = dot2(nib_pair(uw[d], p), xw[4 * d + p], du);
                }
              }
              const float X = xsum[ti * G + j];
              ag[ti] = fmaf(sgi, fmaf(-24.0f, X, dg), ag[ti]);
              au[ti] = fmaf(sui, fmaf(-24.0f, X, du), au[ti]);
            }
          }
        }
      }
#pragma unroll
      for (int ti = 0; ti < TBC; ++ti) {
        L.red[ti][0][sl][r] = ag[ti];
        L.red[ti][1][sl][r] = au[ti];
      }
      __syncthreads();
      if (tid < tc * kRowsGU) {
        const int ti = tid / kRowsGU, rr = tid % kRowsGU;
        float g = 0.0f, uu = 0.0f;
#pragma unroll
        for (int s = 0; s < kSlicesGU; ++s) {
          g += L.red[ti][0][s][rr];
          uu += L.red[ti][1][s][rr];
        }
        const int p = L.plan.list[c0 + ti];
        hws[(size_t)p * I + rb * kRowsGU + rr] = silu(g) * uu;
      }
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ down + combine
struct DnLds {
  PlanLds plan;
  float red[kTB][kSlicesDN][kRowsDN];
  // followed by: h chunk fp32 [kTB][I], group sums fp32 [kTB][Gd]
};

template <int GPS, int TBC>
__global__ void __launch_bounds__(kThreads) ffn_down_kernel(FfnArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DnLds& L = *reinterpret_cast<DnLds*>(smem_raw);
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const int Gd = I / kGroup;
  float* hs = reinterpret_cast<float*>(smem_raw + align256(sizeof(DnLds)));  // [kTB][I]
  float* hsum = hs + (size_t)kTB * I;                                          // [kTB][Gd]
  const int tid = threadIdx.x;
  const int r = tid % kRowsDN, sl = tid / kRowsDN;
  const bool has_shared = a.shared_blob != nullptr;
  const GemvWs W = gemv_ws(T, H, I, K, has_shared);
  const float* hws = reinterpret_cast<const float*>(a.ws + W.h_off);
  float* ows = reinterpret_cast<float*>(a.ws + W.o_off);
  build_plan(L.plan, a.ids, T, K, a.E, has_shared, a.status);
  const int n_rb = H / kRowsDN;
  const int n_units = L.plan.n_units;
  const int n_items = n_units * n_rb;
  const BlobLayout BL = blob_layout(H, I);
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int u = item % n_units, rb = item / n_units;  // units of a row block are adjacent items
    const int n = rb * kRowsDN + r;
    const uint8_t* blob = unit_blob(a, L.plan.unit_expert[u]);
    unit_pairs(L.plan, u, T, K, has_shared);
    const int npairs = L.plan.list_n;
    uint4 cd[GPS];
    _Float16 sdh[GPS];
    if (blob) {
#pragma unroll
      for (int i = 0; i < GPS; ++i) {
        const int jr = sl + kSlicesDN * i;
        const int j = jr < Gd ? jr : Gd - 1;
        cd[i] = *reinterpret_cast<const uint4*>(blob + BL.down_codes + code_off(n, j, Gd, kRowBlockDN));
        const size_t so = scale_off(n, j, Gd, kRowBlockDN);
        sdh[i] = *reinterpret_cast<const _Float16*>(blob + BL.down_scales + so);
      }
    } else {  // expert not resident (status already set): o = 0 for its pairs
#pragma unroll
      for (int i = 0; i < GPS; ++i) {
        cd[i] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        sdh[i] = (_Float16)0.0f;
      }
    }
    for (int c0 = 0; c0 < npairs; c0 += TBC) {
      const int tc = npairs - c0 < TBC ? npairs - c0 : TBC;
#pragma unroll
      for (int i = 0; i < GPS; ++i) asm volatile("" : "+v"(cd[i].x), "+v"(cd[i].y), "+v"(cd[i].z), "+v"(cd[i].w));
      for (int idx = tid; idx < tc * (I / 4); idx += kThreads) {
        const int ti = idx / (I / 4), q = idx % (I / 4);
        const int p = L.plan.list[c0 + ti];
        reinterpret_cast<float4*>(hs + (size_t)ti * I)[q] = reinterpret_cast<const float4*>(hws + (size_t)p * I)[q];
      }
      __syncthreads();
      for (int idx = tid; idx < tc * Gd; idx += kThreads) {
        const int ti = idx / Gd, j = idx % Gd;
        const float* hv = hs + (size_t)ti * I + j * kGroup;
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < kGroup; ++q) s += hv[q];
        hsum[ti * Gd + j] = s;
      }
      __syncthreads();
      float acc[TBC];
#pragma unroll
      for (int ti = 0; ti < TBC; ++ti) acc[ti] = 0.0f;
#pragma unroll
      for (int i = 0; i < GPS; ++i) {
        const int jr = sl + kSlicesDN * i;
        const int j = jr < Gd ? jr : Gd - 1;
        const float sdi = jr < Gd ? (float)sdh[i] : 0.0f;
        {
          const uint32_t cw[4] = {cd[i].x, cd[i].y, cd[i].z, cd[i].w};
#pragma unroll
          for (int ti = 0; ti < TBC; ++ti) {
            if (ti < tc) {
              const float* hv = hs + (size_t)ti * I + j * kGroup;
              float P = 0.0f;
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const float4 h0 = reinterpret_cast<const float4*>(hv + 8 * d)[0];
                const float4 h1 = reinterpret_cast<const float4*>(hv + 8 * d)[1];
                const uint32_t lo = cw[d] & 0x0F0F0F0Fu;
                const uint32_t hi = (cw[d] >> 4) & 0x0F0F0F0Fu;
                // lo bytes: columns +0, +4, +1, +5; hi bytes: +2, +6, +3, +7
                P = fmaf((float)(lo & 0xFF), h0.x, P);
                P = fmaf((float)((lo >> 8) & 0xFF), h1.x, P);
                P = fmaf((float)((lo >> 16) & 0xFF), h0.y, P);
                P = fmaf((float)(lo >> 24), h1.y, P);
                P = fmaf((float)(hi & 0xFF), h0.z, P);
                P = fmaf((float)((hi >> 8) & 0xFF), h1.z, P);
                P = fmaf((float)((hi >> 16) & 0xFF), h0.w, P);
                P = fmaf((float)(hi >> 24), h1.w, P);
              }
              acc[ti] = fmaf(sdi, fmaf(-8.0f, hsum[ti * Gd + j], P), acc[ti]);
            }
          }
        }
      }
#pragma unroll
      for (int ti = 0; ti < TBC; ++ti) L.red[ti][sl][r] = acc[ti];
      __syncthreads();
      if (tid < tc * kRowsDN) {
        const int ti = tid / kRowsDN, rr = tid % kRowsDN;
        float o = 0.0f;
#pragma unroll
        for (int s = 0; s < kSlicesDN; ++s) o += L.red[ti][s][rr];
        const int p = L.plan.list[c0 + ti];
        ows[(size_t)p * H + rb * kRowsDN + rr] = o;
      }
      __syncthreads();
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ combine
__global__ void __launch_bounds__(kThreads) ffn_combine_kernel(FfnArgs a) {
  const int H = a.H, T = a.T, K = a.K;
  const bool has_shared = a.shared_blob != nullptr;
  const GemvWs W = gemv_ws(T, H, a.I, K, has_shared);
  const float* ows = reinterpret_cast<const float*>(a.ws + W.o_off);
  const size_t total = (size_t)T * H;
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += (size_t)gridDim.x * kThreads) {
    const int t = (int)(idx / H);
    const size_t col = idx % H;
    float acc = has_shared ? ows[(size_t)(T * K + t) * H + col] : 0.0f;
    for (int k = 0; k < K; ++k) acc = fmaf(a.w[t * K + k], ows[(size_t)(t * K + k) * H + col], acc);
    a.y[idx] = __builtin_bit_cast(uint16_t, (__bf16)acc);
  }
}

// Dynamic LDS beyond 64 KiB must be allowed per kernel (gfx950 has 160 KiB per CU).
inline void set_lds_limit(const void* fn, size_t lds) {
  if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

inline int pow2_at_least(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

}  // namespace

// one token: the K resolved slots (256 bytes), then the one-pass routing region
size_t gemv_workspace_bytes(int T, int H, int I, int K, int has_shared) {
  return gemv_ws(T, H, I, K, has_shared).bytes + (T == 1 ? 256 + onepass_region_bytes(kMaxE, kMaxK) : 0);
}

size_t decode1_slots_offset(int H, int I, int K, int has_shared) { return gemv_ws(1, H, I, K, has_shared).bytes; }

hipError_t launch_ffn_gemv(const FfnArgs& a, int stage, hipStream_t s) {
  const bool has_shared = a.shared_blob != nullptr;
  const int max_units = (a.T == 1 ? a.K : (a.T * a.K < a.E ? a.T * a.K : a.E)) + (has_shared ? 1 : 0);
  const int tbc = a.T == 1 ? 1 : kTB;  // tokens per chunk: a single token needs no chunk registers
  // gate/up
  if (stage == 0) {
    const int G = a.H / kGroup;
    const int gps = pow2_at_least((G + kSlicesGU - 1) / kSlicesGU);
    const size_t lds = align256(sizeof(GuLds)) + (size_t)kTB * a.H * 2 + (size_t)kTB * G * 4;
    const int items = max_units * (a.I / kRowsGU);
    const int grid = items < 4096 ? items : 4096;
    switch (gps * 8 + tbc) {
#define GU_CASE(N) \
  case N * 8 + 1:  \
    set_lds_limit(reinterpret_cast<const void*>(&ffn_gateup_kernel<N, 1>), lds);                \
    hipLaunchKernelGGL((ffn_gateup_kernel<N, 1>), dim3(grid), dim3(kThreads), lds, s, a); \
    break;         \
  case N * 8 + kTB: \
    set_lds_limit(reinterpret_cast<const void*>(&ffn_gateup_kernel<N, kTB>), lds);                \
    hipLaunchKernelGGL((ffn_gateup_kernel<N, kTB>), dim3(grid), dim3(kThreads), lds, s, a); \
    break;
      GU_CASE(1) GU_CASE(2) GU_CASE(4) GU_CASE(8) GU_CASE(16)
#undef GU_CASE
      default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  // down + combine
  {
    const int Gd = a.I / kGroup;
    const int gps = pow2_at_least((Gd + kSlicesDN - 1) / kSlicesDN);
    const size_t lds = align256(sizeof(DnLds)) + (size_t)kTB * a.I * 4 + (size_t)kTB * Gd * 4;
    const int items = max_units * (a.H / kRowsDN);
    const int grid = items < 4096 ? items : 4096;
    switch (gps * 8 + tbc) {
#define DN_CASE(N) \
  case N * 8 + 1:  \
    set_lds_limit(reinterpret_cast<const void*>(&ffn_down_kernel<N, 1>), lds);                \
    hipLaunchKernelGGL((ffn_down_kernel<N, 1>), dim3(grid), dim3(kThreads), lds, s, a); \
    break;         \
  case N * 8 + kTB: \
    set_lds_limit(reinterpret_cast<const void*>(&ffn_down_kernel<N, kTB>), lds);                \
    hipLaunchKernelGGL((ffn_down_kernel<N, kTB>), dim3(grid), dim3(kThreads), lds, s, a); \
    break;
      DN_CASE(1) DN_CASE(2) DN_CASE(4) DN_CASE(8) DN_CASE(16)
#undef DN_CASE
      default:
        return hipErrorInvalidValue;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const size_t total = (size_t)a.T * a.H;
    const size_t blocks = (total + kThreads - 1) / kThreads;
    const int grid = blocks < 2048 ? (int)blocks : 2048;
    hipLaunchKernelGGL(ffn_combine_kernel, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
}

}  // namespace moe
