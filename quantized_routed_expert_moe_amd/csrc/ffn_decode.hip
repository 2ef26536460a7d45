// Single-token decode expert FFN: the HBM-bound hot path of a decode step.
//
// One token routes to K experts (plus an optional always-on shared expert);
// the layer streams K (+1) int4 expert blobs once ("Strata" README, Models:
// 4-bit grouped integer experts run W4A16). Two kernels, each built so that no
// workgroup barrier stands between issuing the weight loads and using them (a
// barrier waits for every outstanding load): every wave stages the slice of
// x or h it needs into its own LDS region, and the only barrier comes after
// the last weight byte has been consumed.
//
// dec_gateup: work item = (unit, 16 rows of I); wave w owns the contiguous
//   quarter of the groups [w*GW, (w+1)*GW). Lane (row r, phase p) reads groups
//   w*GW + 4i + p of its row in gate and up. Codes become bf16 pairs (16 + u,
//   u = q + 8 the stored nibble, exact in bf16) reduced against x with v_dot2;
//   sum_c q_c x_c = D - 24 * sum_c x_c per group, times the group's fp16 scale.
//   Phases then waves are summed in a fixed order; h = silu(g) * u in fp32.
// dec_down: work item = 8 rows of H for all units at once, so the combine needs
//   no further kernel. The flattened (unit, group) columns are split into four
//   contiguous ranges, one per wave; at step i the 8 phases of a wave read
//   columns 8i .. 8i+7 of its range, which belong to one unit (groups per unit
//   are a multiple of 8). P = sum_c u_c h_c in fp32, sum_c q_c h_c = P - 8 *
//   sum_c h_c. Per-unit sums go over phases, then waves, in a fixed order, and
//   y = o_shared + sum_k w[k] * o_k in rank order, rounded once to bf16.
// No atomics and no data-dependent reduction order: results depend only on
// the inputs, never on slot addresses.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t nib_pair(uint32_t w, int p) {
  const uint32_t sh = p == 0 ? (w << 3) : (w >> (4 * p - 3));
  return (sh & 0x00780078u) | 0x41804180u;  // bf16 pair (16 + u_lo, 16 + u_hi)
}

__device__ inline float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

__device__ inline float bf16_sum2(uint32_t v) {
  return __uint_as_float(v << 16) + __uint_as_float(v & 0xFFFF0000u);
}

// Blob of unit u (u = 0 is the shared expert when present) or nullptr with the
// status word set.
__device__ inline const uint8_t* dec_unit_blob(const FfnArgs& a, int u, bool has_shared) {
  const int k = has_shared ? u - 1 : u;
  if (k < 0) return a.shared_blob;
  const int e = a.ids[k];
  if (e < 0 || e >= a.E) {
    *a.status = MOE_EINVAL;
    return nullptr;
  }
  const int slot = a.slot_table[e];
  if (slot < 0) {
    *a.status = MOE_ENOTRES;
    return nullptr;
  }
  return a.slots + (size_t)slot * a.stride;
}

__device__ inline int unit_pair(int u, int K, bool has_shared) {
  return (has_shared && u == 0) ? K : u - (has_shared ? 1 : 0);
}

// ------------------------------------------------------------------ gate/up
// GPL = groups per lane = ceil(GW / 4) with GW = ceil(G / 4) groups per wave.
template <int GPL>
__global__ void __launch_bounds__(kThreads) dec_gateup_kernel(FfnArgs a) {
  // LDS per wave: x slice [GW*16] dwords (bf16 pairs) + group sums [GW]
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float part[2][kWaves][16];
  const int H = a.H, I = a.I, K = a.K;
  const int G = H / kGroup;
  const int GW = (G + kWaves - 1) / kWaves;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, p = lane >> 4;
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem) + (size_t)wave * (GW * 16 + GW);
  float* Xs = reinterpret_cast<float*>(xs + GW * 16);
  const int j0 = wave * GW;
  const int gw_here = G - j0 < GW ? (G - j0 > 0 ? G - j0 : 0) : GW;  // groups this wave really owns
  const bool has_shared = a.shared_blob != nullptr;
  const int n_units = K + (has_shared ? 1 : 0);
  const int n_rb = I / 16;
  const int n_items = n_units * n_rb;
  const BlobLayout BL = blob_layout(H, I);
  float* hws = reinterpret_cast<float*>(a.ws);  // h [pair][I]; routed pair k, shared pair K
  bool staged = false;
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int u = item / n_rb, rb = item % n_rb;
    const uint8_t* blob = dec_unit_blob(a, u, has_shared);
    const int n = rb * 16 + r;
    uint4 xv[2];
    if (!staged) {  // this wave's slice of x: 32 bytes per lane, issued before the weights
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int q = lane * 2 + v;  // uint4 index within the slice (8 bf16 each)
        xv[v] = q < gw_here * 4 ? reinterpret_cast<const uint4*>(a.x + (size_t)j0 * kGroup)[q]
                                : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    uint4 cg[GPL], cu[GPL];
    _Float16 sgh[GPL], suh[GPL];
    if (blob) {
#pragma unroll
      for (int i = 0; i < GPL; ++i) {
        const int jl = 4 * i + p;
        const int j = j0 + (jl < gw_here ? jl : (gw_here > 0 ? gw_here - 1 : 0));
        const int jj = j < G ? j : G - 1;
        const size_t co = ((size_t)jj * I + n) * 16;
        cg[i] = *reinterpret_cast<const uint4*>(blob + BL.gate_codes + co);
        cu[i] = *reinterpret_cast<const uint4*>(blob + BL.up_codes + co);
        const size_t so = (((size_t)(n / kScaleBlock) * G + jj) * kScaleBlock + n % kScaleBlock) * 2;
        sgh[i] = *reinterpret_cast<const _Float16*>(blob + BL.gate_scales + so);
        suh[i] = *reinterpret_cast<const _Float16*>(blob + BL.up_scales + so);
      }
    }
    if (!staged) {
      // lane pair (2m, 2m+1) holds group m of the slice: its sum in a fixed order
      float s = 0.0f;
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        s += bf16_sum2(xv[v].x);
        s += bf16_sum2(xv[v].y);
        s += bf16_sum2(xv[v].z);
        s += bf16_sum2(xv[v].w);
      }
      const float s_odd = __shfl_xor(s, 1, 64);
      if (lane * 2 < gw_here * 4) {
        reinterpret_cast<uint4*>(xs)[lane * 2] = xv[0];
        reinterpret_cast<uint4*>(xs)[lane * 2 + 1] = xv[1];
        if ((lane & 1) == 0) Xs[lane >> 1] = s + s_odd;
      }
      __builtin_amdgcn_wave_barrier();  // LDS ops of one wave complete in order
      staged = true;
    }
    float ag = 0.0f, au = 0.0f;
    if (blob) {
#pragma unroll
      for (int i = 0; i < GPL; ++i) {
        const int jl = 4 * i + p;
        const bool ok = jl < gw_here;
        const int jc = ok ? jl : 0;
        const uint4* xq = reinterpret_cast<const uint4*>(xs + jc * 16);
        const uint4 x0 = xq[0], x1 = xq[1], x2 = xq[2], x3 = xq[3];
        const uint32_t xw[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                 x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
        const uint32_t gw[4] = {cg[i].x, cg[i].y, cg[i].z, cg[i].w};
        const uint32_t uw[4] = {cu[i].x, cu[i].y, cu[i].z, cu[i].w};
        float dg = 0.0f, du = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            dg = dot2(nib_pair(gw[d], q), xw[4 * d + q], dg);
            du = dot2(nib_pair(uw[d], q), xw[4 * d + q], du);
          }
        }
        const float X = Xs[jc];
        const float sg = ok ? (float)sgh[i] : 0.0f;
        const float su = ok ? (float)suh[i] : 0.0f;
        ag = fmaf(sg, fmaf(-24.0f, X, dg), ag);
        au = fmaf(su, fmaf(-24.0f, X, du), au);
      }
    }
    // phases (lane bits 4..5) in a fixed butterfly, then the four waves in order
    ag += __shfl_xor(ag, 16, 64);
    au += __shfl_xor(au, 16, 64);
    ag += __shfl_xor(ag, 32, 64);
    au += __shfl_xor(au, 32, 64);
    if (p == 0) {
      part[0][wave][r] = ag;
      part[1][wave][r] = au;
    }
    __syncthreads();
    if (tid < 16) {
      float g = 0.0f, uu = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        g += part[0][w][tid];
        uu += part[1][w][tid];
      }
      hws[(size_t)unit_pair(u, K, has_shared) * I + rb * 16 + tid] = blob ? silu(g) * uu : 0.0f;
    }
    __syncthreads();
  }
}

// ------------------------------------------------------------------ down + combine
// CPL = columns per lane; a wave owns CW = 8 * CPL consecutive columns.
template <int CPL>
__global__ void __launch_bounds__(kThreads) dec_down_kernel(FfnArgs a) {
  // LDS per wave: h slice [CW][32] floats + column sums [CW]
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kMaxUnits = kMaxK + 1;
  __shared__ float part[kWaves][kMaxUnits][8];
  __shared__ const uint8_t* ublob[kMaxUnits];
  const int H = a.H, I = a.I, K = a.K;
  const int Gd = I / kGroup;
  const bool has_shared = a.shared_blob != nullptr;
  const int n_units = K + (has_shared ? 1 : 0);
  const int C = n_units * Gd;
  constexpr int CW = 8 * CPL;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 7, p = lane >> 3;
  float* hs = reinterpret_cast<float*>(smem) + (size_t)wave * (CW * 32 + CW);
  float* hsum = hs + CW * 32;
  const int c0 = wave * CW;
  const float* hws = reinterpret_cast<const float*>(a.ws);
  const BlobLayout BL = blob_layout(H, I);
  if (tid < n_units) ublob[tid] = dec_unit_blob(a, tid, has_shared);
  for (int q = tid; q < kWaves * kMaxUnits * 8; q += kThreads) (&part[0][0][0])[q] = 0.0f;
  __syncthreads();  // before any weight load is issued
  const int n_rb = H / 8;
  bool staged = false;
  for (int rb = blockIdx.x; rb < n_rb; rb += gridDim.x) {
    const int n = rb * 8 + r;
    // this wave's h slice: float4 q of the slice is column c0 + q/8, floats 4*(q%8) .. +3
    float4 hv[CPL];
    if (!staged) {
#pragma unroll
      for (int m = 0; m < CPL; ++m) {
        const int q = lane + 64 * m;
        const int c = c0 + q / 8;
        if (c < C) {
          const int u = c / Gd, j = c % Gd;
          hv[m] = reinterpret_cast<const float4*>(hws + (size_t)unit_pair(u, K, has_shared) * I + j * kGroup)[q % 8];
        } else {
          hv[m] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
    }
    uint4 cd[CPL];
    _Float16 sdh[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = c0 + 8 * i + p;
      const int cc = c < C ? c : C - 1;
      const int u = cc / Gd, j = cc % Gd;
      const uint8_t* blob = ublob[u];
      if (blob) {
        cd[i] = *reinterpret_cast<const uint4*>(blob + BL.down_codes + ((size_t)j * H + n) * 16);
        const size_t so = (((size_t)(n / kScaleBlock) * Gd + j) * kScaleBlock + n % kScaleBlock) * 2;
        sdh[i] = *reinterpret_cast<const _Float16*>(blob + BL.down_scales + so);
      } else {
        cd[i] = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
        sdh[i] = (_Float16)0.0f;
      }
    }
    if (!staged) {
#pragma unroll
      for (int m = 0; m < CPL; ++m) {
        const int q = lane + 64 * m;
        reinterpret_cast<float4*>(hs)[q] = hv[m];
        // lanes 8t .. 8t+7 hold one column: sum its 32 floats in a fixed order
        float s = ((hv[m].x + hv[m].y) + hv[m].z) + hv[m].w;
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        if ((lane & 7) == 0) hsum[q / 8] = s;
      }
      __builtin_amdgcn_wave_barrier();
      staged = true;
    }
    float acc = 0.0f;
    int cur = -1;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int cl = 8 * i + p;  // column within the wave's range
      const int ustep = (c0 + 8 * i) / Gd;  // one unit for the whole step (Gd % 8 == 0)
      if (c0 + 8 * i < C) {
        if (ustep != cur) {
          if (cur >= 0) {
            float t = acc;
            t += __shfl_xor(t, 8, 64);
            t += __shfl_xor(t, 16, 64);
            t += __shfl_xor(t, 32, 64);
            if (p == 0) part[wave][cur][r] = t;
          }
          acc = 0.0f;
          cur = ustep;
        }
        const float* hc = hs + cl * 32;
        const uint32_t cw[4] = {cd[i].x, cd[i].y, cd[i].z, cd[i].w};
        float P = 0.0f;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float4 h0 = reinterpret_cast<const float4*>(hc + 8 * d)[0];
          const float4 h1 = reinterpret_cast<const float4*>(hc + 8 * d)[1];
          const uint32_t lo = cw[d] & 0x0F0F0F0Fu;
          const uint32_t hi = (cw[d] >> 4) & 0x0F0F0F0Fu;
          // lo bytes hold columns +0, +4, +1, +5 of the dword; hi bytes +2, +6, +3, +7
          P = fmaf((float)(lo & 0xFF), h0.x, P);
          P = fmaf((float)((lo >> 8) & 0xFF), h1.x, P);
          P = fmaf((float)((lo >> 16) & 0xFF), h0.y, P);
          P = fmaf((float)(lo >> 24), h1.y, P);
          P = fmaf((float)(hi & 0xFF), h0.z, P);
          P = fmaf((float)((hi >> 8) & 0xFF), h1.z, P);
          P = fmaf((float)((hi >> 16) & 0xFF), h0.w, P);
          P = fmaf((float)(hi >> 24), h1.w, P);
        }
        acc = fmaf((float)sdh[i], fmaf(-8.0f, hsum[cl], P), acc);
      }
    }
    if (cur >= 0) {
      float t = acc;
      t += __shfl_xor(t, 8, 64);
      t += __shfl_xor(t, 16, 64);
      t += __shfl_xor(t, 32, 64);
      if (p == 0) part[wave][cur][r] = t;
    }
    __syncthreads();
    if (tid < 8) {
      float y = 0.0f;
      const int base = has_shared ? 1 : 0;
      if (has_shared) {
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) o += part[w][0][tid];
        y = o;
      }
      for (int k = 0; k < K; ++k) {
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) o += part[w][base + k][tid];
        y = fmaf(a.w[k], o, y);
      }
      a.y[(size_t)rb * 8 + tid] = __builtin_bit_cast(uint16_t, (__bf16)y);
    }
    __syncthreads();
    // the next row block rewrites exactly the entries this one wrote, so no re-zeroing
  }
}

inline void set_lds_limit(const void* fn, size_t lds) {
  if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

inline int dec_down_cpl(int n_units, int Gd) {
  const int C = n_units * Gd;
  const int per_wave = (C + kWaves - 1) / kWaves;
  return (per_wave + 7) / 8;
}

inline int round_cpl(int cpl) { return cpl <= 4 ? 4 : cpl <= 8 ? 8 : cpl <= 12 ? 12 : 16; }

}  // namespace

bool decode1_supported(int T, int H, int I, int K, bool has_shared) {
  const int n_units = K + (has_shared ? 1 : 0);
  const int G = H / kGroup, Gd = I / kGroup;
  // gate/up: at most 8 groups per lane; down: whole steps of 8 columns per unit, at most 16 per lane
  return T == 1 && G <= 4 * 4 * 8 && Gd % 8 == 0 && dec_down_cpl(n_units, Gd) <= 16;
}

hipError_t launch_ffn_decode1(const FfnArgs& a, int stage, hipStream_t s) {
  const bool has_shared = a.shared_blob != nullptr;
  const int n_units = a.K + (has_shared ? 1 : 0);
  if (stage == 0) {
    const int G = a.H / kGroup;
    const int GW = (G + kWaves - 1) / kWaves;
    const int gpl = (GW + 3) / 4;
    const size_t lds = (size_t)kWaves * (GW * 16 + GW) * 4;
    const int items = n_units * (a.I / 16);
    const int grid = items < 4096 ? items : 4096;
#define GU(N)                                                                                       \
  do {                                                                                              \
    set_lds_limit(reinterpret_cast<const void*>(&dec_gateup_kernel<N>), lds);                       \
    hipLaunchKernelGGL((dec_gateup_kernel<N>), dim3(grid), dim3(kThreads), lds, s, a);              \
  } while (0)
    if (gpl <= 1) GU(1);
    else if (gpl <= 2) GU(2);
    else if (gpl <= 4) GU(4);
    else GU(8);
#undef GU
    return hipGetLastError();
  }
  {
    const int Gd = a.I / kGroup;
    const int cpl = round_cpl(dec_down_cpl(n_units, Gd));
    const size_t lds = (size_t)kWaves * (8 * cpl * 32 + 8 * cpl) * 4;
    const int n_rb = a.H / 8;
    const int grid = n_rb < 4096 ? n_rb : 4096;
#define DN(N)                                                                                       \
  do {                                                                                              \
    set_lds_limit(reinterpret_cast<const void*>(&dec_down_kernel<N>), lds);                         \
    hipLaunchKernelGGL((dec_down_kernel<N>), dim3(grid), dim3(kThreads), lds, s, a);                \
  } while (0)
    if (cpl == 4) DN(4);
    else if (cpl == 8) DN(8);
    else if (cpl == 12) DN(12);
    else DN(16);
#undef DN
    return hipGetLastError();
  }
}

}  // namespace moe
