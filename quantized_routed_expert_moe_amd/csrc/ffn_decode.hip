// Single-token decode expert FFN: the HBM-bound hot path of a decode step.
//
// One token routes to K experts (plus an optional always-on shared expert);
// the layer streams K (+1) int4 expert blobs once ("Strata" README, Models:
// 4-bit grouped integer experts run W4A16). Two kernels, both shaped for
// streaming: many small workgroups (each reads 24-36 KB of codes, about six
// workgroups per CU), every weight load of a wave issued up front in the
// order the steps consume them, and straight-line code between loads and
// use, so each step waits only for its own loads while later ones are still
// in flight. No workgroup barrier stands between the loads and their use (a
// barrier waits for every outstanding load): each wave stages the slice of x
// or h it needs in its own LDS region.
//
// Arithmetic (both kernels). Activations become fp16 pairs; a code dword w
// (8 offset-binary nibbles u = q + 8, see the blob layout) gives four fp16
// pairs with one AND-OR each (two also need w >> 8):
//   A pairs (nibbles at bits 0..3 / 16..19 of w or w >> 8): 0x6400 | u = 1024 + u = q + 1032
//   B pairs (nibbles at bits 4..7 / 20..23):                 0x5400 | 16u = 64 + u = q + 72
// all exact. v_dot2_f32_f16 multiplies them with the activation pairs of the
// same columns (A pairs cover columns 8d + {0,1,4,5} of dword d, B pairs
// 8d + {2,3,6,7}) and accumulates in fp32, so per group
//   sum_c q_c a_c = D - (1032 * A_sum + 72 * B_sum)
// with A_sum / B_sum the sums of the fp16 activations over those columns,
// computed once per group when the activations are staged. The group's fp16
// scale multiplies that in fp32. Activations that do not fit fp16 (|v| >=
// 65520) set MOE_EUNSUP in the status word; bf16 x converts exactly for
// |x| in [2^-17, 65504].
//
// dec_gateup: one workgroup per (unit, 8 rows of I); wave w owns the
//   contiguous quarter of the groups [w*GW, (w+1)*GW). Lane (row r of 8,
//   phase p of 8) takes groups w*GW + 8i + p of its row in gate and up: per
//   step a wave reads eight 128-byte lines per matrix. Phases then waves are
//   summed in a fixed order; h = silu(g) * u is stored as fp16.
// dec_down: one workgroup per 8 rows of H (two quads of 4) for all units at
//   once, so the combine needs no further kernel; each wave's staged h slice
//   and its LDS reads serve both quads. The flattened (unit, group) columns are
//   split into four contiguous ranges, one per wave; at step i lane (row r of
//   4 in each quad, phase p of 16) takes column 16i + p of its wave's range; the 16
//   columns of a step belong to one unit (groups per unit are a multiple of
//   16). Per-unit sums go over phases, then waves, in a fixed order, and
//   y = o_shared + sum_k w[k] * o_k in rank order, rounded once to bf16.
// Workgroups are dealt to the 8 XCDs in contiguous runs of items, so the
// workgroups that share a 16-row block of the blob run in one L2.
// No atomics and no data-dependent reduction order: results depend only on
// the inputs, never on slot addresses.
#include "moe_internal.h"
#include "onepass.h"
#include "timeline.h"
#include "wave_ops.h"

namespace moe {
MOE_TL_UNIT(decode, MOE_TL_DEC_ROUTE_GATEUP, 3)
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kXcds = 8;

// Expert codes and scales are read once per token: their loads carry the
// non-temporal hint, so that the streamed weights do not evict from the caches
// what the next dispatches read again (router weights, x, h, the hand-off words).
typedef unsigned int StreamU32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 stream_u4(const uint8_t* p) {
  const StreamU32x4 v = __builtin_nontemporal_load(reinterpret_cast<const StreamU32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t stream_u32(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
// Blob of unit u (u = 0 is the shared expert when present) or nullptr with the
// status word set; ids = the token's routed experts in rank order.
// With pre_slots (moe_layer) the routing kernel has resolved the slots already:
// pre is a.pre_slots as a constant-space pointer, so that the workgroup's slot
// (u is uniform) comes from one scalar load.
typedef const __attribute__((address_space(4))) int32_t* const_i32p;
__device__ inline const uint8_t* dec_unit_blob(const FfnArgs& a, int u, bool has_shared, const int32_t* ids,
                                               const_i32p pre) {
  const int k = has_shared ? u - 1 : u;
  if (k < 0) return a.shared_blob;
  int slot;
  if (pre) {
    slot = pre[k];
  } else {
    const int e = ids[k];
    if (e < 0 || e >= a.E) {
      *a.status = MOE_EINVAL;
      return nullptr;
    }
    slot = a.slot_table[e];
  }
  if (slot < 0) {
    *a.status = MOE_ENOTRES;
    return nullptr;
  }
  return a.slots + (size_t)slot * a.stride;
}

__device__ inline int unit_pair(int u, int K, bool has_shared) {
  return (has_shared && u == 0) ? K : u - (has_shared ? 1 : 0);
}

// Item of workgroup bid when items are dealt to the XCDs in contiguous runs
// (workgroups are dispatched to XCD bid % 8).
__device__ inline int xcd_item(int bid, int n_items) {
  return n_items % kXcds == 0 ? (bid % kXcds) * (n_items / kXcds) + bid / kXcds : bid;
}

// One-pass path: the blob of unit u from the selector's slot word of this call,
// polled by the first wave only (one poller per workgroup) and handed to the
// others through LDS.
__device__ inline const uint8_t* onepass_unit_blob(const FfnArgs& a, int u, bool has_shared, const uint64_t* words,
                                                   uint32_t ep, int wave) {
  const int k = has_shared ? u - 1 : u;
  if (k < 0) return a.shared_blob;
  __shared__ int32_t slot_sh;
  if (wave == 0) {
    const int32_t sl = onepass_wait_slot(words, a.E, k, ep, blockIdx.x % kOnepassCopies);
    if ((threadIdx.x & 63) == 0) slot_sh = sl;
  }
  __syncthreads();
  const int32_t slot = slot_sh;
  if (slot < 0) {
    *a.status = slot == (int32_t)0x80000000 ? MOE_EHIP : MOE_ENOTRES;  // hand-off timed out / not resident
    return nullptr;
  }
  return a.slots + (size_t)slot * a.stride;
}

// ------------------------------------------------------------------ gate/up
// GPL = groups per lane = ceil(GW / 8) with GW = ceil(G / 4) groups per wave.
// bid: the workgroup's index among the gate/up workgroups. ONEPASS: the unit's
// slot comes from the one-pass hand-off words (epoch ep) instead of the table.
template <int GPL, bool ONEPASS>
__device__ __forceinline__ void dec_gateup_body(const FfnArgs& a, int bid, const uint64_t* words, uint32_t ep,
                                                const TlRow& tl) {
  // LDS per wave: x slice as fp16 pairs [GW][16] dwords + group corrections [GW]
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float part[2][kWaves][8];
  const int H = a.H, I = a.I, K = a.K;
  const int G = H / kGroup;
  const int GW = (G + kWaves - 1) / kWaves;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 7, p = lane >> 3;
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem) + (size_t)wave * (GW * 17);
  float* Cs = reinterpret_cast<float*>(xs + GW * 16);
  const int j0 = wave * GW;
  const int gw_here = G - j0 < GW ? (G - j0 > 0 ? G - j0 : 0) : GW;  // groups this wave really owns
  const bool has_shared = a.shared_blob != nullptr;
  // the resolved slots' pointer in registers now, with the first argument loads (left
  // to the compiler, it is loaded after them: one more round trip before the weights)
  const_i32p pre = (const_i32p)a.pre_slots;
  asm volatile("" : "+s"(pre));
  const int n_hb = I / 8;
  // ONEPASS: the ranks' slots arrive one after another, so each unit's row blocks
  // are dealt round-robin over the XCDs (every XCD streams rank 0 first); else
  // each XCD takes a contiguous run of items
  const int item = ONEPASS ? bid : xcd_item(bid, (K + (has_shared ? 1 : 0)) * n_hb);
  const int u = item / n_hb, hb = item % n_hb;
  // 1. this wave's slice of x: uint4 q (8 bf16) of the slice = columns 8q .. 8q+7
  //    (issued before the two dependent loads that find the unit's blob)
  uint4 xv[2];
#pragma unroll
  for (int v = 0; v < 2; ++v) {
    int q = j0 * 4 + lane * 2 + v;
    q = q < G * 4 ? q : G * 4 - 1;
    xv[v] = reinterpret_cast<const uint4*>(a.x)[q];
  }
  // 2. x -> fp16 pairs, group corrections, into LDS (lanes 2m, 2m+1 hold group m),
  //    before the weight loads, whose registers are not live yet (register
  //    pressure). The standalone kernel stages x after the slot lookup (x has
  //    arrived during its two dependent loads); the one-pass items stage it while
  //    the selection runs, so that their weight loads follow the slot at once.
  bool bad = false;
  auto stage_x = [&]() {
    const bool live = lane * 2 < gw_here * 4;
    uint32_t xh[8];
    float sa = 0.0f, sb = 0.0f;
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const uint32_t d[4] = {xv[v].x, xv[v].y, xv[v].z, xv[v].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t lo = to_f16_bits(__uint_as_float(d[c] << 16), &bad);
        const uint32_t hi = to_f16_bits(__uint_as_float(d[c] & 0xFFFF0000u), &bad);
        const uint32_t pr = live ? (lo | (hi << 16)) : 0u;
        xh[4 * v + c] = pr;
        const float s2 = f16_lo(pr) + f16_hi(pr);
        if (c & 1) sb += s2;
        else sa += s2;
      }
    }
    bad = bad && live;
    const float sa_t = quad_xor_add<1>(sa);  // same bits on both lanes of the pair
    const float sb_t = quad_xor_add<1>(sb);
    if (lane * 2 < GW * 4) {
      reinterpret_cast<uint4*>(xs)[lane * 2] = make_uint4(xh[0], xh[1], xh[2], xh[3]);
      reinterpret_cast<uint4*>(xs)[lane * 2 + 1] = make_uint4(xh[4], xh[5], xh[6], xh[7]);
      if ((lane & 1) == 0) Cs[lane >> 1] = fmaf(1032.0f, sa_t, 72.0f * sb_t);
    }
    __builtin_amdgcn_wave_barrier();  // LDS ops of one wave complete in order
  };
  const uint8_t* blob;
  if constexpr (ONEPASS) {
    stage_x();
    blob = onepass_unit_blob(a, u, has_shared, words, ep, wave);
  } else {
    blob = dec_unit_blob(a, u, has_shared, a.ids, pre);
  }
  tl_mark(tl, 3);
  const uint8_t* src = blob ? blob : a.slots;  // any readable blob; its terms get scale 0
  const BlobLayout BL = blob_layout(H, I);
  const int n = hb * 8 + r;
  if constexpr (!ONEPASS) stage_x();
  // 3. codes and scale dwords of every step, in step order
  uint4 cg[GPL], cu[GPL];
  uint32_t sgw[GPL], suw[GPL];
#pragma unroll
  for (int i = 0; i < GPL; ++i) {
    const int jl = 8 * i + p;
    int j = j0 + (jl < gw_here ? jl : gw_here - 1);
    j = j < 0 ? 0 : (j < G ? j : G - 1);
    const size_t co = code_off(n, j, G, kRowBlockGU);  // 8 rows x 8 groups: 1 KB contiguous per wave
    cg[i] = stream_u4(src + BL.gate_codes + co);
    cu[i] = stream_u4(src + BL.up_codes + co);
    const size_t sd = scale_off(n, j, G, kRowBlockGU) >> 2;  // dword holding the scale
    sgw[i] = stream_u32(src + BL.gate_scales + 4 * sd);
    suw[i] = stream_u32(src + BL.up_scales + 4 * sd);
  }
  __builtin_amdgcn_sched_barrier(0);  // every load is issued before the steps
  tl_mark(tl, 4);
  // 4. the steps, each reading its LDS operands (other waves of the SIMD cover
  //    the LDS latency: few registers live means six or more waves per SIMD)
  float ag = 0.0f, au = 0.0f;
  const int sh = (r & 1) * 16;
#pragma unroll
  for (int i = 0; i < GPL; ++i) {
    const int jl = 8 * i + p;
    const int jc = jl < gw_here ? jl : 0;
    const uint4* xq = reinterpret_cast<const uint4*>(xs + jc * 16);
    const uint4 x0 = xq[0], x1 = xq[1], x2 = xq[2], x3 = xq[3];
    const float C = Cs[jc];
    const bool ok = blob != nullptr && jl < gw_here;
    float dg = 0.0f, du = 0.0f;
    dg = code_dot(cg[i].x, x0.x, x0.y, x0.z, x0.w, dg);
    du = code_dot(cu[i].x, x0.x, x0.y, x0.z, x0.w, du);
    dg = code_dot(cg[i].y, x1.x, x1.y, x1.z, x1.w, dg);
    du = code_dot(cu[i].y, x1.x, x1.y, x1.z, x1.w, du);
    dg = code_dot(cg[i].z, x2.x, x2.y, x2.z, x2.w, dg);
    du = code_dot(cu[i].z, x2.x, x2.y, x2.z, x2.w, du);
    dg = code_dot(cg[i].w, x3.x, x3.y, x3.z, x3.w, dg);
    du = code_dot(cu[i].w, x3.x, x3.y, x3.z, x3.w, du);
    const float sg = ok ? f16_lo(sgw[i] >> sh) : 0.0f;
    const float su = ok ? f16_lo(suw[i] >> sh) : 0.0f;
    ag = fmaf(sg, dg - C, ag);
    au = fmaf(su, du - C, au);
    // step i is computed here: no later LDS read moves above it (register pressure)
    asm volatile("" : "+v"(ag), "+v"(au)::"memory");
  }
  if (bad) *a.status = MOE_EUNSUP;
  // 5. phases (lane bits 3..5), read from lanes 0..7, then the four waves in order
  ag = sum_rows(dpp_add<8>(ag));
  au = sum_rows(dpp_add<8>(au));
  if (p == 0) {
    part[0][wave][r] = ag;
    part[1][wave][r] = au;
  }
  __syncthreads();
  if (tid < 8) {
    float g = 0.0f, uu = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      g += part[0][w][tid];
      uu += part[1][w][tid];
    }
    const float hv = blob ? silu(g) * uu : 0.0f;
    if (!(fabsf(hv) < 65520.0f)) *a.status = MOE_EUNSUP;  // h does not fit fp16
    reinterpret_cast<_Float16*>(a.ws)[(size_t)unit_pair(u, K, has_shared) * I + hb * 8 + tid] = (_Float16)hv;
  }
  tl_end(tl);
}

template <int GPL>
__global__ void __launch_bounds__(kThreads) dec_gateup_kernel(FfnArgs a) {
  const TlRow tl = tl_begin(MOE_TL_DEC_GATEUP);
  dec_gateup_body<GPL, false>(a, blockIdx.x, nullptr, 0, tl);
}

// moe_layer's one-pass single-token path in one dispatch: workgroups 0 .. E-1
// compute the router logits and publish them (onepass.h); the last of them
// selects, publishes each rank's slot as soon as that rank is selected, and
// writes logits, ids, w and the resolved slots (for the down kernel); the other
// workgroups are the gate/up items, which stage x and then wait for their unit's
// slot word. The arithmetic is
// that of router_gemv1_kernel, route_select_kernel and dec_gateup_kernel, so
// the results are the same bits. Workgroups are dispatched in index order on
// each XCD and the GEMV workgroups wait for nothing, so every word that a
// waiting workgroup needs is eventually written (each wait is also bounded).
template <int GPL, int EPL>
__global__ void __launch_bounds__(kThreads) dec_route_gateup_kernel(FfnArgs a, OnepassRoute r) {
  const TlRow tl = tl_begin(MOE_TL_DEC_ROUTE_GATEUP);
  const uint32_t ep = onepass_epoch(r.words);
  const int E = a.E;
  if ((int)blockIdx.x >= E) {
    dec_gateup_body<GPL, true>(a, blockIdx.x - E, r.words, ep, tl);
    return;
  }
  __shared__ double part[4];
  const bool selector = (int)blockIdx.x == E - 1 && threadIdx.x < 64;
  // the selector's slot-table loads go out first and land while it waits
  const int lane = threadIdx.x & 63;
  int32_t tv[EPL];
  if (selector) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = lane * EPL + i;
      tv[i] = a.slot_table[e < E ? e : E - 1];
    }
  }
  onepass_publish_logit(a.x, r.w_router, a.H, blockIdx.x, r.words, ep, part);
  tl_mark(tl, 0);
  if (!selector) {
    tl_end(tl);
    return;
  }
  // wait, select and publish the slots first; the output stores come after
  float lg[EPL];
  const bool ok = onepass_wait_logits<EPL>(r.words, E, ep, a.status, lg);
  tl_mark(tl, 1);
  float sel[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) sel[i] = lg[i];
  int32_t id = 0;
  float wt = 0.0f;
  int32_t slot = (int32_t)0x80000000;  // the hand-off failed: consumers report it
  if (ok) {
    // each rank's slot is published in the round that selects it (kOnepassCopies
    // copies, lane c writes copy c), so the gate/up items of rank k start while
    // the later ranks are still being selected; the slots ride with their
    // experts through the selection (the payload)
    auto publish = [&](int k, int32_t, int32_t sk) {
      if (lane < kOnepassCopies) ll_store(r.words + onepass_slot_word(E, k, lane), ep, (uint32_t)sk);
      if (lane == k) slot = sk;
    };
    wave_select_values<EPL>(sel, tv, E, a.K, r.flags, lane, id, wt, publish);
  } else {
    for (int k = 0; k < a.K; ++k)
      if (lane < kOnepassCopies) ll_store(r.words + onepass_slot_word(E, k, lane), ep, (uint32_t)slot);
  }
  tl_mark(tl, 2);
  if (!ok) {
    tl_end(tl);
    return;
  }
  if (lane < a.K) {
    r.ids[lane] = id;
    r.w[lane] = wt;
    const_cast<int32_t*>(a.pre_slots)[lane] = slot;
  }
  onepass_store_logits<EPL>(lg, E, r.logits);
  tl_end(tl);
}

// ------------------------------------------------------------------ down + combine
// CPL = columns per lane; a wave owns CW = 16 * CPL consecutive columns.
// PRE: the K slots were resolved by the routing kernel (a.pre_slots); else they
// are looked up as slot_table[ids[k]]. Either way the slot loads go out before
// h, so that the weight loads wait for the slots only (loads complete in order:
// a slot load issued after h would also wait for h).
template <int CPL, bool PRE>
__global__ void __launch_bounds__(kThreads) dec_down_kernel(FfnArgs a) {
  const TlRow tl = tl_begin(MOE_TL_DEC_DOWN);
  // LDS per wave: h slice as fp16 pairs [CW][16] dwords + column corrections [CW]
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int kMaxUnits = kMaxK + 1;
  constexpr int CW = 16 * CPL;
  // row quads per workgroup (rows 4 qb .. 4 qb + 4 RQ - 1): two quads share the h
  // staging and the LDS reads (8.5-8.8 us against 8.9-9.1 with one; four quads
  // left too few workgroups: 9.8-10.3)
  constexpr int RQ = 2;
  __shared__ float part[kWaves][kMaxUnits][4 * RQ];
  __shared__ float wsh[kMaxK];
  // the argument pointers the first loads need, in registers with the others (one
  // batch of argument loads instead of two round trips)
  // (typed as global pointers: through the asm the compiler would otherwise lose
  // their address space and emit slower flat accesses)
  const __attribute__((address_space(1))) int32_t* ids_p = (const __attribute__((address_space(1))) int32_t*)a.ids;
  const __attribute__((address_space(1))) float* w_p = (const __attribute__((address_space(1))) float*)a.w;
  asm volatile("" : "+s"(ids_p), "+s"(w_p));
  const int H = a.H, I = a.I, K = a.K;
  const int Gd = I / kGroup;
  const bool has_shared = a.shared_blob != nullptr;
  const int n_units = K + (has_shared ? 1 : 0);
  const int C = n_units * Gd;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 3, p = lane >> 2;
  uint32_t* hs = reinterpret_cast<uint32_t*>(smem) + (size_t)wave * (CW * 17);
  float* Cc = reinterpret_cast<float*>(hs + CW * 16);
  const int c0 = wave * CW;
  const uint4* h4 = reinterpret_cast<const uint4*>(a.ws);  // h: fp16 [pair][I]
  const BlobLayout BL = blob_layout(H, I);
  const int qb = xcd_item(blockIdx.x, H / (4 * RQ)) * RQ;
  const int n = qb * 4 + r;  // quad q's row: n + 4 q
  // the slot of rank kk (lane kk + 1 with a shared expert), every lane's load
  // unconditional (a clamped rank): a load under a lane-dependent branch would be
  // waited for at the branch. PRE: one load; else the id, then its table entry.
  const int kk = lane - (has_shared ? 1 : 0);
  const int kc = kk < 0 ? 0 : (kk < K ? kk : K - 1);
  int32_t pre_v = 0, e_v = 0;
  if constexpr (PRE) {
    pre_v = a.pre_slots[kc];
  } else {
    e_v = ids_p[kc];
  }
  // the routing weights, loaded early and kept in LDS for the combine
  const float wk = (wave == 0 && lane < K) ? w_p[lane] : 0.0f;
  if constexpr (!PRE) pre_v = a.slot_table[e_v >= 0 && e_v < a.E ? e_v : 0];
  // the status pointer in registers now, with the other arguments (left to the
  // compiler, its load lands after the slot lookup, one more round trip on the
  // path to the weight loads)
  __attribute__((address_space(1))) int32_t* status = (__attribute__((address_space(1))) int32_t*)a.status;
  asm volatile("" : "+s"(status));
  // 1. this wave's h slice: uint4 q = lane + 64m = column c0 + q/4, halves 8*(q%4) .. +7;
  //    (unit, group) of the lane's column advance by 16 columns per m. Issued before
  //    the slot lookup below: it does not depend on the unit slots.
  uint4 hv[CPL];
  {
    int cu = c0 + lane / 4;
    cu = cu < C ? cu : C - 1;
    int hu = cu / Gd, hj = cu % Gd;
#pragma unroll
    for (int m = 0; m < CPL; ++m) {
      const int uu = hu < n_units ? hu : n_units - 1;
      const int jj = hu < n_units ? hj : Gd - 1;
      hv[m] = h4[((size_t)unit_pair(uu, K, has_shared) * I + jj * kGroup) / 8 + lane % 4];
      hj += 16;  // Gd is a multiple of 16: at most one wrap
      const int w1 = hj >= Gd;
      hj -= w1 ? Gd : 0;
      hu += w1;
    }
  }
  // unit slots (loaded above): lane u of every wave holds unit u's slot, -1 when
  // it cannot be used (the status word says why); the shared expert (unit 0 when
  // present) is marked 0 and read from shared_blob
  int my_slot = -1;
  if (lane < n_units) {
    const int k = has_shared ? lane - 1 : lane;
    if (k < 0) {
      my_slot = 0;
    } else {
      if (!PRE && (e_v < 0 || e_v >= a.E)) {
        *status = MOE_EINVAL;
      } else {
        my_slot = pre_v;
        if (my_slot < 0) *status = MOE_ENOTRES;
      }
    }
  }
  // this wave's entries of the partial sums start at zero (only this wave writes them)
  for (int q = lane; q < kMaxUnits * 4 * RQ; q += 64) (&part[wave][0][0])[q] = 0.0f;
  // 2. codes and scale dwords of every step; a step is one unit for all lanes
  bool uok[CPL];
  int ustep[CPL];  // unit of step i (>= n_units past the last column)
  uint4 cd[RQ][CPL];
  uint32_t sdw[RQ][CPL];
  {
    int us = c0 / Gd, js = c0 % Gd;  // unit and group of the step's first column (wave-uniform)
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      ustep[i] = us;
      const int uc = us < n_units ? us : n_units - 1;
      const int jc = us < n_units ? js : Gd - 16;
      const int sl = __builtin_amdgcn_readlane(my_slot, uc);
      uok[i] = sl >= 0;
      const uint8_t* src = (has_shared && uc == 0) ? a.shared_blob : a.slots + (size_t)(sl > 0 ? sl : 0) * a.stride;
      const int j = jc + p;
      // 4 rows x 16 groups: 1 KB of contiguous codes per wave
#pragma unroll
      for (int q = 0; q < RQ; ++q) {
        cd[q][i] = stream_u4(src + BL.down_codes + code_off(n + 4 * q, j, Gd, kRowBlockDN));
        sdw[q][i] = stream_u32(src + BL.down_scales + (scale_off(n + 4 * q, j, Gd, kRowBlockDN) & ~(size_t)3));
      }
      js += 16;
      if (js >= Gd) {
        js -= Gd;
        ++us;
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // every load is issued before h is used
  tl_mark(tl, 0);
  if (wave == 0 && lane < K) wsh[lane] = wk;
  // 3. h slice into LDS with its column corrections (lanes 4t .. 4t+3 hold one column)
#pragma unroll
  for (int m = 0; m < CPL; ++m) {
    const int q = lane + 64 * m;
    const bool live = c0 + q / 4 < C;
    const uint32_t d[4] = {live ? hv[m].x : 0u, live ? hv[m].y : 0u, live ? hv[m].z : 0u, live ? hv[m].w : 0u};
    float sa = (f16_lo(d[0]) + f16_hi(d[0])) + (f16_lo(d[2]) + f16_hi(d[2]));
    float sb = (f16_lo(d[1]) + f16_hi(d[1])) + (f16_lo(d[3]) + f16_hi(d[3]));
    sa = quad_xor_add<2>(quad_xor_add<1>(sa));  // same bits on the column's four lanes
    sb = quad_xor_add<2>(quad_xor_add<1>(sb));
    reinterpret_cast<uint4*>(hs)[q] = make_uint4(d[0], d[1], d[2], d[3]);
    if ((lane & 3) == 0) Cc[q / 4] = fmaf(1032.0f, sa, 72.0f * sb);
  }
  __builtin_amdgcn_wave_barrier();
  tl_mark(tl, 1);
  // 4. the steps; the LDS operands of step i+1 are read during step i
  const int sh = (r & 1) * 16;
  float acc[RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q) acc[q] = 0.0f;
  int cur = -1;
  uint4 hn[4];
  float Cn;
  {
    const uint4* hq = reinterpret_cast<const uint4*>(hs + p * 16);
    hn[0] = hq[0], hn[1] = hq[1], hn[2] = hq[2], hn[3] = hq[3];
    Cn = Cc[p];
  }
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int cs = c0 + 16 * i;
    const uint4 h0 = hn[0], h1 = hn[1], h2 = hn[2], h3 = hn[3];
    const float Ccol = Cn;
    if (i + 1 < CPL) {
      const uint4* hq = reinterpret_cast<const uint4*>(hs + (16 * (i + 1) + p) * 16);
      hn[0] = hq[0], hn[1] = hq[1], hn[2] = hq[2], hn[3] = hq[3];
      Cn = Cc[16 * (i + 1) + p];
    }
    if (cs < C) {  // uniform across the wave
      const int us = ustep[i];
      if (us != cur) {
        if (cur >= 0) {
#pragma unroll
          for (int q = 0; q < RQ; ++q) {
            const float t = sum_rows(dpp_add<8>(dpp_add<4>(acc[q])));  // phases (lane bits 2..5), read from lanes 0..3
            if (p == 0) part[wave][cur][4 * q + r] = t;
          }
        }
#pragma unroll
        for (int q = 0; q < RQ; ++q) acc[q] = 0.0f;
        cur = us;
      }
#pragma unroll
      for (int q = 0; q < RQ; ++q) {
        float P = 0.0f;
        P = code_dot(cd[q][i].x, h0.x, h0.y, h0.z, h0.w, P);
        P = code_dot(cd[q][i].y, h1.x, h1.y, h1.z, h1.w, P);
        P = code_dot(cd[q][i].z, h2.x, h2.y, h2.z, h2.w, P);
        P = code_dot(cd[q][i].w, h3.x, h3.y, h3.z, h3.w, P);
        const float s = uok[i] ? f16_lo(sdw[q][i] >> sh) : 0.0f;
        acc[q] = fmaf(s, P - Ccol, acc[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < RQ; ++q) asm volatile("" : "+v"(acc[q])::"memory");  // as in dec_gateup: one step of operands ahead
  }
  if (cur >= 0) {
#pragma unroll
    for (int q = 0; q < RQ; ++q) {
      const float t = sum_rows(dpp_add<8>(dpp_add<4>(acc[q])));
      if (p == 0) part[wave][cur][4 * q + r] = t;
    }
  }
  tl_mark(tl, 2);
  __syncthreads();
  if (tid < 4 * RQ) {
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
      y = fmaf(wsh[k], o, y);
    }
    a.y[(size_t)qb * 4 + tid] = __builtin_bit_cast(uint16_t, (__bf16)y);  // row 4 qb + tid
  }
  // after a one-pass dispatch: every workgroup of it has read the region's call
  // number (that dispatch has completed), so the call is numbered done here (at the
  // end: its load would otherwise be waited for with this wave's h and code loads)
  if (a.onepass && blockIdx.x == 0 && tid == 0)
    __hip_atomic_store(a.onepass, (uint64_t)onepass_epoch(a.onepass), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  tl_end(tl);
}

inline void set_lds_limit(const void* fn, size_t lds) {
  if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

inline int dec_down_cpl(int n_units, int Gd) {
  const int C = n_units * Gd;
  const int per_wave = (C + kWaves - 1) / kWaves;
  return (per_wave + 15) / 16;
}

inline int round_cpl(int cpl) { return cpl <= 2 ? 2 : cpl <= 4 ? 4 : cpl <= 6 ? 6 : 8; }

}  // namespace

bool decode1_supported(int T, int H, int I, int K, bool has_shared) {
  const int n_units = K + (has_shared ? 1 : 0);
  const int G = H / kGroup, Gd = I / kGroup;
  // gate/up: at most 4 groups per lane; down: whole steps of 16 columns per unit, at most 8 per lane
  return T == 1 && G <= 4 * 8 * 4 && Gd % 16 == 0 && H % 8 == 0 && dec_down_cpl(n_units, Gd) <= 8;
}

hipError_t launch_ffn_decode1_onepass(const FfnArgs& a, const OnepassRoute& r, hipStream_t s) {
  const bool has_shared = a.shared_blob != nullptr;
  const int n_units = a.K + (has_shared ? 1 : 0);
  const int G = a.H / kGroup;
  const int GW = (G + kWaves - 1) / kWaves;
  const int gpl = (GW + 7) / 8;
  const int epl = (a.E + 63) / 64;
  const size_t lds = (size_t)kWaves * GW * 17 * 4;
  const int grid = a.E + n_units * (a.I / 8);
#define RG(N, M)                                                                                    \
  do {                                                                                              \
    set_lds_limit(reinterpret_cast<const void*>(&dec_route_gateup_kernel<N, M>), lds);              \
    hipLaunchKernelGGL((dec_route_gateup_kernel<N, M>), dim3(grid), dim3(kThreads), lds, s, a, r);  \
  } while (0)
#define RGE(N)               \
  do {                       \
    if (epl <= 1) RG(N, 1);  \
    else if (epl <= 2) RG(N, 2); \
    else if (epl <= 4) RG(N, 4); \
    else if (epl <= 8) RG(N, 8); \
    else RG(N, 16);          \
  } while (0)
  if (gpl <= 1) RGE(1);
  else if (gpl <= 2) RGE(2);
  else RGE(4);
#undef RGE
#undef RG
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  FfnArgs d = a;
  d.onepass = r.words;
  return launch_ffn_decode1(d, 1, s);
}

hipError_t launch_ffn_decode1(const FfnArgs& a, int stage, hipStream_t s) {
  const bool has_shared = a.shared_blob != nullptr;
  const int n_units = a.K + (has_shared ? 1 : 0);
  if (stage == 0) {
    const int G = a.H / kGroup;
    const int GW = (G + kWaves - 1) / kWaves;
    const int gpl = (GW + 7) / 8;
    const size_t lds = (size_t)kWaves * GW * 17 * 4;
    const int grid = n_units * (a.I / 8);
#define GU(N)                                                                                       \
  do {                                                                                              \
    set_lds_limit(reinterpret_cast<const void*>(&dec_gateup_kernel<N>), lds);                       \
    hipLaunchKernelGGL((dec_gateup_kernel<N>), dim3(grid), dim3(kThreads), lds, s, a);              \
  } while (0)
    if (gpl <= 1) GU(1);
    else if (gpl <= 2) GU(2);
    else GU(4);
#undef GU
    return hipGetLastError();
  }
  {
    const int Gd = a.I / kGroup;
    const int cpl = round_cpl(dec_down_cpl(n_units, Gd));
    const size_t lds = (size_t)kWaves * 16 * cpl * 17 * 4;
    const int grid = a.H / 8;  // 8 rows of H per workgroup
#define DN(N)                                                                                       \
  do {                                                                                              \
    if (a.pre_slots) {                                                                              \
      set_lds_limit(reinterpret_cast<const void*>(&dec_down_kernel<N, true>), lds);                 \
      hipLaunchKernelGGL((dec_down_kernel<N, true>), dim3(grid), dim3(kThreads), lds, s, a);        \
    } else {                                                                                        \
      set_lds_limit(reinterpret_cast<const void*>(&dec_down_kernel<N, false>), lds);                \
      hipLaunchKernelGGL((dec_down_kernel<N, false>), dim3(grid), dim3(kThreads), lds, s, a);       \
    }                                                                                               \
  } while (0)
    if (cpl == 2) DN(2);
    else if (cpl == 4) DN(4);
    else if (cpl == 6) DN(6);
    else DN(8);
#undef DN
    return hipGetLastError();
  }
}

}  // namespace moe
