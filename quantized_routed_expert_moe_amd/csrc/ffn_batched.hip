// Small-batch expert FFN (2 <= T <= 32 tokens): the decode kernels' design
// for several tokens per expert.
//
// A unit is one distinct expert of the batch (or the always-on shared expert)
// with every (token, rank) pair routed to it, so each expert's bytes stream
// from HBM once however many tokens use it ("Strata" README, Models: W4A16
// experts). Four kernels:
//   bat_plan     one workgroup: units in order of their first pair (the shared
//                expert first), each unit's pairs in pair order, and per unit
//                one record (slot, first pair, pair count) into the workspace;
//                also x as fp16 pairs with its per-group corrections, once.
//                Pair p = t*K + k for routed pairs, T*K + t for the shared
//                expert's.
//   bat_gateup   one workgroup per (unit, 8 rows of I), as dec_gateup: one
//                record load, then the weights of the item into registers,
//                then the unit's tokens 4 at a time; each chunk copies its
//                tokens' fp16 x slices and corrections into the wave's LDS,
//                and the fp16 pairs of the codes are formed once per step for
//                all tokens of the chunk. h = silu(g) * u in fp16 per pair.
//   bat_down     one workgroup per (unit, 16 rows of H); each wave owns 4 rows
//                (one 4-row block of the blob) and all groups of the unit, so
//                no wave waits for another; per chunk of 4 pairs the wave
//                stages their h rows and writes o[pair] (fp32) for its rows.
//   bat_combine  y[t] = o_shared[t] + sum_k w[t][k] * o[t*K + k] in rank order,
//                rounded once to bf16.
// Arithmetic as in the single-token kernels: codes become exact fp16 pairs
// (q + 1032, q + 72) for v_dot2_f32_f16 against fp16 activations, one
// correction per group, the fp16 scale applied per group in fp32. No atomics
// on floating-point values; every sum has a fixed order.
#include "moe_internal.h"
#include "wave_ops.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kTB = 4;                 // pairs per gate/up chunk
constexpr int kTBD = 8;                // pairs per down chunk
constexpr int kUnitPairs = 64;         // pairs one unit can hold (a routed unit has at most T)
constexpr int kPlanThreads = 1024;
constexpr int kBatMaxPairs = 512;      // routed pairs T*K the plan covers

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

__host__ __device__ inline int bat_umax(int T, int K, int E, int has_shared) {
  return (T * K < E ? T * K : E) + (has_shared ? 1 : 0);
}
__host__ __device__ inline int bat_pmax(int T, int K, int has_shared) { return T * K + (has_shared ? T : 0); }

// Workspace: plan ints [n_units | rec[U][4] | ptab[U][kUnitPairs]], x16 fp16
// [T][H], xc fp32 [T][G] (per-group corrections of x16), h fp16 [P][I] with
// rows in unit order (row rec[u].y + i is pair ptab[u][i]), o fp32 [P][H] with
// rows in pair order. rec[u] = {slot (-1: the shared expert, -2: not usable),
// first h row of the unit, pair count (0 past the last unit), expert}; the
// pair table has a fixed stride, so a workgroup loads its unit's record and
// pairs in one round trip.
struct BatWs {
  size_t x16_off, xc_off, h_off, o_off, bytes;
  int U, P;
};
__host__ __device__ inline BatWs bat_ws(int T, int H, int I, int E, int K, int has_shared) {
  BatWs w;
  w.U = bat_umax(T, K, E, has_shared);
  w.P = bat_pmax(T, K, has_shared);
  const size_t plan_ints = 4 + (size_t)w.U * (4 + kUnitPairs);
  w.x16_off = align256(plan_ints * 4);
  w.xc_off = align256(w.x16_off + (size_t)T * H * 2);
  w.h_off = align256(w.xc_off + (size_t)T * (H / kGroup) * 4);
  w.o_off = align256(w.h_off + (size_t)w.P * I * 2);
  w.bytes = align256(w.o_off + (size_t)w.P * H * 4);
  return w;
}

struct PlanView {
  int* n_units;
  int4* rec;
  int* ptab;
};
__device__ inline PlanView plan_view(uint8_t* ws, int U, int P) {
  int* p = reinterpret_cast<int*>(ws);
  PlanView v;
  v.n_units = p;
  v.rec = reinterpret_cast<int4*>(p + 4);  // 16-byte aligned
  v.ptab = p + 4 + 4 * U;
  return v;
}

__device__ inline const uint8_t* rec_blob(const FfnArgs& a, int slot) {
  return slot >= 0 ? a.slots + (size_t)slot * a.stride : (slot == -1 ? a.shared_blob : nullptr);
}

__device__ inline int pair_token(int p, int T, int K) { return p < T * K ? p / K : p - T * K; }

// Exclusive prefix sum of one int per thread over the block (blockDim.x =
// kPlanThreads), in thread order; *total gets the sum. All threads call it.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  constexpr int nw = kPlanThreads / 64;
  // inclusive scan inside the wave (Hillis-Steele through LDS-free shuffles)
  int s = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(s, off, 64);
    if (lane >= off) s += o;
  }
  if (lane == 63) wsum[wave] = s;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < nw; ++w) {
    before += w < wave ? wsum[w] : 0;
    all += wsum[w];
  }
  __syncthreads();
  *total = all;
  return before + s - v;
}

// x as fp16 pairs (x16) and the per-group corrections xc = 1032 * A + 72 * B,
// where A sums columns 8d + {0,1,4,5} and B columns 8d + {2,3,6,7} of the
// group: thread i converts dword i of x; the 16 dwords of a group are one row
// of 16 lanes, whose sums are taken with DPP rotations (lane 0 of the row writes).
__device__ inline void plan_convert_x(const FfnArgs& a, const BatWs& W, int i) {
  const int n_dw = a.T * a.H / 2;
  const bool live = i < n_dw;
  const uint32_t v = live ? reinterpret_cast<const uint32_t*>(a.x)[i] : 0u;
  bool bad = false;
  const uint32_t lo = to_f16_bits(__uint_as_float(v << 16), &bad);
  const uint32_t hi = to_f16_bits(__uint_as_float(v & 0xFFFF0000u), &bad);
  const uint32_t pr = lo | (hi << 16);
  if (live) reinterpret_cast<uint32_t*>(a.ws + W.x16_off)[i] = pr;
  if (bad && live) *a.status = MOE_EUNSUP;
  const float s2 = f16_lo(pr) + f16_hi(pr);
  float sa = (i & 1) ? 0.0f : s2;  // dword 2k of a group: columns of A pairs
  float sb = (i & 1) ? s2 : 0.0f;
  sa = dpp_add<8>(dpp_add<4>(dpp_add<2>(dpp_add<1>(sa))));
  sb = dpp_add<8>(dpp_add<4>(dpp_add<2>(dpp_add<1>(sb))));
  if (live && (i & 15) == 0) reinterpret_cast<float*>(a.ws + W.xc_off)[i >> 4] = fmaf(1032.0f, sa, 72.0f * sb);
}

// ------------------------------------------------------------------ plan
__global__ void __launch_bounds__(kPlanThreads) bat_plan_kernel(FfnArgs a) {
  __shared__ int first[kMaxE];  // lowest pair using expert e, then the unit of expert e
  __shared__ int cnt[kBatMaxPairs + 1];
  __shared__ int uoff[kBatMaxPairs + 1];
  __shared__ int unit_expert_lds[kBatMaxPairs + 1];
  __shared__ int wsum[kPlanThreads / 64];
  const int T = a.T, K = a.K, E = a.E;
  const int P = T * K;
  const bool has_shared = a.shared_blob != nullptr;
  const int base = has_shared ? 1 : 0;
  const BatWs W = bat_ws(T, a.H, a.I, E, K, has_shared);
  const PlanView pl = plan_view(a.ws, W.U, W.P);
  const int tid = threadIdx.x;
  if (blockIdx.x > 0) {
    plan_convert_x(a, W, (blockIdx.x - 1) * kPlanThreads + tid);
    return;
  }
  for (int e = tid; e < E; e += kPlanThreads) first[e] = 0x7FFFFFFF;
  for (int u = tid; u <= kBatMaxPairs; u += kPlanThreads) cnt[u] = 0;
  __syncthreads();
  const int p = tid;  // P <= kBatMaxPairs < kPlanThreads: one pair per thread
  const int e = p < P ? a.ids[p] : -1;
  const bool valid = p < P && e >= 0 && e < E;
  if (p < P && !valid) *a.status = MOE_EINVAL;
  if (valid) atomicMin(&first[e], p);
  __syncthreads();
  // leaders (the first pair of each expert) become the routed units, in pair order
  const bool leader = valid && first[e] == p;
  int n_routed;
  const int lead_idx = block_exclusive_scan(leader ? 1 : 0, wsum, &n_routed);
  __syncthreads();  // every read of first[] as "lowest pair" is done
  if (leader) {
    first[e] = base + lead_idx;
    unit_expert_lds[base + lead_idx] = e;
  }
  __syncthreads();
  const int up = valid ? first[e] : -1;
  // the pair's place in its unit: any order serves, as every pair's arithmetic
  // is its own and its output row is its pair index
  const int rank = valid ? atomicAdd(&cnt[up], 1) : 0;
  if (valid) {
    if (rank < kUnitPairs) pl.ptab[up * kUnitPairs + rank] = p;
    else *a.status = MOE_EUNSUP;  // only with an expert repeated within a token's ids
  }
  __syncthreads();
  // unit offsets: the shared unit holds T pairs, routed units their counts
  const int n_units = base + n_routed;
  const int c = tid < n_units ? (has_shared && tid == 0 ? T : cnt[tid]) : 0;
  int total;
  const int off = block_exclusive_scan(c, wsum, &total);
  if (tid < n_units) uoff[tid] = off;
  __syncthreads();
  if (has_shared && tid < T) pl.ptab[tid] = T * K + tid;
  // unit records: the slot is resolved here once for every workgroup of the layer
  if (tid == 0) *pl.n_units = n_units;
  for (int u = tid; u < W.U; u += kPlanThreads) {
    int4 rc = make_int4(-2, 0, 0, -1);
    if (u < n_units) {
      const int ex = (has_shared && u == 0) ? -1 : unit_expert_lds[u];
      rc.y = uoff[u];
      rc.z = (has_shared && u == 0) ? T : cnt[u];
      rc.w = ex;
      if (ex == -1) {
        rc.x = -1;
      } else {
        const int slot = a.slot_table[ex];
        if (slot < 0) *a.status = MOE_ENOTRES;
        rc.x = slot < 0 ? -2 : slot;
      }
    }
    pl.rec[u] = rc;
  }
}

// ------------------------------------------------------------------ unit header
// The record of unit u and, in lane i, its pair i (lanes past the count: 0).
// One round trip; a workgroup of a unit past the plan's last leaves at once.
struct UnitHead {
  int slot, p0, np, my_pair;
};
__device__ inline UnitHead unit_head(const PlanView& pl, int u, int lane) {
  const int4 rc = pl.rec[u];
  const int pv = pl.ptab[u * kUnitPairs + lane];
  UnitHead h;
  h.slot = rc.x;
  h.p0 = rc.y;
  h.np = rc.z;
  h.my_pair = lane < rc.z ? pv : 0;
  return h;
}

// ------------------------------------------------------------------ gate/up
// GPL = groups per lane = ceil(GW / 8) with GW = ceil(G / 4) groups per wave.
template <int GPL>
__global__ void __launch_bounds__(kThreads) bat_gateup_kernel(FfnArgs a) {
  // LDS per wave: for each of the chunk's tokens, the x slice as fp16 pairs
  // [GW][16] dwords and the group corrections [GW]
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float part[kTB][2][kWaves][8];
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const int G = H / kGroup;
  const int GW = (G + kWaves - 1) / kWaves;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 7, p = lane >> 3;
  const bool has_shared = a.shared_blob != nullptr;
  const BatWs W = bat_ws(T, H, I, a.E, K, has_shared);
  const PlanView pl = plan_view(a.ws, W.U, W.P);
  // one item per workgroup; a unit's items are consecutive workgroups, so its rows
  // stream from HBM together
  const int n_hb = I / 8;
  const int u = blockIdx.x / n_hb, hb = blockIdx.x % n_hb;
  const UnitHead uh = unit_head(pl, u, lane);
  const int p0 = uh.p0, np = uh.np;
  if (np == 0) return;
  if (np > kUnitPairs) {
    if (tid == 0) *a.status = MOE_EUNSUP;
    return;
  }
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem) + (size_t)wave * kTB * (GW * 17);
  const int j0 = wave * GW;
  const int gw_here = G - j0 < GW ? (G - j0 > 0 ? G - j0 : 0) : GW;
  const uint8_t* blob = rec_blob(a, uh.slot);
  const uint8_t* src = blob ? blob : a.slots;  // any readable blob; its terms get scale 0
  const uint4* x16 = reinterpret_cast<const uint4*>(a.ws + W.x16_off);
  const float* xc = reinterpret_cast<const float*>(a.ws + W.xc_off);
  // a chunk's x slices: uint4 v of a token's slice is columns 8 (lane + 64 v) .. +7
  // of the wave's groups; every token's loads are issued before any is stored
  constexpr int XQ = (GPL + 1) / 2;  // uint4 per lane and token (GW <= 8 * GPL groups)
  uint4 xv[kTB][XQ];
  float cv[kTB];
  auto load_x = [&](int c0) {
    const int tc = np - c0 < kTB ? np - c0 : kTB;
#pragma unroll
    for (int ti = 0; ti < kTB; ++ti) {
      const int t = pair_token(__builtin_amdgcn_readlane(uh.my_pair, c0 + (ti < tc ? ti : tc - 1)), T, K);
#pragma unroll
      for (int v = 0; v < XQ; ++v) {
        int q = j0 * 4 + lane + 64 * v;
        q = q < G * 4 ? q : G * 4 - 1;
        xv[ti][v] = x16[(size_t)t * (H / 8) + q];
      }
      int jj = j0 + (lane < GW ? lane : 0);
      jj = jj < G ? jj : G - 1;
      cv[ti] = xc[(size_t)t * G + jj];
    }
  };
  // ... into the wave's LDS (zeros past the wave's groups); the values are selected
  // on every lane, outside the stores' branches, so each load is waited for on every path
  auto stage_x = [&](int tc) {
#pragma unroll
    for (int ti = 0; ti < kTB; ++ti) {
      uint32_t* xt = xs + (size_t)ti * (GW * 17);
#pragma unroll
      for (int v = 0; v < XQ; ++v) {
        const int q = lane + 64 * v;
        const bool keep = q < gw_here * 4;
        const uint4 val = make_uint4(keep ? xv[ti][v].x : 0u, keep ? xv[ti][v].y : 0u, keep ? xv[ti][v].z : 0u,
                                     keep ? xv[ti][v].w : 0u);
        if (ti < tc && q < GW * 4) reinterpret_cast<uint4*>(xt)[q] = val;
      }
      const float cval = lane < gw_here ? cv[ti] : 0.0f;
      if (ti < tc && lane < GW) reinterpret_cast<float*>(xt + GW * 16)[lane] = cval;
    }
    __builtin_amdgcn_wave_barrier();
  };
  const BlobLayout BL = blob_layout(H, I);
  const int n = hb * 8 + r;
  uint4 cg[GPL], cu[GPL];
  uint32_t sgw[GPL], suw[GPL];
#pragma unroll
  for (int i = 0; i < GPL; ++i) {
    const int jl = 8 * i + p;
    int j = j0 + (jl < gw_here ? jl : gw_here - 1);
    j = j < 0 ? 0 : (j < G ? j : G - 1);
    const size_t co = code_off(n, j, G, kRowBlockGU);
    cg[i] = *reinterpret_cast<const uint4*>(src + BL.gate_codes + co);
    cu[i] = *reinterpret_cast<const uint4*>(src + BL.up_codes + co);
    const size_t sd = scale_off(n, j, G, kRowBlockGU) >> 2;
    sgw[i] = reinterpret_cast<const uint32_t*>(src + BL.gate_scales)[sd];
    suw[i] = reinterpret_cast<const uint32_t*>(src + BL.up_scales)[sd];
  }
  load_x(0);  // after the weights: these need the pair table, the weights only the record
  __builtin_amdgcn_sched_barrier(0);
  _Float16* hws = reinterpret_cast<_Float16*>(a.ws + W.h_off);
  const int sh = (r & 1) * 16;
  stage_x(np < kTB ? np : kTB);
  for (int c0 = 0;;) {
    const int tc = np - c0 < kTB ? np - c0 : kTB;
    float ag[kTB], au[kTB];
#pragma unroll
    for (int ti = 0; ti < kTB; ++ti) ag[ti] = au[ti] = 0.0f;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int jl = 8 * i + p;
      const bool ok = blob != nullptr && jl < gw_here;
      const int jc = jl < gw_here ? jl : 0;
      // the weights are opaque per chunk: nothing is hoisted to before the loop,
      // where it would wait for them ahead of the staging
      asm volatile("" : "+v"(cg[i].x), "+v"(cg[i].y), "+v"(cg[i].z), "+v"(cg[i].w), "+v"(sgw[i]));
      asm volatile("" : "+v"(cu[i].x), "+v"(cu[i].y), "+v"(cu[i].z), "+v"(cu[i].w), "+v"(suw[i]));
      const float sg = ok ? f16_lo(sgw[i] >> sh) : 0.0f;
      const float su = ok ? f16_lo(suw[i] >> sh) : 0.0f;
      // a code dword at a time: its four fp16 pairs of gate and of up, then every
      // token of the chunk against the activation dwords of the same 8 columns (each
      // token's sum still runs over the chunk's 16 dwords in order)
      const uint32_t wg[4] = {cg[i].x, cg[i].y, cg[i].z, cg[i].w};
      const uint32_t wu[4] = {cu[i].x, cu[i].y, cu[i].z, cu[i].w};
      float dg[kTB], du[kTB];
#pragma unroll
      for (int ti = 0; ti < kTB; ++ti) dg[ti] = du[ti] = 0.0f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t g8 = wg[d] >> 8, u8 = wu[d] >> 8;
        const uint32_t pg0 = (wg[d] & 0x000F000Fu) | 0x64006400u, pg1 = (wg[d] & 0x00F000F0u) | 0x54005400u;
        const uint32_t pg2 = (g8 & 0x000F000Fu) | 0x64006400u, pg3 = (g8 & 0x00F000F0u) | 0x54005400u;
        const uint32_t pu0 = (wu[d] & 0x000F000Fu) | 0x64006400u, pu1 = (wu[d] & 0x00F000F0u) | 0x54005400u;
        const uint32_t pu2 = (u8 & 0x000F000Fu) | 0x64006400u, pu3 = (u8 & 0x00F000F0u) | 0x54005400u;
#pragma unroll
        for (int ti = 0; ti < kTB; ++ti) {
          if (ti < tc) {
            const uint4 xq = reinterpret_cast<const uint4*>(xs + (size_t)ti * (GW * 17) + jc * 16)[d];
            dg[ti] = dot2h(pg3, xq.w, dot2h(pg2, xq.z, dot2h(pg1, xq.y, dot2h(pg0, xq.x, dg[ti]))));
            du[ti] = dot2h(pu3, xq.w, dot2h(pu2, xq.z, dot2h(pu1, xq.y, dot2h(pu0, xq.x, du[ti]))));
          }
        }
      }
#pragma unroll
      for (int ti = 0; ti < kTB; ++ti) {
        if (ti < tc) {
          const float C = reinterpret_cast<const float*>(xs + (size_t)ti * (GW * 17) + GW * 16)[jc];
          ag[ti] = fmaf(sg, dg[ti] - C, ag[ti]);
          au[ti] = fmaf(su, du[ti] - C, au[ti]);
        }
      }
    }
    // phases (lane bits 3..5), read from lanes 0..7
#pragma unroll
    for (int ti = 0; ti < kTB; ++ti) {
      const float g = sum_rows(dpp_add<8>(ag[ti]));
      const float uu = sum_rows(dpp_add<8>(au[ti]));
      if (p == 0) {
        part[ti][0][wave][r] = g;
        part[ti][1][wave][r] = uu;
      }
    }
    // the waves in order; pair of the token: thread tid < 8 * tc
    __syncthreads();
    if (tid < 8 * tc) {
      const int ti = tid >> 3, rr = tid & 7;
      float g = 0.0f, uu = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        g += part[ti][0][w][rr];
        uu += part[ti][1][w][rr];
      }
      const float hv = blob ? silu(g) * uu : 0.0f;
      if (!(fabsf(hv) < 65520.0f)) *a.status = MOE_EUNSUP;
      hws[(size_t)(p0 + c0 + ti) * I + hb * 8 + rr] = (_Float16)hv;
    }
    c0 += kTB;
    if (c0 >= np) break;
    __syncthreads();  // part[] is read before the next chunk writes it
    load_x(c0);
    stage_x(np - c0 < kTB ? np - c0 : kTB);
  }
}

// ------------------------------------------------------------------ down
// One workgroup per (unit, 64 rows of H); wave w owns rows 16w .. 16w+15 of the
// item, as four 4-row blocks of the blob. SPL = steps per lane = ceil(Gd / 16):
// at step i lane (row r of 4, phase p of 16) takes group 16i + p of its row in
// each block. The workgroup stages the h rows of kTBD pairs at a time into LDS,
// all of a chunk's loads issued together; the first chunk's before the weights.
constexpr int kDnRowsPerItem = 64;
constexpr int kDnBlocks = 4;  // 4-row blocks per wave

template <int SPL>
__global__ void __launch_bounds__(kThreads) bat_down_kernel(FfnArgs a) {
  // LDS: for each of the chunk's pairs, the h row as fp16 pairs [Gd][16] dwords
  // and the group corrections [Gd]
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const int Gd = I / kGroup;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 3, p = lane >> 2;
  const bool has_shared = a.shared_blob != nullptr;
  const BatWs W = bat_ws(T, H, I, a.E, K, has_shared);
  const PlanView pl = plan_view(a.ws, W.U, W.P);
  const int n_rb = H / kDnRowsPerItem;
  const int u = blockIdx.x / n_rb, rb = blockIdx.x % n_rb;
  const UnitHead uh = unit_head(pl, u, lane);
  const int p0 = uh.p0, np = uh.np;
  if (np == 0) return;
  if (np > kUnitPairs) {
    if (tid == 0) *a.status = MOE_EUNSUP;
    return;
  }
  uint32_t* hsl = reinterpret_cast<uint32_t*>(smem);
  const int per_pair = Gd * 4;  // uint4 of one h row
  // uint4 q of a chunk (thread tid holds q = tid + kThreads v) is pair q / per_pair,
  // group (q / 4) % Gd, columns 8 (q % 4) .. +7: the four lanes of a group are a quad
  constexpr int HQ = kTBD * SPL * 64 / kThreads;  // kTBD * Gd * 4 <= kThreads * HQ
  const uint4* h4 = reinterpret_cast<const uint4*>(a.ws + W.h_off);
  uint4 hv[HQ];
  auto load_h = [&](int c0) {
    const int tc = np - c0 < kTBD ? np - c0 : kTBD;
#pragma unroll
    for (int v = 0; v < HQ; ++v) {
      const int q = tid + kThreads * v;
      const int ti = q / per_pair;
      const bool live = ti < tc;
      const int row = p0 + c0 + (live ? ti : 0);
      const int rem = live ? q - ti * per_pair : 0;
      hv[v] = h4[(size_t)row * (I / 8) + rem];  // past the chunk: a row of it, never stored
    }
  };
  load_h(0);  // before the weights: staging waits for these only
  const uint8_t* blob = rec_blob(a, uh.slot);
  const uint8_t* src = blob ? blob : a.slots;
  const BlobLayout BL = blob_layout(H, I);
  const int n0 = rb * kDnRowsPerItem + wave * 16 + r;  // row of block b: n0 + 4b
  uint4 cd[kDnBlocks][SPL];
  uint32_t sdw[kDnBlocks][SPL];
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
#pragma unroll
    for (int b = 0; b < kDnBlocks; ++b) {
      int j = 16 * i + p;
      j = j < Gd ? j : Gd - 1;
      const int n = n0 + 4 * b;
      cd[b][i] = *reinterpret_cast<const uint4*>(src + BL.down_codes + code_off(n, j, Gd, kRowBlockDN));
      sdw[b][i] = reinterpret_cast<const uint32_t*>(src + BL.down_scales)[scale_off(n, j, Gd, kRowBlockDN) >> 2];
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  float* ows = reinterpret_cast<float*>(a.ws + W.o_off);
  const int sh = (r & 1) * 16;
  // a chunk's h rows and their group corrections into LDS
  auto stage_h = [&](int tc) {
#pragma unroll
    for (int v = 0; v < HQ; ++v) {
      const int q = tid + kThreads * v;
      const int ti = q / per_pair;
      const int rem = q - ti * per_pair;
      const uint32_t d[4] = {hv[v].x, hv[v].y, hv[v].z, hv[v].w};
      float sa = (f16_lo(d[0]) + f16_hi(d[0])) + (f16_lo(d[2]) + f16_hi(d[2]));
      float sb = (f16_lo(d[1]) + f16_hi(d[1])) + (f16_lo(d[3]) + f16_hi(d[3]));
      sa = quad_xor_add<2>(quad_xor_add<1>(sa));
      sb = quad_xor_add<2>(quad_xor_add<1>(sb));
      if (ti < tc) {
        uint32_t* ht = hsl + (size_t)ti * (Gd * 17);
        reinterpret_cast<uint4*>(ht)[rem] = hv[v];
        if ((lane & 3) == 0) reinterpret_cast<float*>(ht + Gd * 16)[rem >> 2] = fmaf(1032.0f, sa, 72.0f * sb);
      }
    }
  };
  // the first chunk is staged ahead of the loop, so that only the weights' first
  // use waits for them
  stage_h(np < kTBD ? np : kTBD);
  __syncthreads();
  for (int c0 = 0;;) {
    const int tc = np - c0 < kTBD ? np - c0 : kTBD;
    // one pair at a time: its four row sums over every step, then the phase sum
    // (lane bits 2..5, read from lanes 0..3); o rows are in pair order
    for (int ti = 0; ti < tc; ++ti) {
      const uint32_t* ht = hsl + (size_t)ti * (Gd * 17);
      float acc[kDnBlocks];
#pragma unroll
      for (int b = 0; b < kDnBlocks; ++b) acc[b] = 0.0f;
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int j = 16 * i + p;
        const bool ok = blob != nullptr && j < Gd;
        const int jc = j < Gd ? j : 0;
        // the codes and scales are opaque per pair, so their fp16 pairs are formed
        // per pair instead of being hoisted out of the pair loop (register
        // pressure), and nothing before the chunk loop waits for the weights
#pragma unroll
        for (int b = 0; b < kDnBlocks; ++b)
          asm volatile("" : "+v"(cd[b][i].x), "+v"(cd[b][i].y), "+v"(cd[b][i].z), "+v"(cd[b][i].w), "+v"(sdw[b][i]));
        const uint4* hq = reinterpret_cast<const uint4*>(ht + jc * 16);
        const uint4 h0 = hq[0], h1 = hq[1], h2 = hq[2], h3 = hq[3];
        const float C = reinterpret_cast<const float*>(ht + Gd * 16)[jc];
#pragma unroll
        for (int b = 0; b < kDnBlocks; ++b) {
          float P = 0.0f;
          P = code_dot(cd[b][i].x, h0.x, h0.y, h0.z, h0.w, P);
          P = code_dot(cd[b][i].y, h1.x, h1.y, h1.z, h1.w, P);
          P = code_dot(cd[b][i].z, h2.x, h2.y, h2.z, h2.w, P);
          P = code_dot(cd[b][i].w, h3.x, h3.y, h3.z, h3.w, P);
          const float sc = ok ? f16_lo(sdw[b][i] >> sh) : 0.0f;
          acc[b] = fmaf(sc, P - C, acc[b]);
        }
        asm volatile("" ::: "memory");  // one step's h operands at a time (register pressure)
      }
      const int pr = __builtin_amdgcn_readlane(uh.my_pair, c0 + ti);
#pragma unroll
      for (int b = 0; b < kDnBlocks; ++b) {
        const float o = sum_rows(dpp_add<8>(dpp_add<4>(acc[b])));
        if (p == 0) ows[(size_t)pr * H + n0 + 4 * b] = o;
      }
    }
    c0 += kTBD;
    if (c0 >= np) break;
    __syncthreads();  // every wave is done with this chunk
    load_h(c0);
    stage_h(np - c0 < kTBD ? np - c0 : kTBD);
    __syncthreads();
  }
}

// ------------------------------------------------------------------ combine
// y[t][col] = o_shared + sum over k in rank order; every o and w load of an
// output is issued before the sums.
__global__ void __launch_bounds__(kThreads) bat_combine_kernel(FfnArgs a) {
  const int H = a.H, T = a.T, K = a.K;
  const bool has_shared = a.shared_blob != nullptr;
  const BatWs W = bat_ws(T, H, a.I, a.E, K, has_shared);
  const float* ows = reinterpret_cast<const float*>(a.ws + W.o_off);
  const size_t total = (size_t)T * H;
  for (size_t idx = (size_t)blockIdx.x * kThreads + threadIdx.x; idx < total; idx += (size_t)gridDim.x * kThreads) {
    const int t = (int)(idx / H);
    const size_t col = idx % H;
    float acc = has_shared ? ows[(size_t)(T * K + t) * H + col] : 0.0f;
    for (int k0 = 0; k0 < K; k0 += 8) {
      float ov[8], wv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = k0 + j < K ? k0 + j : K - 1;
        ov[j] = ows[(size_t)(t * K + k) * H + col];
        wv[j] = a.w[t * K + k];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (k0 + j < K) acc = fmaf(wv[j], ov[j], acc);
    }
    a.y[idx] = __builtin_bit_cast(uint16_t, (__bf16)acc);
  }
}

inline void set_lds_limit(const void* fn, size_t lds) {
  if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

}  // namespace

bool batched_supported(int T, int H, int I, int K) {
  const int G = H / kGroup, Gd = I / kGroup;
  // gate/up: at most 4 groups per lane; down: at most 4 steps of 16 groups
  return T >= 2 && T <= kGemvMaxT && T * K <= kBatMaxPairs && G <= 4 * 8 * 4 && Gd <= 4 * 16 && H % kDnRowsPerItem == 0 &&
         I % 8 == 0;
}

size_t batched_workspace_bytes(int T, int H, int I, int E, int K, int has_shared) {
  return bat_ws(T, H, I, E, K, has_shared).bytes;
}

hipError_t launch_ffn_batched(const FfnArgs& a, int stage, hipStream_t s) {
  const bool has_shared = a.shared_blob != nullptr;
  const BatWs W = bat_ws(a.T, a.H, a.I, a.E, a.K, has_shared);
  if (stage == 0) {
    const int conv_blocks = (a.T * a.H / 2 + kPlanThreads - 1) / kPlanThreads;
    hipLaunchKernelGGL(bat_plan_kernel, dim3(1 + conv_blocks), dim3(kPlanThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int G = a.H / kGroup;
    const int GW = (G + kWaves - 1) / kWaves;
    const int gpl = (GW + 7) / 8;
    const size_t lds = (size_t)kWaves * kTB * GW * 17 * 4;
    const int grid = W.U * (a.I / 8);
#define GU(N)                                                                                       \
  do {                                                                                              \
    set_lds_limit(reinterpret_cast<const void*>(&bat_gateup_kernel<N>), lds);                       \
    hipLaunchKernelGGL((bat_gateup_kernel<N>), dim3(grid), dim3(kThreads), lds, s, a);              \
  } while (0)
    if (gpl <= 1) GU(1);
    else if (gpl <= 2) GU(2);
    else GU(4);
#undef GU
    return hipGetLastError();
  }
  {
    const int Gd = a.I / kGroup;
    const int spl = (Gd + 15) / 16;
    const size_t lds = (size_t)kTBD * Gd * 17 * 4;
    const int grid = W.U * (a.H / kDnRowsPerItem);
#define DN(N)                                                                                       \
  do {                                                                                              \
    set_lds_limit(reinterpret_cast<const void*>(&bat_down_kernel<N>), lds);                         \
    hipLaunchKernelGGL((bat_down_kernel<N>), dim3(grid), dim3(kThreads), lds, s, a);                \
  } while (0)
    if (spl <= 1) DN(1);
    else if (spl <= 2) DN(2);
    else DN(4);
#undef DN
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t total = (size_t)a.T * a.H;
  const size_t blocks = (total + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(bat_combine_kernel, dim3(blocks < 2048 ? (int)blocks : 2048), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
