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
constexpr int kTB = 4;                 // pairs per chunk
constexpr int kPlanThreads = 1024;
constexpr int kBatMaxPairs = 512;      // routed pairs T*K the plan covers

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

__host__ __device__ inline int bat_umax(int T, int K, int E, int has_shared) {
  return (T * K < E ? T * K : E) + (has_shared ? 1 : 0);
}
__host__ __device__ inline int bat_pmax(int T, int K, int has_shared) { return T * K + (has_shared ? T : 0); }

// Workspace: plan ints [n_units | rec[U][4] | pair_list[P]], x16 fp16 [T][H],
// xc fp32 [T][G] (per-group corrections of x16), h fp16 [P][I] with rows in
// unit order (row i = pair_list[i]), o fp32 [P][H] with rows in pair order.
// rec[u] = {slot (-1: the shared expert, -2: not usable), first row of the
// unit in pair_list, pair count (0 past the last unit), expert}.
struct BatWs {
  size_t x16_off, xc_off, h_off, o_off, bytes;
  int U, P;
};
__host__ __device__ inline BatWs bat_ws(int T, int H, int I, int E, int K, int has_shared) {
  BatWs w;
  w.U = bat_umax(T, K, E, has_shared);
  w.P = bat_pmax(T, K, has_shared);
  const size_t plan_ints = 4 + (size_t)w.U * 4 + w.P;
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
  int* pair_list;
};
__device__ inline PlanView plan_view(uint8_t* ws, int U, int P) {
  int* p = reinterpret_cast<int*>(ws);
  PlanView v;
  v.n_units = p;
  v.rec = reinterpret_cast<int4*>(p + 4);  // 16-byte aligned
  v.pair_list = p + 4 + 4 * U;
  return v;
}

// The plan's unit count through the scalar cache: it is written by the plan
// kernel and read-only for the kernels after it.
__device__ inline int plan_n_units(const PlanView& pl) {
  return *(const __attribute__((address_space(4))) int*)(pl.n_units);
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
  __shared__ int unit_of_pair[kBatMaxPairs];
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
  if (p < P) unit_of_pair[p] = up;
  if (valid) atomicAdd(&cnt[up], 1);  // integer counts: the order of additions does not matter
  __syncthreads();
  // rank of the pair among its unit's pairs (pair order)
  int rank = 0;
  if (valid)
    for (int q = 0; q < p; ++q) rank += unit_of_pair[q] == up;
  // unit offsets: the shared unit holds T pairs, routed units their counts
  const int n_units = base + n_routed;
  const int c = tid < n_units ? (has_shared && tid == 0 ? T : cnt[tid]) : 0;
  int total;
  const int off = block_exclusive_scan(c, wsum, &total);
  if (tid < n_units) uoff[tid] = off;
  __syncthreads();
  if (valid) pl.pair_list[uoff[up] + rank] = p;
  if (has_shared && tid < T) pl.pair_list[tid] = T * K + tid;
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
  // stream from HBM together, and the workgroups past the plan's last unit leave at once
  const int n_hb = I / 8;
  {
    const int item = blockIdx.x;
    const int u = item / n_hb, hb = item % n_hb;
    if (u >= plan_n_units(pl)) return;
    const int4 rc = pl.rec[u];
    const int p0 = rc.y, np = rc.z;
    uint32_t* xs = reinterpret_cast<uint32_t*>(smem) + (size_t)wave * kTB * (GW * 17);
    const int j0 = wave * GW;
    const int gw_here = G - j0 < GW ? (G - j0 > 0 ? G - j0 : 0) : GW;
    const uint8_t* blob = rec_blob(a, rc.x);
    const uint8_t* src = blob ? blob : a.slots;  // any readable blob; its terms get scale 0
    if (np > 64) {  // only with an expert repeated within a token's ids (moe_route never does that)
      if (tid == 0) *a.status = MOE_EUNSUP;
      return;
    }
    const int my_pair = pl.pair_list[p0 + (lane < np ? lane : np - 1)];  // lane i: the unit's pair i
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
    __builtin_amdgcn_sched_barrier(0);
    _Float16* hws = reinterpret_cast<_Float16*>(a.ws + W.h_off);
    const uint4* x16 = reinterpret_cast<const uint4*>(a.ws + W.x16_off);
    const float* xc = reinterpret_cast<const float*>(a.ws + W.xc_off);
    const int sh = (r & 1) * 16;
    for (int c0 = 0; c0 < np; c0 += kTB) {
      const int tc = np - c0 < kTB ? np - c0 : kTB;
      // copy the chunk's fp16 x slices and corrections into the wave's LDS: uint4 q
      // of a token's slice is columns 8q .. 8q+7 of the wave's groups; every
      // token's loads are issued before any is stored
      constexpr int XQ = (GPL + 1) / 2;  // uint4 per lane and token (GW <= 8 * GPL groups)
      uint4 xv[kTB][XQ];
      float cv[kTB];
  #pragma unroll
      for (int ti = 0; ti < kTB; ++ti) {
        const int t = pair_token(__builtin_amdgcn_readlane(my_pair, c0 + (ti < tc ? ti : tc - 1)), T, K);
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
  #pragma unroll
      for (int ti = 0; ti < kTB; ++ti) {
        uint32_t* xt = xs + (size_t)ti * (GW * 17);
  #pragma unroll
        for (int v = 0; v < XQ; ++v) {
          const int q = lane + 64 * v;
          if (q < GW * 4) reinterpret_cast<uint4*>(xt)[q] = (ti < tc && q < gw_here * 4) ? xv[ti][v] : make_uint4(0u, 0u, 0u, 0u);
        }
        if (lane < GW) reinterpret_cast<float*>(xt + GW * 16)[lane] = (ti < tc && lane < gw_here) ? cv[ti] : 0.0f;
      }
      __builtin_amdgcn_wave_barrier();
      float ag[kTB], au[kTB];
  #pragma unroll
      for (int ti = 0; ti < kTB; ++ti) ag[ti] = au[ti] = 0.0f;
  #pragma unroll
      for (int i = 0; i < GPL; ++i) {
        const int jl = 8 * i + p;
        const bool ok = blob != nullptr && jl < gw_here;
        const int jc = jl < gw_here ? jl : 0;
        const float sg = ok ? f16_lo(sgw[i] >> sh) : 0.0f;
        const float su = ok ? f16_lo(suw[i] >> sh) : 0.0f;
        uint32_t pg[16], pu[16];
        code_pairs(cg[i], pg);
        code_pairs(cu[i], pu);
  #pragma unroll
        for (int ti = 0; ti < kTB; ++ti) {
          if (ti < tc) {
            const uint32_t* xt = xs + (size_t)ti * (GW * 17);
            const uint4* xq = reinterpret_cast<const uint4*>(xt + jc * 16);
            const uint4 x0 = xq[0], x1 = xq[1], x2 = xq[2], x3 = xq[3];
            const uint32_t xw[16] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w,
                                     x2.x, x2.y, x2.z, x2.w, x3.x, x3.y, x3.z, x3.w};
            const float C = reinterpret_cast<const float*>(xt + GW * 16)[jc];
            float dg = 0.0f, du = 0.0f;
  #pragma unroll
            for (int k = 0; k < 16; ++k) {
              dg = dot2h(pg[k], xw[k], dg);
              du = dot2h(pu[k], xw[k], du);
            }
            ag[ti] = fmaf(sg, dg - C, ag[ti]);
            au[ti] = fmaf(su, du - C, au[ti]);
          }
          // token ti is done here: the next token's LDS reads are not hoisted above (register pressure)
          asm volatile("" : "+v"(ag[ti]), "+v"(au[ti])::"memory");
        }
      }
      // phases (lane bits 3..5), read from lanes 0..7, then the waves in order
  #pragma unroll
      for (int ti = 0; ti < kTB; ++ti) {
        const float g = sum_rows(dpp_add<8>(ag[ti]));
        const float uu = sum_rows(dpp_add<8>(au[ti]));
        if (p == 0) {
          part[ti][0][wave][r] = g;
          part[ti][1][wave][r] = uu;
        }
      }
      // pair of the token thread tid < 8 * tc finishes, read while every lane is active
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
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ down
// One workgroup per (unit, 64 rows of H); wave w owns rows 16w .. 16w+15 of the
// item, as four 4-row blocks of the blob. SPL = steps per lane = ceil(Gd / 16):
// at step i lane (row r of 4, phase p of 16) takes group 16i + p of its row in
// each block. The chunk's h rows are staged once per wave and serve all four
// blocks.
constexpr int kDnRowsPerItem = 64;
constexpr int kDnBlocks = 4;  // 4-row blocks per wave

template <int SPL>
__global__ void __launch_bounds__(kThreads) bat_down_kernel(FfnArgs a) {
  // LDS per wave: for each of the chunk's pairs, the h row as fp16 pairs
  // [Gd][16] dwords and the group corrections [Gd]
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const int Gd = I / kGroup;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 3, p = lane >> 2;
  const bool has_shared = a.shared_blob != nullptr;
  const BatWs W = bat_ws(T, H, I, a.E, K, has_shared);
  const PlanView pl = plan_view(a.ws, W.U, W.P);
  // one item per workgroup, a unit's items consecutive (as in bat_gateup)
  const int n_rb = H / kDnRowsPerItem;
  {
    const int item = blockIdx.x;
    const int u = item / n_rb, rb = item % n_rb;
    if (u >= plan_n_units(pl)) return;
    const int4 rc = pl.rec[u];
    const int p0 = rc.y, np = rc.z;
    if (np > 64) {  // only with an expert repeated within a token's ids (moe_route never does that)
      if (lane == 0) *a.status = MOE_EUNSUP;
      return;
    }
    const int my_pair = pl.pair_list[p0 + (lane < np ? lane : np - 1)];  // lane i: the unit's pair i
    uint32_t* hsl = reinterpret_cast<uint32_t*>(smem) + (size_t)wave * kTB * (Gd * 17);
    const uint8_t* blob = rec_blob(a, rc.x);
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
    const uint4* h4 = reinterpret_cast<const uint4*>(a.ws + W.h_off);  // h fp16 [position][I]
    float* ows = reinterpret_cast<float*>(a.ws + W.o_off);
    const int sh = (r & 1) * 16;
    const int per_pair = Gd * 4;  // uint4 of one h row
    for (int c0 = 0; c0 < np; c0 += kTB) {
      const int tc = np - c0 < kTB ? np - c0 : kTB;
      // stage the chunk's h rows: uint4 q of the chunk = pair q / per_pair, group (q / 4) % Gd,
      // halves 8 * (q % 4) .. +7; the four lanes of a group are adjacent
      for (int q0 = 0; q0 < kTB * per_pair; q0 += 64) {
        const int q = q0 + lane;
        const int ti = q / per_pair;
        const int rem = q - ti * per_pair;
        const bool live = ti < tc;
        uint4 hv = h4[(size_t)(p0 + c0 + (live ? ti : 0)) * (I / 8) + rem];
        if (!live) hv = make_uint4(0u, 0u, 0u, 0u);
        const uint32_t d[4] = {hv.x, hv.y, hv.z, hv.w};
        float sa = (f16_lo(d[0]) + f16_hi(d[0])) + (f16_lo(d[2]) + f16_hi(d[2]));
        float sb = (f16_lo(d[1]) + f16_hi(d[1])) + (f16_lo(d[3]) + f16_hi(d[3]));
        sa = quad_xor_add<2>(quad_xor_add<1>(sa));
        sb = quad_xor_add<2>(quad_xor_add<1>(sb));
        if (ti < kTB) {
          uint32_t* ht = hsl + (size_t)ti * (Gd * 17);
          reinterpret_cast<uint4*>(ht)[rem] = hv;
          if ((lane & 3) == 0) reinterpret_cast<float*>(ht + Gd * 16)[rem >> 2] = fmaf(1032.0f, sa, 72.0f * sb);
        }
      }
      __builtin_amdgcn_wave_barrier();
      float acc[kDnBlocks][kTB];
  #pragma unroll
      for (int b = 0; b < kDnBlocks; ++b)
  #pragma unroll
        for (int ti = 0; ti < kTB; ++ti) acc[b][ti] = 0.0f;
  #pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int j = 16 * i + p;
        const bool ok = blob != nullptr && j < Gd;
        const int jc = j < Gd ? j : 0;
  #pragma unroll
        for (int ti = 0; ti < kTB; ++ti) {
          // the codes are opaque per pair, so their fp16 pairs are formed per pair
          // instead of being hoisted out for all blocks and steps (register pressure)
#pragma unroll
          for (int b = 0; b < kDnBlocks; ++b)
            asm volatile("" : "+v"(cd[b][i].x), "+v"(cd[b][i].y), "+v"(cd[b][i].z), "+v"(cd[b][i].w));
          if (ti < tc) {
            const uint32_t* ht = hsl + (size_t)ti * (Gd * 17);
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
              acc[b][ti] = fmaf(sc, P - C, acc[b][ti]);
            }
          }
          asm volatile("" ::: "memory");  // one pair's h operands at a time (register pressure)
        }
      }
      // phases (lane bits 2..5), read from lanes 0..3
  #pragma unroll
      for (int ti = 0; ti < kTB; ++ti) {
        const int pr = __builtin_amdgcn_readlane(my_pair, c0 + ti);  // o rows are in pair order
  #pragma unroll
        for (int b = 0; b < kDnBlocks; ++b) {
          const float o = sum_rows(dpp_add<8>(dpp_add<4>(acc[b][ti])));
          if (ti < tc && p == 0) ows[(size_t)pr * H + n0 + 4 * b] = o;
        }
      }
      __builtin_amdgcn_wave_barrier();  // the next chunk rewrites this wave's LDS
    }
  }
}

// ------------------------------------------------------------------ combine
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
    for (int k = 0; k < K; ++k) acc = fmaf(a.w[t * K + k], ows[(size_t)(t * K + k) * H + col], acc);
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
    const size_t lds = (size_t)kWaves * kTB * Gd * 17 * 4;
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
