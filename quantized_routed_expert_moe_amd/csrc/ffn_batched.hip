// Small-batch expert FFN (2 <= T <= 32 tokens).
//
// A unit is one distinct expert of the batch (or the always-on shared expert)
// with every (token, rank) pair routed to it, so each expert's bytes stream
// from HBM once however many tokens use it ("Strata" README, Models: W4A16
// experts). Four kernels:
//   bat_plan      one workgroup: units in order of their first pair (the
//                 shared expert first), each unit's pairs in pair order, and
//                 per unit one record (slot, first pair, pair count) into the
//                 workspace; other workgroups convert x to fp16 once. Pair
//                 p = t*K + k for routed pairs, T*K + t for the shared
//                 expert's. Under moe_layer the same workgroup first selects
//                 every token's top-k from the logits (one wave per token,
//                 the selection of route_select_kernel, so the same ids and
//                 weights), which saves the routing launch.
//   bmx_gateup    MFMA over (unit pairs x 16 weight rows) tiles; h =
//                 silu(g) * u in fp16, one row per pair in unit order.
//   bmx_down      the same for the down matrix; o (fp32) at each pair's row.
//   bat_combine   y[t] = o_shared[t] + sum_k w[t][k] * o[t*K + k] in rank
//                 order, rounded once to bf16.
// No atomics on floating-point values; every sum has a fixed order.
#include <type_traits>

#include "lds_dma.h"
#include "moe_internal.h"
#include "timeline.h"
#include "wave_ops.h"

namespace moe {
MOE_TL_UNIT(batched, MOE_TL_BAT_PLAN, 4)
namespace {

constexpr int kThreads = 256;
constexpr int kUnitPairs = 64;         // pairs one unit can hold (a routed unit has at most T)
constexpr int kPlanThreads = 1024;
constexpr int kBatMaxPairs = 512;      // routed pairs T*K the plan covers
static_assert(kMaxE <= kPlanThreads, "the plan loads one slot-table entry per thread");

__host__ __device__ inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

__host__ __device__ inline int bat_umax(int T, int K, int E, int has_shared) {
  return (T * K < E ? T * K : E) + (has_shared ? 1 : 0);
}
__host__ __device__ inline int bat_pmax(int T, int K, int has_shared) { return T * K + (has_shared ? T : 0); }

// Workspace: plan ints [n_units | rec[U][4] | ptab[U][kUnitPairs]], x16 fp16
// [T][H], h fp16 [P][I] with rows in unit order (row rec[u].y + i is pair ptab[u][i]), o fp32 [P][H] with
// rows in pair order. rec[u] = {slot (-1: the shared expert, -2: not usable),
// first h row of the unit, pair count (0 past the last unit), expert}; the
// pair table has a fixed stride, so a workgroup loads its unit's record and
// pairs in one round trip.
struct BatWs {
  size_t x16_off, h_off, o_off, bytes;
  int U, P;
};
__host__ __device__ inline BatWs bat_ws(int T, int H, int I, int E, int K, int has_shared) {
  BatWs w;
  w.U = bat_umax(T, K, E, has_shared);
  w.P = bat_pmax(T, K, has_shared);
  const size_t plan_ints = 4 + (size_t)w.U * (4 + kUnitPairs);
  w.x16_off = align256(plan_ints * 4);
  w.h_off = align256(w.x16_off + (size_t)T * H * 2);
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

// x as fp16 (x16): thread i converts dword i of x; a value that does not fit
// fp16 sets MOE_EUNSUP (bf16 converts exactly for |x| in [2^-17, 65504]).
__device__ inline void plan_convert_x(const FfnArgs& a, const BatWs& W, int i) {
  if (i >= a.T * a.H / 2) return;
  const uint32_t v = reinterpret_cast<const uint32_t*>(a.x)[i];
  bool bad = false;
  const uint32_t lo = to_f16_bits(__uint_as_float(v << 16), &bad);
  const uint32_t hi = to_f16_bits(__uint_as_float(v & 0xFFFF0000u), &bad);
  reinterpret_cast<uint32_t*>(a.ws + W.x16_off)[i] = lo | (hi << 16);
  if (bad) *a.status = MOE_EUNSUP;
}

// ------------------------------------------------------------------ plan
// EPL > 0: workgroup 0 first selects the top-k of every token from a.route_logits
// (wave v takes tokens v, v + 16, ...; EPL = experts per lane) and writes ids and w.
template <int EPL>
__global__ void __launch_bounds__(kPlanThreads) bat_plan_kernel(FfnArgs a) {
  const TlRow tl = tl_begin(MOE_TL_BAT_PLAN);
  __shared__ int first[kMaxE];  // lowest pair using expert e, then the unit of expert e
  __shared__ int slot_lds[kMaxE];  // the slot table, loaded at the start
  __shared__ int ids_lds[kBatMaxPairs];
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
    tl_end(tl);
    return;
  }
  // the slot table (E <= kPlanThreads entries, one per thread) and the ids or
  // logits go out first: the records need the table only after the dedup, so no
  // dependent load is left for later
  const int sv = tid < E ? a.slot_table[tid] : 0;
  const int p = tid;  // P <= kBatMaxPairs < kPlanThreads: one pair per thread
  int e = -1;
  if constexpr (EPL == 0) {
    e = p < P ? a.ids[p] : -1;
  } else {
    const int wave = tid >> 6, lane = tid & 63;
    for (int t = wave; t < T; t += kPlanThreads / 64) {
      int32_t id;
      float wt;
      wave_select<EPL>(a.route_logits + (size_t)t * E, E, K, a.route_flags, lane, id, wt);
      if (lane < K) {
        const_cast<int32_t*>(a.ids)[t * K + lane] = id;
        const_cast<float*>(a.w)[t * K + lane] = wt;
        ids_lds[t * K + lane] = id;
      }
    }
  }
  for (int x = tid; x < E; x += kPlanThreads) first[x] = 0x7FFFFFFF;
  for (int u = tid; u <= kBatMaxPairs; u += kPlanThreads) cnt[u] = 0;
  if (tid < E) slot_lds[tid] = sv;
  __syncthreads();
  if constexpr (EPL > 0) e = p < P ? ids_lds[p] : -1;
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
        const int slot = slot_lds[ex];
        if (slot < 0) *a.status = MOE_ENOTRES;
        rc.x = slot < 0 ? -2 : slot;
      }
    }
    pl.rec[u] = rc;
  }
  tl_end(tl);
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

// ------------------------------------------------------------------ MFMA helpers
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ inline f16x8_t dequant_qs(uint32_t cw, _Float16 sc) {
  const f16x2_t s2 = {sc, sc};
  const f16x2_t off_a = {(_Float16)-1032.0f, (_Float16)-1032.0f}, off_b = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t w8 = cw >> 8;
  const uint32_t m0 = (cw & 0x000F000Fu) | 0x64006400u, m1 = (cw & 0x00F000F0u) | 0x54005400u;
  const uint32_t m2 = (w8 & 0x000F000Fu) | 0x64006400u, m3 = (w8 & 0x00F000F0u) | 0x54005400u;
  uint32_t b[4];
  b[0] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, m0) + off_a) * s2);
  b[1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, m1) + off_b) * s2);
  b[2] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, m2) + off_a) * s2);
  b[3] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2_t, m3) + off_b) * s2);
  return __builtin_bit_cast(f16x8_t, make_uint4(b[0], b[1], b[2], b[3]));
}
__device__ inline f16x8_t as_f16x8(const uint4& v) { return __builtin_bit_cast(f16x8_t, v); }
// Buffer loads of expert codes and scales (a read past the descriptor's range
// returns zeros). Each unit's weights are read once per layer, so the loads
// carry the non-temporal hint (cache-policy bit 1, nt) and leave the caches to
// the data that is read again (x, the plan records, h).
constexpr int kStreamPolicy = 2;
__device__ inline uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamPolicy));
}
__device__ inline uint16_t bload2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kStreamPolicy);
}
__device__ inline uint32_t dword_of(const uint4& v, int i) { return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w)); }

// Scale of one chunk: 0 for a chunk past the groups or an unusable unit; a
// magnitude >= 8192 sets *bad.
__device__ inline _Float16 chunk_scale(uint16_t bits, bool ok, bool* bad) {
  const _Float16 s = __builtin_bit_cast(_Float16, bits);
  if (ok && !((float)__builtin_fabsf16(s) < 8192.0f)) *bad = true;
  return ok ? s : (_Float16)0.0f;
}

// ------------------------------------------------------------------ gate/up and down
// The unit's pairs are the M rows of v_mfma_f32_16x16x32_f16 and 16 weight
// rows its N columns, so one dequantised weight fragment serves every pair of
// the unit and the work per item hardly depends on the pair count. Lane l
// (n = l % 16, q = l / 16) loads the 16-byte code chunk of (row n, group
// 4c + q); MFMA i of chunk c takes dword i of every lane, i.e. columns
// 32 (4c + q) + 8i .. +7 of each quarter's group, and the A fragment of lane
// (m, q) holds the same columns of pair row m. B = fp16(q * s): the code's
// exact fp16 value (1024 + u or 64 + u under an fp16 pattern, minus 1032 or
// 72) times the group's fp16 scale, rounded once (relative error <= 2^-11),
// so a chunk's four groups share one accumulator. A scale of magnitude
// >= 8192 could overflow that product and sets MOE_EUNSUP. The D fragment of
// lane l holds pair rows 4 (l / 16) + v of weight row l % 16.
//
// Each wave owns whole 16-row tiles over every group, so its D fragments are
// final sums and no partial crosses waves. The A rows (x of the pairs'
// tokens, or the unit's h rows), KM per M-tile, go to LDS by direct
// buffer-to-LDS loads issued before the weight loads and waited for alone;
// A rows past the unit's pairs, the 16-byte pad after each row (which keeps
// the 8 lanes of a ds_read_b128 phase on distinct banks) and a tail are
// zeros, so every fragment is read as is. A unit with more pairs than KM
// runs further M-tiles (the weights are read again). The weight loads are
// buffer loads with a per-lane offset and a per-chunk constant; a group past
// the last reads other blob bytes or zeros past its end and gets scale 0.
// Workgroup sizes are chosen so that the items of a 16-token layer are
// resident at once with a small spread of rows per CU:
//   gate/up: NW waves of one 16-row tile each (96 rows where I allows); the
//     codes and scales of CW chunks are in flight per wave, the load of
//     chunk c + CW issued once chunk c is done.
//   down: NW waves of one tile each, all codes loaded up front.
__host__ __device__ inline int bmx_row_bytes(int cols) { return cols * 2 + 16; }
constexpr int kBmxTail = 256;  // zero bytes after the rows: reads of a group past the last stay inside
__host__ __device__ inline size_t bmx_lds(int cols, int KM) { return (size_t)KM * bmx_row_bytes(cols) + kBmxTail; }

// Zero the pads of rows < live, rows live .. KM - 1 whole, and the tail (the
// workgroup's nt threads; LDS stores, waited for before the next barrier).
__device__ inline void bmx_zero_rows(unsigned char* base, int cols, int KM, int live, int tid, int nt) {
  const int RB = bmx_row_bytes(cols);
  const uint4 z = make_uint4(0u, 0u, 0u, 0u);
  for (int r = tid; r < live; r += nt) *reinterpret_cast<uint4*>(base + r * RB + cols * 2) = z;
  const int n16 = (KM - live) * (RB / 16) + kBmxTail / 16;
  uint4* d = reinterpret_cast<uint4*>(base + live * RB);
  for (int i = tid; i < n16; i += nt) d[i] = z;
}

// s_waitcnt: at most vm vector-memory operations outstanding and every LDS access done
__host__ __device__ constexpr int vm_lds_imm(int vm) { return vmcnt_imm(vm) & ~(15 << 8); }

template <int NW, int CQ, int CW, int KM>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(3))) bmx_gateup_kernel(FfnArgs a) {
  const TlRow tl = tl_begin(MOE_TL_BMX_GATEUP);
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const int G = H / kGroup;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q = lane >> 4;
  const bool has_shared = a.shared_blob != nullptr;
  const BatWs W = bat_ws(T, H, I, a.E, K, has_shared);
  const PlanView pl = plan_view(a.ws, W.U, W.P);
  const int n_nt = I / (16 * NW);
  const int u = blockIdx.x / n_nt, nt = blockIdx.x % n_nt;
  const UnitHead uh = unit_head(pl, u, lane);
  const int p0 = uh.p0, np = uh.np;
  if (np == 0) {
    tl_end(tl);
    return;
  }
  tl_mark(tl, 0);
  if (np > kUnitPairs) {
    if (tid == 0) *a.status = MOE_EUNSUP;
    return;
  }
  const uint8_t* blob = rec_blob(a, uh.slot);
  const uint8_t* src = blob ? blob : a.slots;  // any readable blob; its terms get scale 0
  const BlobLayout BL = blob_layout(H, I);
  const int XB = bmx_row_bytes(H);
  unsigned char* xs = smem;  // [KM][XB], then the zero tail
  const __amdgpu_buffer_rsrc_t xr = buf_rsrc(a.ws + W.x16_off, (uint32_t)((size_t)T * H * 2));
  const __amdgpu_buffer_rsrc_t br = buf_rsrc(src, (uint32_t)BL.bytes);
  const int row = (nt * NW + wave) * 16 + n;  // this lane's weight row (B column n)
  const uint4* xap = reinterpret_cast<const uint4*>(xs + n * XB + q * 64);  // A row n (lane % 16)
  _Float16* hws = reinterpret_cast<_Float16*>(a.ws + W.h_off);
  const uint32_t c_off = (uint32_t)code_off(row, q, G, kRowBlockGU), s_off = (uint32_t)scale_off(row, q, G, kRowBlockGU);
  uint4 cg[CW], cu[CW];
  uint16_t sgb[CW], sub[CW];
  uint32_t zo = 0;
  auto load_chunk = [&](int c) {
    const uint32_t dc = (uint32_t)c * 4 * kRowBlockGU * 16, ds = (uint32_t)c * 4 * kRowBlockGU * 2;
    cg[c % CW] = bload16(br, c_off, zo + (uint32_t)BL.gate_codes + dc);
    cu[c % CW] = bload16(br, c_off, zo + (uint32_t)BL.up_codes + dc);
    sgb[c % CW] = bload2(br, s_off, zo + (uint32_t)BL.gate_scales + ds);
    sub[c % CW] = bload2(br, s_off, zo + (uint32_t)BL.up_scales + ds);
  };
  bool bad = false;
  for (int m0 = 0; m0 < np; m0 += KM) {
    if (m0 > 0) __syncthreads();  // every wave is done with the staged rows
    // an opaque zero offset per M-tile keeps the weight loads (and their fp16 forms)
    // inside the tile, not hoisted out of the loop and held for every chunk at once
    asm volatile("" : "+s"(zo));
    const int rows = np - m0 < KM ? np - m0 : KM;
    for (int r = 0; r < rows; ++r) {
      const int t = pair_token(__builtin_amdgcn_readlane(uh.my_pair, m0 + r), T, K);
      stage_lds(xr, (uint32_t)((size_t)t * H * 2), H / 8, xs + r * XB, wave, lane, NW);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < CW; ++c) load_chunk(c);
    __builtin_amdgcn_sched_barrier(0);
    bmx_zero_rows(xs, H, KM, rows, tid, NW * 64);
    __builtin_amdgcn_s_waitcnt(vm_lds_imm(4 * CW));  // the staged rows (issued first) and the zeros are in LDS
    __builtin_amdgcn_s_barrier();
    if (m0 == 0) tl_mark(tl, 1);
    f32x4_t ag = {0.0f, 0.0f, 0.0f, 0.0f}, au = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < CQ; ++c) {
      if (4 * c >= G) continue;  // a chunk wholly past the groups
      uint4 xa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xa[i] = xap[16 * c + i];
      const bool ok = blob != nullptr && 4 * c + q < G;
      const _Float16 sg = chunk_scale(sgb[c % CW], ok, &bad);
      const _Float16 su = chunk_scale(sub[c % CW], ok, &bad);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ag = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(xa[i]), dequant_qs(dword_of(cg[c % CW], i), sg), ag, 0, 0, 0);
        au = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(xa[i]), dequant_qs(dword_of(cu[c % CW], i), su), au, 0, 0, 0);
      }
      if (c + CW < CQ && 4 * (c + CW) < G) load_chunk(c + CW);
      __builtin_amdgcn_sched_barrier(0);  // one chunk's operands at a time (register pressure)
    }
    tl_mark(tl, 2);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * q + v;
      if (m < rows) {
        const float hv = blob ? silu(ag[v]) * au[v] : 0.0f;
        if (!(fabsf(hv) < 65520.0f)) bad = true;
        hws[(size_t)(p0 + m0 + m) * I + row] = (_Float16)hv;
      }
    }
  }
  if (bad) *a.status = MOE_EUNSUP;
  tl_end(tl);
}

template <int NW, int CQ, int KM>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(CQ <= 6 ? 6 : 4))) bmx_down_kernel(FfnArgs a) {
  const TlRow tl = tl_begin(MOE_TL_BMX_DOWN);
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const int Gd = I / kGroup;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q = lane >> 4;
  const bool has_shared = a.shared_blob != nullptr;
  const BatWs W = bat_ws(T, H, I, a.E, K, has_shared);
  const PlanView pl = plan_view(a.ws, W.U, W.P);
  const int n_nt = H / (16 * NW);
  const int u = blockIdx.x / n_nt, nt = blockIdx.x % n_nt;
  const UnitHead uh = unit_head(pl, u, lane);
  const int p0 = uh.p0, np = uh.np;
  if (np == 0) {
    tl_end(tl);
    return;
  }
  tl_mark(tl, 0);
  if (np > kUnitPairs) {
    if (tid == 0) *a.status = MOE_EUNSUP;
    return;
  }
  const uint8_t* blob = rec_blob(a, uh.slot);
  const uint8_t* src = blob ? blob : a.slots;
  const BlobLayout BL = blob_layout(H, I);
  const int HB = bmx_row_bytes(I);
  unsigned char* hs = smem;  // [KM][HB], then the zero tail
  const __amdgpu_buffer_rsrc_t hr = buf_rsrc(a.ws + W.h_off, (uint32_t)((size_t)W.P * I * 2));
  const __amdgpu_buffer_rsrc_t br = buf_rsrc(src, (uint32_t)BL.bytes);
  const int row = (nt * NW + wave) * 16 + n;
  const uint4* hap = reinterpret_cast<const uint4*>(hs + n * HB + q * 64);
  float* ows = reinterpret_cast<float*>(a.ws + W.o_off);
  const uint32_t c_off = (uint32_t)code_off(row, q, Gd, kRowBlockDN), s_off = (uint32_t)scale_off(row, q, Gd, kRowBlockDN);
  uint4 cd[CQ];
  uint16_t sdb[CQ];
  uint32_t zo = 0;
  bool bad = false;
  for (int m0 = 0; m0 < np; m0 += KM) {
    if (m0 > 0) __syncthreads();
    asm volatile("" : "+s"(zo));  // weight loads stay inside the M-tile (register pressure)
    const int rows = np - m0 < KM ? np - m0 : KM;
    for (int r = 0; r < rows; ++r)
      stage_lds(hr, (uint32_t)((size_t)(p0 + m0 + r) * I * 2), I / 8, hs + r * HB, wave, lane, NW);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < CQ; ++c) {
      cd[c] = bload16(br, c_off, zo + (uint32_t)BL.down_codes + (uint32_t)c * 4 * kRowBlockDN * 16);
      sdb[c] = bload2(br, s_off, zo + (uint32_t)BL.down_scales + (uint32_t)c * 4 * kRowBlockDN * 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    bmx_zero_rows(hs, I, KM, rows, tid, NW * 64);
    __builtin_amdgcn_s_waitcnt(vm_lds_imm(2 * CQ));
    __builtin_amdgcn_s_barrier();
    if (m0 == 0) tl_mark(tl, 1);
    f32x4_t ao = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = 0; c < CQ; ++c) {
      if (4 * c >= Gd) continue;
      uint4 ha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ha[i] = hap[16 * c + i];
      const _Float16 sd = chunk_scale(sdb[c], blob != nullptr && 4 * c + q < Gd, &bad);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ao = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(ha[i]), dequant_qs(dword_of(cd[c], i), sd), ao, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);  // one chunk's operands at a time (register pressure)
    }
    tl_mark(tl, 2);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * q + v;
      const int pr = __shfl(uh.my_pair, m0 + (m < rows ? m : 0), 64);
      if (m < rows) ows[(size_t)pr * H + row] = ao[v];
    }
  }
  if (bad) *a.status = MOE_EUNSUP;
  tl_end(tl);
}

// ------------------------------------------------------------------ combine
// y[t][col] = o_shared + sum over k in rank order; every o and w load of an
// output is issued before the sums.
__global__ void __launch_bounds__(kThreads) bat_combine_kernel(FfnArgs a) {
  const TlRow tl = tl_begin(MOE_TL_BAT_COMBINE);
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
  tl_end(tl);
}

inline void set_lds_limit(const void* fn, size_t lds) {
  if (lds > 65536) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
}

}  // namespace

bool batched_routes(int E) { return E >= 1 && E <= 1024; }

bool batched_supported(int T, int H, int I, int K) {
  const int G = H / kGroup, Gd = I / kGroup;
  // gate/up: at most 32 chunks of 4 groups (LDS: 16 rows of x); down: at most 16
  return T >= 2 && T <= kGemvMaxT && T * K <= kBatMaxPairs && G <= 128 && Gd <= 64;
}

size_t batched_workspace_bytes(int T, int H, int I, int E, int K, int has_shared) {
  return bat_ws(T, H, I, E, K, has_shared).bytes;
}

hipError_t launch_ffn_batched(const FfnArgs& a, int stage, hipStream_t s) {
  const bool has_shared = a.shared_blob != nullptr;
  const BatWs W = bat_ws(a.T, a.H, a.I, a.E, a.K, has_shared);
  constexpr int KM = 16;  // pairs per M-tile
  if (stage == 0) {
    const int conv_blocks = (a.T * a.H / 2 + kPlanThreads - 1) / kPlanThreads;
    const dim3 pg(1 + conv_blocks), pb(kPlanThreads);
    const int epl = (a.E + 63) / 64;
    if (!a.route_logits) hipLaunchKernelGGL(bat_plan_kernel<0>, pg, pb, 0, s, a);
    else if (epl <= 1) hipLaunchKernelGGL(bat_plan_kernel<1>, pg, pb, 0, s, a);
    else if (epl <= 2) hipLaunchKernelGGL(bat_plan_kernel<2>, pg, pb, 0, s, a);
    else if (epl <= 4) hipLaunchKernelGGL(bat_plan_kernel<4>, pg, pb, 0, s, a);
    else if (epl <= 8) hipLaunchKernelGGL(bat_plan_kernel<8>, pg, pb, 0, s, a);
    else hipLaunchKernelGGL(bat_plan_kernel<16>, pg, pb, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int chunks = (a.H / kGroup + 3) / 4;
    const size_t lds = bmx_lds(a.H, KM);
    // 96-row workgroups where I allows (two resident per CU), else 64 or 32 rows
    const int nw = a.I % 96 == 0 ? 6 : (a.I % 64 == 0 ? 4 : 2);
#define GU(NW, CQ)                                                                                  \
  do {                                                                                              \
    constexpr int CW = CQ < 6 ? CQ : 6;                                                             \
    set_lds_limit(reinterpret_cast<const void*>(&bmx_gateup_kernel<NW, CQ, CW, KM>), lds);          \
    hipLaunchKernelGGL((bmx_gateup_kernel<NW, CQ, CW, KM>), dim3(W.U * (a.I / (16 * NW))), dim3(NW * 64), lds, s, a); \
  } while (0)
#define GU_NW(CQ)                \
  do {                           \
    if (nw == 6) GU(6, CQ);      \
    else if (nw == 4) GU(4, CQ); \
    else GU(2, CQ);              \
  } while (0)
    if (chunks <= 4) GU_NW(4);
    else if (chunks <= 8) GU_NW(8);
    else if (chunks <= 16) GU_NW(16);
    else GU_NW(32);
#undef GU_NW
#undef GU
    return hipGetLastError();
  }
  {
    const int chunks = (a.I / kGroup + 3) / 4;
    const size_t lds = bmx_lds(a.I, KM);
    const int nw = a.H % 64 == 0 ? 4 : 2;
#define DN(NW, CQ)                                                                                  \
  do {                                                                                              \
    set_lds_limit(reinterpret_cast<const void*>(&bmx_down_kernel<NW, CQ, KM>), lds);                \
    hipLaunchKernelGGL((bmx_down_kernel<NW, CQ, KM>), dim3(W.U * (a.H / (16 * NW))), dim3(NW * 64), lds, s, a); \
  } while (0)
#define DN_NW(CQ)           \
  do {                      \
    if (nw == 4) DN(4, CQ); \
    else DN(2, CQ);         \
  } while (0)
    if (chunks <= 2) DN_NW(2);
    else if (chunks <= 4) DN_NW(4);
    else if (chunks <= 6) DN_NW(6);
    else if (chunks <= 8) DN_NW(8);
    else DN_NW(16);
#undef DN_NW
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
