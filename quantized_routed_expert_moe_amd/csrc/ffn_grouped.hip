// Prefill expert FFN: expert-grouped GEMMs on fp16 MFMA with LDS-staged int4
// weight tiles dequantised in registers.
//
// With many tokens per expert the FFN is a dense contraction per expert
// ("Strata on a Mac", Switches: the prompt's expert GEMMs), so it runs on the
// matrix cores:
//   1. plan (one workgroup): histogram of the T*K (token, rank) pairs by
//      expert, segment offsets, the list of M-tiles per unit (a unit is an
//      expert with its pairs, or the shared expert with every token), each
//      unit's blob address, and the scatter of pair indices into segments.
//      The order of pairs inside a segment does not matter: every output row
//      of an MFMA tile depends on its own A row only.
//   2. convert (the plan kernel's other workgroups, while the plan runs): x
//      (bf16) -> fp16 in the workspace. bf16 carries 8 significant
//      bits, so every |x| in [2^-17, 65504] converts exactly; smaller values
//      round to the fp16 subnormal grid (absolute error <= 2^-25), and a
//      value that would overflow fp16 sets MOE_EUNSUP in the status word
//      rather than being clamped.
//   3. gate/up GEMM (grouped_gemm_kernel<0>): tile = 128 pair rows x (128
//      gate + 128 up) weight rows, K = H in stages of 64 (two quantisation
//      groups). A rows are gathered from the fp16 x; the weights are staged
//      in LDS as int4 codes and B = fp16(q * s) is formed in registers right
//      before the MFMAs (q exact, one rounding of the product: relative error
//      <= 2^-11). v_mfma_f32_16x16x32_f16 with fp32 accumulation. The tile's
//      columns interleave gate and up in blocks of 16, so each lane holds
//      matching g and u and writes h = silu(g) * u in fp16 (the next A
//      operand; overflow sets the status word).
//   4. down GEMM (grouped_gemm_kernel<1>): A = h rows, B = fp16(q * s) of the
//      down matrix; o is written in fp16 at the pair's own index: one rounding
//      of relative error <= 2^-11 per routed term (bf16 would carry up to 2^-8
//      of the term's magnitude into y, more than a 2e-2 * rms bar absorbs when
//      the weighted terms are several times rms(y)); a value that does not
//      fit fp16 sets MOE_EUNSUP. fp16 halves the o bytes written here and
//      read by the combine (o is the largest buffer of a prompt layer).
//   5. combine: y[t] = o_shared[t] + sum_k w[t][k] * o[t][k] in rank order,
//      fp32, rounded once to bf16.
#include <type_traits>

#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = 128;  // rows of an M-tile (pairs of one unit)
constexpr int kGThreads = 256;
constexpr int kPlanThreads = 1024;

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct TileDesc {
  int unit, row0, rows, pad;
};

struct GroupedWs {
  size_t n_mt, tiles, ublob, unit_mt0, sorted, xh, h, o, bh, done, bytes;
  int max_units, max_mt;
};

// The pairs are counted and scattered by up to kHistBlocks workgroups, each a
// contiguous slice of at least kHistPairs pairs; the plan workgroup turns their
// counts into segment offsets and a base per (workgroup, expert).
constexpr int kHistBlocks = 64;
constexpr int kHistPairs = 2048;
__host__ __device__ inline int hist_blocks(size_t P) {
  const size_t nb = (P + kHistPairs - 1) / kHistPairs;
  return nb < 1 ? 1 : (nb > (size_t)kHistBlocks ? kHistBlocks : (int)nb);
}

// Partial passes (chunked paged prefill) record what they computed in the
// workspace: done[e] (e < E) = 1 once expert e was computed by a pass of the
// current chunk, done[E] the same for the shared expert, done[E + 1] = kSession
// from the chunk's first pass until the combine has run.
constexpr int32_t kSession = 0x50415254;

__host__ __device__ inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

__host__ __device__ inline GroupedWs grouped_ws(int T, int H, int I, int E, int K, int has_shared) {
  GroupedWs w;
  const size_t P = (size_t)T * K;
  const size_t PA = P + (has_shared ? T : 0);
  w.max_units = (int)((P < (size_t)E ? P : (size_t)E) + (has_shared ? 1 : 0));
  w.max_mt = (int)((PA + kBM - 1) / kBM) + w.max_units;
  w.n_mt = 0;  // int n_mt, int n_units
  w.tiles = al256(w.n_mt + 16);
  w.ublob = al256(w.tiles + (size_t)w.max_mt * sizeof(TileDesc));
  w.unit_mt0 = al256(w.ublob + (size_t)w.max_units * sizeof(void*));
  w.sorted = al256(w.unit_mt0 + ((size_t)w.max_units + 1) * sizeof(int32_t));
  w.xh = al256(w.sorted + PA * sizeof(int32_t));
  w.h = al256(w.xh + (size_t)T * H * 2);
  w.o = al256(w.h + PA * (size_t)I * 2);
  w.bh = al256(w.o + PA * (size_t)H * 2);  // o: fp16
  w.done = al256(w.bh + 2 * (size_t)kHistBlocks * E * sizeof(int32_t));  // bh: counts [NB][E], bases [NB][E]
  w.bytes = al256(w.done + ((size_t)E + 2) * sizeof(int32_t));
  return w;
}

// ------------------------------------------------------------------ plan
// Block-wide exclusive scan of one int per thread (kPlanThreads threads).
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) {
      const int s = wsum[w];
      wsum[w] = run;
      run += s;
    }
    *total = run;
  }
  __syncthreads();
  const int r = wsum[wave] + incl - v;
  __syncthreads();
  return r;
}

__device__ void convert_x_f16(const FfnArgs& a, size_t first, size_t stride);

// The pair slice of workgroup b of the histogram and scatter kernels.
__device__ inline void hist_slice(int P, int NB, int b, int* begin, int* end) {
  const int per = (P + NB - 1) / NB;
  *begin = b * per < P ? b * per : P;
  *end = *begin + per < P ? *begin + per : P;
}

// Workgroups 0 .. NB-1 count the experts of their slice of pairs (NB = hist_blocks);
// the others convert x to fp16 meanwhile.
__global__ void __launch_bounds__(kPlanThreads) grouped_hist_kernel(FfnArgs a) {
  const int T = a.T, K = a.K, E = a.E, P = T * K;
  const int NB = hist_blocks((size_t)P);
  if ((int)blockIdx.x >= NB) {
    convert_x_f16(a, (size_t)(blockIdx.x - NB) * kPlanThreads + threadIdx.x, (size_t)(gridDim.x - NB) * kPlanThreads);
    return;
  }
  __shared__ int cnt[kMaxE];
  const GroupedWs W = grouped_ws(T, a.H, a.I, E, K, a.shared_blob != nullptr);
  int32_t* bh = reinterpret_cast<int32_t*>(a.ws + W.bh);
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPlanThreads) cnt[e] = 0;
  __syncthreads();
  int p_begin, p_end;
  hist_slice(P, NB, blockIdx.x, &p_begin, &p_end);
  // eight pairs per thread and round, their ids loaded before any is used
  for (int p0 = p_begin + tid; p0 < p_end; p0 += 8 * kPlanThreads) {
    int ev[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + j * kPlanThreads;
      ev[j] = p < p_end ? a.ids[p] : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (p0 + j * kPlanThreads < p_end) {
        const int e = ev[j];
        if (e >= 0 && e < E)
          atomicAdd(&cnt[e], 1);
        else
          *a.status = MOE_EINVAL;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads) bh[blockIdx.x * E + e] = cnt[e];
}

// One workgroup: segments, tiles and unit records from the histogram workgroups'
// counts, and the base of every (histogram workgroup, expert) for the scatter.
__global__ void __launch_bounds__(kPlanThreads) grouped_plan_kernel(FfnArgs a) {
  __shared__ int cnt[kMaxE];
  __shared__ int wsum[kPlanThreads / 64];
  __shared__ int total;
  const int T = a.T, K = a.K, E = a.E;
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(T, a.H, a.I, E, K, has_shared);
  int* n_mt = reinterpret_cast<int*>(a.ws + W.n_mt);
  TileDesc* tiles = reinterpret_cast<TileDesc*>(a.ws + W.tiles);
  const uint8_t** ublob = reinterpret_cast<const uint8_t**>(a.ws + W.ublob);
  int32_t* unit_mt0 = reinterpret_cast<int32_t*>(a.ws + W.unit_mt0);
  int32_t* sorted = reinterpret_cast<int32_t*>(a.ws + W.sorted);
  const int tid = threadIdx.x;
  const int P = T * K;
  const int NB = hist_blocks((size_t)P);
  int32_t* bh = reinterpret_cast<int32_t*>(a.ws + W.bh);
  // expert e's count: the sum over the histogram workgroups (E <= kPlanThreads:
  // one expert per thread), sixteen loads in flight at a time
  {
    int c = 0;
    for (int b0 = 0; b0 < NB; b0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = (tid < E && b0 + j < NB) ? bh[(b0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) c += v[j];
    }
    if (tid < E) cnt[tid] = c;
  }
  __syncthreads();
  const int base_rows = has_shared ? T : 0;  // the shared unit's rows come first
  const int base_unit = has_shared ? 1 : 0;
  // thread e: segment start and unit index of expert e (experts in id order)
  // (every expert keeps its segment in a partial pass, so the rows of an expert, and with
  // them its results, are those of a full pass; an expert without a slot gets no tiles)
  const bool partial = a.mode & kModePartial;
  const bool do_shared = has_shared && (!partial || (a.mode & kModePartialShared));
  const int c = tid < E ? cnt[tid] : 0;
  const int slot = c > 0 ? a.slot_table[tid] : -1;
  const int row0 = block_exclusive_scan(c, wsum, &total) + base_rows;
  const int uidx = block_exclusive_scan(c > 0 ? 1 : 0, wsum, &total) + base_unit;
  const int n_units = total + base_unit;
  const int mt_here = (c > 0 && (slot >= 0 || !partial)) ? (c + kBM - 1) / kBM : 0;
  const int mt0 = block_exclusive_scan(mt_here, wsum, &total);
  const int shared_mt = do_shared ? (T + kBM - 1) / kBM : 0;
  if (partial) {
    // marks of what this pass computes; the chunk's first pass starts them afresh
    int32_t* done = reinterpret_cast<int32_t*>(a.ws + W.done);
    const bool first = a.mode & kModePartialFirst;
    const bool here = c > 0 && slot >= 0;
    if (tid < E && (first || here)) done[tid] = here ? 1 : 0;
    if (tid == 0) {
      if (first || do_shared) done[E] = do_shared ? 1 : 0;
      if (first) done[E + 1] = kSession;
    }
  }
  if (tid < E) {
    if (c > 0) {
      if (slot < 0 && !partial) *a.status = MOE_ENOTRES;
      ublob[uidx] = slot < 0 ? nullptr : a.slots + (size_t)slot * a.stride;
      unit_mt0[uidx] = shared_mt + mt0;
      for (int m = 0; m < mt_here; ++m) {
        const int rows = c - m * kBM < kBM ? c - m * kBM : kBM;
        tiles[shared_mt + mt0 + m] = TileDesc{uidx, row0 + m * kBM, rows, 0};
      }
    }
  }
  if (has_shared) {
    if (tid == 0) {
      ublob[0] = a.shared_blob;
      unit_mt0[0] = 0;
    }
    for (int m = tid; m < shared_mt; m += kPlanThreads) {
      const int rows = T - m * kBM < kBM ? T - m * kBM : kBM;
      tiles[m] = TileDesc{0, m * kBM, rows, 0};
    }
    for (int t = tid; t < T; t += kPlanThreads) sorted[t] = P + t;
  }
  if (tid == 0) {
    n_mt[0] = shared_mt + total;
    n_mt[1] = n_units;
    unit_mt0[n_units] = shared_mt + total;
  }
  // bases: histogram workgroup b places its pairs of expert e from the segment
  // start + the counts of workgroups 0 .. b-1 (sixteen counts loaded before their
  // bases are stored: a load after a store to the same array waits for it)
  if (tid < E) {
    int run = row0;
    for (int b0 = 0; b0 < NB; b0 += 16) {
      int v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = b0 + j < NB ? bh[(b0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        if (b0 + j < NB) bh[(kHistBlocks + b0 + j) * E + tid] = run;
        run += v[j];
      }
    }
  }
}

// Workgroup b (of hist_blocks) writes the pair indices of its slice into their
// experts' segments of `sorted`, from its bases; the order inside a segment
// follows the LDS atomics (any order serves, as every output row of a GEMM tile
// depends on its own A row only).
__global__ void __launch_bounds__(kPlanThreads) grouped_scatter_kernel(FfnArgs a) {
  __shared__ int cur[kMaxE];
  const int T = a.T, K = a.K, E = a.E, P = T * K;
  const int NB = hist_blocks((size_t)P);
  const GroupedWs W = grouped_ws(T, a.H, a.I, E, K, a.shared_blob != nullptr);
  const int32_t* base = reinterpret_cast<const int32_t*>(a.ws + W.bh) + (size_t)(kHistBlocks + blockIdx.x) * E;
  int32_t* sorted = reinterpret_cast<int32_t*>(a.ws + W.sorted);
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPlanThreads) cur[e] = base[e];
  __syncthreads();
  int p_begin, p_end;
  hist_slice(P, NB, blockIdx.x, &p_begin, &p_end);
  for (int p0 = p_begin + tid; p0 < p_end; p0 += 8 * kPlanThreads) {
    int ev[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + j * kPlanThreads;
      ev[j] = p < p_end ? a.ids[p] : -1;
    }
    int at[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = ev[j];
      at[j] = (e >= 0 && e < E) ? atomicAdd(&cur[e], 1) : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (at[j] >= 0) sorted[at[j]] = p0 + j * kPlanThreads;
  }
}

// ------------------------------------------------------------------ GEMM
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// x (bf16) to fp16 pairs in the workspace, by threads first .. first + stride - 1
// of a grid-stride loop over 16-byte pieces (T * H is a multiple of 8: H is a
// multiple of 64). Each round loads kConvRound pieces before it stores any: a
// load after a store would wait for it (the pointers might alias).
constexpr int kConvRound = 4;
__device__ void convert_x_f16(const FfnArgs& a, size_t first, size_t stride) {
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(a.T, a.H, a.I, a.E, a.K, has_shared);
  uint4* __restrict__ xh = reinterpret_cast<uint4*>(a.ws + W.xh);
  const size_t n8 = (size_t)a.T * a.H / 8;
  const uint4* __restrict__ xb = reinterpret_cast<const uint4*>(a.x);
  bool bad = false;
  for (size_t i0 = first; i0 < n8; i0 += stride * kConvRound) {
    uint4 v[kConvRound];
#pragma unroll
    for (int r = 0; r < kConvRound; ++r) {
      const size_t i = i0 + (size_t)r * stride;
      v[r] = xb[i < n8 ? i : 0];
    }
#pragma unroll
    for (int r = 0; r < kConvRound; ++r) {
      const size_t i = i0 + (size_t)r * stride;
      if (i >= n8) continue;
      const uint32_t d[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
      uint32_t o[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float lo = __uint_as_float(d[c] << 16), hi = __uint_as_float(d[c] & 0xFFFF0000u);
        bad |= !(fabsf(lo) < 65520.0f) || !(fabsf(hi) < 65520.0f);
        const f16x2 h = {(_Float16)lo, (_Float16)hi};
        o[c] = __builtin_bit_cast(uint32_t, h);
      }
      xh[i] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
  if (bad) *a.status = MOE_EUNSUP;
}

// SiLU of the prompt GEMMs' epilogue: z / (1 + e^-z) with the hardware base-2
// exponential and reciprocal (each within about 1 ulp of fp32), a few
// instructions instead of the library exp and the IEEE division; h is rounded
// to fp16 next (2^-11), far coarser than these errors. For z -> -inf the
// exponential overflows to +inf and the result is -0; z is a finite sum here.
__device__ inline float silu(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.44269504088896341f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ inline float f16_lo_f(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xFFFFu)); }
__device__ inline float f16_hi_f(uint32_t v) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16)); }

// MODE 0: gate/up with SwiGLU epilogue (writes h in segment order).
// MODE 1: down (writes o at the pair's index).
//
// Tile: 128 pair rows x 256 weight rows, K in stages of 64 (two quantisation
// groups). Wave w owns tile columns 64 w .. +63 for all 128 rows, so every
// dequantised B fragment feeds eight MFMAs (one per 16-row block). Every operand
// byte reaches LDS through buffer_load ... lds (no register staging, no LDS store
// instructions), three stages deep: while stage st is computed, the loads of
// stages st + 1 and st + 2 are in flight. Within a stage the order is fixed: per
// 16-row block four MFMAs, the A read two blocks ahead and a share of the next
// k-half's dequantisation (the second half's during the first, the next stage's
// first half during the second), so LDS latency and VALU work run under the
// MFMAs; the one barrier per stage sits between the two halves. A stage buffer holds the A rows (fp16,
// 16-byte chunks XOR-swizzled by row, which ds_read_b128 reaches without bank
// conflicts), the weight codes (int4, one 16-byte chunk per column and group,
// a quarter of their fp16 size) and the fp16 group scales. A lane dequantises
// the B operand of v_mfma_f32_16x16x32_f16 (8 consecutive k of one column) from
// one code dword: nibble pair p of the dword holds k 2p and 2p + 1 (bits 4p and
// 4p + 16); the pair OR-ed under an fp16 pattern gives 1024 + u (pairs 0, 2) or
// 64 + u (pairs 1, 3) exactly, a packed add of -1032 or -72 gives q, a packed
// multiply by the scale rounds q * s once. A tile with at most 64 rows computes
// only its first four 16-row blocks.
//
// Block -> tile: the n_mt * n_nt tiles are ordered (unit, N-tile, M-tile) and
// cut into 8 contiguous ranges, one per XCD (blocks are dispatched to XCDs
// round-robin by block id), so the M-tiles of one unit that share a weight
// N-tile run back to back on one XCD and meet its weight bytes in that XCD's
// L2.
constexpr int kTM = 128, kTN = 256, kTK = 64;

// Tile of this workgroup: the tiles, (unit, N-tile, M-tile) in order, are cut into
// 8 contiguous ranges, one per XCD (blocks go to XCDs round-robin by block id), so
// the M-tiles of one unit that share a weight N-tile run back to back in one L2.
// False for a block past the plan's tiles.
struct GemmTile {
  TileDesc td;
  const uint8_t* blob;
  int nt;
};
__device__ inline bool grouped_tile(const FfnArgs& a, const GroupedWs& W, int n_nt, GemmTile& g) {
  const int* cnts = reinterpret_cast<const int*>(a.ws + W.n_mt);
  const int n_mt = cnts[0], n_units = cnts[1];
  const int N = n_mt * n_nt;
  const int chunk = (N + 7) / 8;
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  if (jx >= chunk) return false;
  const int t = xcd * chunk + jx;
  if (t >= N) return false;
  const int32_t* unit_mt0 = reinterpret_cast<const int32_t*>(a.ws + W.unit_mt0);
  int lo = 0, hi = n_units - 1;  // last unit whose first tile index <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (unit_mt0[mid] * n_nt <= t)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int m_first = unit_mt0[lo], m_cnt = unit_mt0[lo + 1] - m_first;
  const int rr = t - m_first * n_nt;
  g.nt = rr / m_cnt;
  g.td = reinterpret_cast<const TileDesc*>(a.ws + W.tiles)[m_first + rr % m_cnt];
  g.blob = reinterpret_cast<const uint8_t* const*>(a.ws + W.ublob)[g.td.unit];
  return true;
}

template <int MODE>
__host__ __device__ inline int gemm_n_tiles(int H, int I) {
  return MODE == 0 ? (I + 127) / 128 : (H + kTN - 1) / kTN;
}

// One stage of operands in LDS (25,600 bytes).
struct __align__(16) GemmStage {
  _Float16 a[kTM * kTK];   // row r, chunk c (8 k) at r * 64 + 8 (c ^ (r & 7))
  uint32_t bc[2 * kTN * 4];  // group g, column c: code dwords at (g * 256 + c) * 4 .. +3
  uint16_t bs[2 * kTN];      // group g, column c: fp16 scale bits at g * 256 + c
};

template <int MODE>
__global__ void __launch_bounds__(kGThreads, 2) grouped_gemm_kernel(FfnArgs a) {
  // three stage buffers (separate objects, so that a stage can name the one it
  // reads and the one it fills)
  __shared__ GemmStage S0, S1, S2;
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(T, H, I, a.E, K, has_shared);
  const int n_nt = gemm_n_tiles<MODE>(H, I);
  GemmTile gt;
  if (!grouped_tile(a, W, n_nt, gt)) return;
  const TileDesc td = gt.td;
  const uint8_t* blob = gt.blob;
  const int nt = gt.nt;
  const int32_t* sorted = reinterpret_cast<const int32_t*>(a.ws + W.sorted);
  const int P = T * K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Kd = MODE == 0 ? H : I;  // reduced dimension
  const int G = Kd / kGroup;
  const int n_st = Kd / kTK;
  const bool half = td.rows <= 64;  // only the first four 16-row blocks hold pairs
  const BlobLayout BL = blob_layout(H, I);

  // Loaders (each lane keeps 32-bit byte offsets from wave-uniform bases, so a load
  // takes a scalar base and one offset register; the host checks that they fit;
  // named scalars rather than arrays: a private array indexed before unrolling
  // would be moved to LDS).
  // A: LDS chunk q = v * 256 + tid (v < 4) is row q / 8, position q % 8, which holds
  // columns 8 ((q % 8) ^ (row % 8)) .. +7; a wave fills 1 KB (8 rows), each row's 128
  // bytes read by eight consecutive lanes; a padding row reads the tile's first row
  // (its products are never stored).
  auto a_off = [&](int v) -> uint32_t {
    const int q = v * kGThreads + tid;
    int row = q >> 3;
    row = row < td.rows ? row : 0;
    const int col8 = ((q & 7) ^ ((q >> 3) & 7)) * 8;
    if (MODE == 0) {
      const int p = sorted[td.row0 + row];
      const int tok = p < P ? p / K : p - P;
      return ((uint32_t)tok * (uint32_t)H + col8) * 2u;
    }
    return ((uint32_t)(td.row0 + row) * (uint32_t)I + col8) * 2u;
  };
  const uint8_t* const a_base = a.ws + (MODE == 0 ? W.xh : W.h);
  const __amdgpu_buffer_rsrc_t a_rs =
      buf_rsrc(a_base, MODE == 0 ? (uint32_t)((size_t)T * H * 2) : (uint32_t)((W.o - W.h)));
  const uint32_t ao0 = a_off(0), ao1 = a_off(1), ao2 = a_off(2), ao3 = a_off(3);
  // B: tile column c -> weight row; past the last row of a partial tile a real row
  // (never stored). Codes: thread tid loads column tid's chunk of each group; scales:
  // thread tid loads the 4 bytes of columns 2 p, 2 p + 1 (p = tid % 128, an even and
  // the next row of one row block) of group tid / 128.
  const int R = MODE == 0 ? kRowBlockGU : kRowBlockDN;
  const int n_rows = MODE == 0 ? I : H;
  auto b_row = [&](int c, size_t& codes, size_t& scales) {
    int brow;
    if (MODE == 0) {
      const int mat = (c >> 4) & 1;  // gate and up alternate in blocks of 16 columns
      brow = nt * 128 + (c >> 5) * 16 + (c & 15);
      codes = mat ? BL.up_codes : BL.gate_codes;
      scales = mat ? BL.up_scales : BL.gate_scales;
    } else {
      brow = nt * kTN + c;
      codes = BL.down_codes;
      scales = BL.down_scales;
    }
    return brow;
  };
  const uint8_t* const b_base = blob ? blob : a.slots;  // any readable blob; its terms get scale 0
  uint32_t bco, bso;
  {
    size_t cb, sb;
    int brow = b_row(tid, cb, sb);
    brow = brow < n_rows ? brow : n_rows - 1;
    bco = (uint32_t)(cb + code_off(brow, 0, G, R));
    const int c2 = 2 * (tid & 127);
    brow = b_row(c2, cb, sb);
    brow = brow < n_rows - 1 ? brow : n_rows - 2;  // the pair stays inside the matrix
    bso = (uint32_t)(sb + scale_off(brow, (tid >> 7), G, R));
  }
  const __amdgpu_buffer_rsrc_t b_rs = buf_rsrc(b_base, (uint32_t)BL.bytes);
  const uint32_t scale_mask = blob ? 0xFFFFu : 0u;  // a unit without a blob contributes zeros
  // all operands of stage st into the stage buffer Sb (7 loads per lane: 4 A, 2 codes, 1 scale pair)
  auto issue = [&](int st, GemmStage* Sb) {
    const uint32_t sa = (uint32_t)st * (kTK * 2);
    ld16_lds(a_rs, ao0, sa, Sb->a + (0 * 4 + wave) * 512);
    ld16_lds(a_rs, ao1, sa, Sb->a + (1 * 4 + wave) * 512);
    ld16_lds(a_rs, ao2, sa, Sb->a + (2 * 4 + wave) * 512);
    ld16_lds(a_rs, ao3, sa, Sb->a + (3 * 4 + wave) * 512);
    const uint32_t sc = (uint32_t)st * 2 * R * 16;  // group 2 st, then 2 st + 1 (R * 16 bytes on)
    ld16_lds(b_rs, bco, sc, Sb->bc + (0 * kTN + wave * 64) * 4);
    ld16_lds(b_rs, bco, sc + R * 16, Sb->bc + (1 * kTN + wave * 64) * 4);
    ld4_lds(b_rs, bso, (uint32_t)st * 2 * R * 2, Sb->bs + wave * 128);
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Dequantisation constants, held in registers so that each AND-OR is one
  // v_and_or_b32: nibbles at bits 0..3 / 16..19 under 0x6400 give 1024 + u,
  // nibbles at bits 4..7 / 20..23 under 0x5400 give 64 + u (both exact), so one
  // shift by 8 serves all four pairs of a code dword.
  uint32_t k_mlo = 0x000F000Fu, k_mhi = 0x00F000F0u, k_elo = 0x64006400u, k_ehi = 0x54005400u;
  asm volatile("" : "+v"(k_mlo), "+v"(k_mhi), "+v"(k_elo), "+v"(k_ehi));
  const f16x2 off_lo = {(_Float16)-1032.0f, (_Float16)-1032.0f}, off_hi = {(_Float16)-72.0f, (_Float16)-72.0f};

  // one stage on stage buffer Sb; NB = 16-row blocks computed (8, or 4 for a half tile)
  auto dequant = [&](uint32_t cw, uint32_t sw) -> f16x8 {
    const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)sw);
    const f16x2 s2 = {sc, sc};
    const uint32_t w8 = cw >> 8;
    const uint32_t m0 = (cw & k_mlo) | k_elo, m1 = (cw & k_mhi) | k_ehi;
    const uint32_t m2 = (w8 & k_mlo) | k_elo, m3 = (w8 & k_mhi) | k_ehi;
    uint32_t bq[4];
    bq[0] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m0) + off_lo) * s2);
    bq[1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m1) + off_hi) * s2);
    bq[2] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m2) + off_lo) * s2);
    bq[3] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m3) + off_hi) * s2);
    return __builtin_bit_cast(f16x8, make_uint4(bq[0], bq[1], bq[2], bq[3]));
  };
  auto read_a = [&](const GemmStage* Sb, int h, int i) {  // row i 16 + lane % 16, chunk 4 h + lane / 16
    return *reinterpret_cast<const f16x8*>(
        &Sb->a[(i * 16 + (lane & 15)) * kTK + (((h * 4 + (lane >> 4)) ^ (lane & 7)) * 8)]);
  };
  const int colb = wave * 64 + (lane & 15);
  // B operands: raw code dwords and scales of one k-half (4 column blocks), then
  // their dequantised fragments; fbA = the first half of the stage being computed,
  // fbB = its second half
  uint32_t rc0, rc1, rc2, rc3, rs0, rs1, rs2, rs3;
  f16x8 fbA0, fbA1, fbA2, fbA3, fbB0, fbB1, fbB2, fbB3;
  auto read_b = [&](const GemmStage* Sb, int h) {
#define BLD(n)                                                          \
  rc##n = Sb->bc[(h * kTN + colb + n * 16) * 4 + (lane >> 4)]; \
  rs##n = Sb->bs[h * kTN + colb + n * 16] & scale_mask;
    BLD(0) BLD(1) BLD(2) BLD(3)
#undef BLD
  };
  f16x8 fa0, fa1;  // the next two A fragments

  using NB8 = std::integral_constant<int, 8>;
  using NB4 = std::integral_constant<int, 4>;
  auto sbuf = [&](int i) { return i == 0 ? &S0 : i == 1 ? &S1 : &S2; };
  // The stage loop, one copy per block count. Before it, stages 0 and 1 are loaded
  // and stage 0's first k-half dequantised (all loads waited for, so the compiler
  // sees none of them pending in the loop). Iteration st, with R, N and W the
  // buffers of stages st, st + 1 and st + 2 (st % 3 ...):
  //   part A: the first k-half's MFMAs of stage st (its B fragments were
  //     dequantised in iteration st - 1), with the second half's dequantisation
  //     and the A reads two blocks ahead under them;
  //   this wave's loads of stage st + 1 have landed; barrier: every wave's have,
  //     and every wave is done with stage st - 1, whose buffer W now receives
  //   the loads of stage st + 2 (past the last stage: the last stage again, so every
  //     iteration issues the same loads; nothing reads that copy);
  //   part B: the second half's MFMAs of stage st, with the first half of stage
  //     st + 1 read from N and dequantised under them.
  // The barrier sits between two runs of MFMAs, so the matrix unit is still busy
  // while the waves meet. The body takes the three buffers as restrict pointers, so
  // the compiler does not make the reads of R and N wait for the loads into W; the
  // waits are explicit.
  auto run = [&](auto NBC) {
    constexpr int NB = decltype(NBC)::value;
    issue(0, &S0);
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0) (gfx9 s_waitcnt encoding)
    __builtin_amdgcn_s_barrier();
    issue(n_st > 1 ? 1 : 0, &S1);
    read_b(&S0, 0);
    fbA0 = dequant(rc0, rs0);
    fbA1 = dequant(rc1, rs1);
    fbA2 = dequant(rc2, rs2);
    fbA3 = dequant(rc3, rs3);
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    __builtin_amdgcn_s_barrier();
    auto body = [&](int st, const GemmStage* __restrict__ Rb, const GemmStage* __restrict__ Nb,
                    GemmStage* __restrict__ Wb) {
      // part A
      read_b(Rb, 1);
      fa0 = read_a(Rb, 0, 0);
      fa1 = read_a(Rb, 0, 1);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const f16x8 fa = fa0;
        fa0 = fa1;
        fa1 = read_a(Rb, (i + 2) / NB, (i + 2) % NB);
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fbA0, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fbA1, acc[i][1], 0, 0, 0);
        acc[i][2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fbA2, acc[i][2], 0, 0, 0);
        acc[i][3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fbA3, acc[i][3], 0, 0, 0);
        // one fragment every other block (NB = 8) or every block (NB = 4)
        if (i == (NB == 8 ? 1 : 0)) fbB0 = dequant(rc0, rs0);
        if (i == (NB == 8 ? 3 : 1)) fbB1 = dequant(rc1, rs1);
        if (i == (NB == 8 ? 5 : 2)) fbB2 = dequant(rc2, rs2);
        if (i == (NB == 8 ? 7 : 3)) fbB3 = dequant(rc3, rs3);
        __builtin_amdgcn_sched_barrier(0);  // blocks in this order
      }
      __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
      __builtin_amdgcn_s_barrier();
      issue(st + 2 < n_st ? st + 2 : n_st - 1, Wb);
      __builtin_amdgcn_sched_barrier(0);
      // part B
      read_b(Nb, 0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const f16x8 fa = fa0;
        fa0 = fa1;
        if (i + 2 < NB) fa1 = read_a(Rb, 1, i + 2);
        acc[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fbB0, acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fbB1, acc[i][1], 0, 0, 0);
        acc[i][2] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fbB2, acc[i][2], 0, 0, 0);
        acc[i][3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fbB3, acc[i][3], 0, 0, 0);
        if (i == (NB == 8 ? 1 : 0)) fbA0 = dequant(rc0, rs0);
        if (i == (NB == 8 ? 3 : 1)) fbA1 = dequant(rc1, rs1);
        if (i == (NB == 8 ? 5 : 2)) fbA2 = dequant(rc2, rs2);
        if (i == (NB == 8 ? 7 : 3)) fbA3 = dequant(rc3, rs3);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    int rb = 0, nb = 1, wb = 2;  // buffer indices (st % 3, (st + 1) % 3, (st + 2) % 3)
    for (int st = 0; st < n_st; ++st) {
      body(st, sbuf(rb), sbuf(nb), sbuf(wb));
      __builtin_amdgcn_sched_barrier(0);
      const int t0 = rb;
      rb = nb;
      nb = wb;
      wb = t0;
    }
    // the last iteration's loads into LDS land before the wave can end (the
    // workgroup's LDS may be handed to another workgroup after that)
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
  };
  if (half)
    run(NB4{});
  else
    run(NB8{});

  // epilogue: lane holds D[row = 4 (lane / 16) + v][col = lane % 16] of each 16 x 16 block
  const int nb_live = half ? 4 : 8;
  if (MODE == 0) {
    uint16_t* hws = reinterpret_cast<uint16_t*>(a.ws + W.h);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col_i = nt * 128 + (wave * 2 + q) * 16 + (lane & 15);  // intermediate index
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = i * 16 + 4 * (lane >> 4) + v;
          if (i < nb_live && row < td.rows && col_i < I) {
            const float g = acc[i][2 * q][v], u = acc[i][2 * q + 1][v];
            const float hv = blob ? silu(g) * u : 0.0f;
            if (!(fabsf(hv) < 65520.0f)) *a.status = MOE_EUNSUP;  // h does not fit the fp16 operand
            hws[(size_t)(td.row0 + row) * I + col_i] = __builtin_bit_cast(uint16_t, (_Float16)hv);
          }
        }
      }
    }
  } else {
    _Float16* ows = reinterpret_cast<_Float16*>(a.ws + W.o);
    bool bad = false;
    // every row's pair index first, in one batch: loaded between the stores, each
    // load would wait for the stores before it (they might alias), 32 round trips
    int prow[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i * 16 + 4 * (lane >> 4) + v;
        prow[i][v] = sorted[td.row0 + (row < td.rows ? row : 0)];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i * 16 + 4 * (lane >> 4) + v;
        if (i < nb_live && row < td.rows) {
          const int p = prow[i][v];
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int col = nt * kTN + wave * 64 + n * 16 + (lane & 15);
            if (col < H) {
              const float ov = acc[i][n][v];
              bad |= !(fabsf(ov) < 65520.0f);  // o does not fit its fp16 store
              ows[(size_t)p * H + col] = (_Float16)ov;
            }
          }
        }
      }
    }
    if (bad) *a.status = MOE_EUNSUP;
  }
}

// ------------------------------------------------------------------ INT8 / NVFP4 GEMM
// The prompt path of the INT8 group-32 and NVFP4 experts ("Strata" README, the
// models table: INT8 group-32 linears; NVFP4 experts, E2M1 pairs, group-16 E4M3
// scales, an FP32 per-tensor global scale), on the same plan, fp16 x, fp16 o and
// combine as the int4 GEMM. Blob: fmt_layout (rows of codes, row-major, then the
// scales [rows][cols / g], then for NVFP4 the three global scales).
//
// Tile: 128 pair rows x 64 weight rows (MODE 0: rows of I in gate and in up;
// MODE 1: rows of H), K in stages of 64 columns. Wave w owns weight rows 16w ..
// 16w + 15 of the tile for all pair rows. The A rows (x or h, fp16) reach LDS by
// buffer-to-LDS loads, two stages deep, 16-byte chunks XOR-swizzled by row as in
// the int4 GEMM. Lane (n = lane % 16, q = lane / 16) streams columns 16q .. 16q
// + 15 of the stage of its weight row with one buffer load per matrix (int8: 16
// bytes, NVFP4: 8 bytes), one stage ahead; MFMA s (s = 0, 1) of a stage takes
// columns 16q + 8s .. +7 in quarter q, and the A fragment the same columns. B =
// int8: fp16(q * s) with one rounding: the codes (offset binary u = q + 128)
// become fp16 1024 + u by v_perm_b32 under a 0x64 byte, minus 1152, times the
// fp16 group scale; a scale of magnitude >= 512, whose product with a code could
// leave fp16, sets MOE_EUNSUP. NVFP4: e2m1 * e4m3 exactly (v_cvt_scalef32_pk_f16_fp4
// gives the code's exact fp16, the product of a 2-bit and a 4-bit significand is
// exact in fp16 and at most 6 * 448), the per-tensor global scale applied to the
// fp32 sums. Each 16-column run lies inside one scale group (int8: group
// (stage * 64 + 16q) / 32; NVFP4: stage * 4 + q).
constexpr int kFM = 128, kFN = 64, kFK = 64;

template <int FMT>
__device__ inline f16x8 fmt_dequant(uint32_t w0, uint32_t w1, _Float16 sc) {
  const f16x2 s2 = {sc, sc};
  uint32_t b[4];
  if constexpr (FMT == MOE_FMT_INT8_G32) {
    const f16x2 off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    // bytes [u0, 0x64, u1, 0x64] and [u2, 0x64, u3, 0x64] of each dword
    const uint32_t m0 = __builtin_amdgcn_perm(0x64646464u, w0, 0x04010400u);
    const uint32_t m1 = __builtin_amdgcn_perm(0x64646464u, w0, 0x04030402u);
    const uint32_t m2 = __builtin_amdgcn_perm(0x64646464u, w1, 0x04010400u);
    const uint32_t m3 = __builtin_amdgcn_perm(0x64646464u, w1, 0x04030402u);
    b[0] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m0) + off) * s2);
    b[1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m1) + off) * s2);
    b[2] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m2) + off) * s2);
    b[3] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m3) + off) * s2);
  } else {
    // w0: 8 E2M1 codes, byte i = columns 2i (low nibble), 2i + 1
    b[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0) * s2);
    b[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1) * s2);
    b[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2) * s2);
    b[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3) * s2);
    (void)w1;
  }
  return __builtin_bit_cast(f16x8, make_uint4(b[0], b[1], b[2], b[3]));
}

template <int FMT, int MODE>
__global__ void __launch_bounds__(kGThreads, 2) fmt_gemm_kernel(FfnArgs a) {
  __shared__ __align__(16) _Float16 As[2][kFM * kFK];
  constexpr bool kI8 = FMT == MOE_FMT_INT8_G32;
  constexpr int NM = MODE == 0 ? 2 : 1;  // matrices per tile
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(T, H, I, a.E, K, has_shared);
  GemmTile gt;
  if (!grouped_tile(a, W, MODE == 0 ? I / kFN : H / kFN, gt)) return;
  const TileDesc td = gt.td;
  const uint8_t* blob = gt.blob;
  const int32_t* sorted = reinterpret_cast<const int32_t*>(a.ws + W.sorted);
  const int P = T * K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, q = lane >> 4;
  const int Kd = MODE == 0 ? H : I;  // reduced dimension
  const int n_st = Kd / kFK;
  const int NB = td.rows <= 64 ? 4 : 8;  // 16-row blocks that hold pairs
  // A: LDS chunk c = v * 256 + tid (v < 4) is row c / 8, position c % 8, which holds
  // columns 8 ((c % 8) ^ (row % 8)) .. +7 of the stage; a padding row reads the
  // tile's first row (its products are never stored)
  auto a_off = [&](int v) -> uint32_t {
    const int c = v * kGThreads + tid;
    int row = c >> 3;
    row = row < td.rows ? row : 0;
    const int col8 = ((c & 7) ^ (row & 7)) * 8;
    if (MODE == 0) {
      const int p = sorted[td.row0 + row];
      const int tok = p < P ? p / K : p - P;
      return ((uint32_t)tok * (uint32_t)H + col8) * 2u;
    }
    return ((uint32_t)(td.row0 + row) * (uint32_t)I + col8) * 2u;
  };
  const __amdgpu_buffer_rsrc_t a_rs =
      buf_rsrc(a.ws + (MODE == 0 ? W.xh : W.h), MODE == 0 ? (uint32_t)((size_t)T * H * 2) : (uint32_t)((W.o - W.h)));
  const uint32_t ao0 = a_off(0), ao1 = a_off(1), ao2 = a_off(2), ao3 = a_off(3);
  auto issue_a = [&](int st, int buf) {
    const uint32_t sa = (uint32_t)st * (kFK * 2);
    _Float16* d = As[buf];
    ld16_lds(a_rs, ao0, sa, d + (0 * 4 + wave) * 512);
    ld16_lds(a_rs, ao1, sa, d + (1 * 4 + wave) * 512);
    ld16_lds(a_rs, ao2, sa, d + (2 * 4 + wave) * 512);
    ld16_lds(a_rs, ao3, sa, d + (3 * 4 + wave) * 512);
  };
  // B: this lane's weight row and its byte offsets within the blob
  const FmtLayout L = fmt_layout(FMT, H, I);
  const uint8_t* src = blob ? blob : a.slots;  // any readable blob; its terms get scale 0
  const __amdgpu_buffer_rsrc_t b_rs = buf_rsrc(src, (uint32_t)L.bytes);
  const int wr = gt.nt * kFN + wave * 16 + n;
  const uint32_t row_codes = kI8 ? (uint32_t)Kd : (uint32_t)Kd / 2, row_scales = kI8 ? Kd / 32 * 2 : Kd / 16;
  uint32_t co[NM], so[NM];
  float glob[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const size_t cb = MODE == 1 ? L.down_codes : (m == 0 ? L.gate_codes : L.up_codes);
    const size_t sb = MODE == 1 ? L.down_scales : (m == 0 ? L.gate_scales : L.up_scales);
    co[m] = (uint32_t)(cb + (size_t)wr * row_codes) + (uint32_t)q * (kI8 ? 16u : 8u);
    so[m] = (uint32_t)(sb + (size_t)wr * row_scales) + (kI8 ? (uint32_t)(q >> 1) * 2u : (uint32_t)q);
    glob[m] = 1.0f;
    if constexpr (!kI8) glob[m] = reinterpret_cast<const float*>(src + L.globals)[MODE == 1 ? 2 : m];
  }
  // per stage: codes advance 64 (int8) or 32 (NVFP4) bytes, scales 4 bytes
  uint4 cw[2][NM];
  uint32_t sw[2][NM];
  auto issue_b = [&](int st, auto bufc) {
    constexpr int buf = decltype(bufc)::value;  // a constant index: the buffers stay in registers
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if constexpr (kI8) {
        cw[buf][m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(b_rs, co[m], (uint32_t)st * 64u, 0));
        sw[buf][m] = __builtin_amdgcn_raw_buffer_load_b16(b_rs, so[m], (uint32_t)st * 4u, 0);
      } else {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(b_rs, co[m], (uint32_t)st * 32u, 0);
        cw[buf][m] = make_uint4((uint32_t)v[0], (uint32_t)v[1], 0u, 0u);
        sw[buf][m] = __builtin_amdgcn_raw_buffer_load_b8(b_rs, so[m], (uint32_t)st * 4u, 0);
      }
    }
  };
  f32x4 acc[NM][8];
#pragma unroll
  for (int m = 0; m < NM; ++m)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[m][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  auto scale_of = [&](uint32_t raw, int m) -> _Float16 {
    float sf;
    if constexpr (kI8) {
      sf = (float)__builtin_bit_cast(_Float16, (uint16_t)raw);
      if (blob && !(fabsf(sf) < 512.0f)) bad = true;
    } else {
      sf = __builtin_amdgcn_cvt_f32_fp8((int)raw, 0);  // exact in fp16 (E4M3 has 4 significant bits)
    }
    (void)m;
    return blob ? (_Float16)sf : (_Float16)0.0f;
  };
  // A fragment of block i, MFMA s: row 16 i + n, columns 16 q + 8 s .. +7 of the stage
  auto read_a = [&](int buf, int i, int s) {
    const int row = i * 16 + n, c = 2 * q + s;
    return *reinterpret_cast<const f16x8*>(&As[buf][row * kFK + ((c ^ (row & 7)) * 8)]);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  issue_a(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  issue_b(0, B0{});
  __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // vmcnt(0)
  __builtin_amdgcn_s_barrier();
  // stage st on buffer cur = st % 2 (stages in pairs, so the index is a constant)
  auto stage = [&](int st, auto curc) {
    constexpr int cur = decltype(curc)::value;
    if (st + 1 < n_st) {
      issue_a(st + 1, cur ^ 1);  // the other buffer: every wave finished reading it last stage
      __builtin_amdgcn_sched_barrier(0);
      issue_b(st + 1, std::integral_constant<int, cur ^ 1>{});
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const _Float16 sc = scale_of(sw[cur][m], m);
      const f16x8 b0 = fmt_dequant<FMT>(cw[cur][m].x, cw[cur][m].y, sc);
      const f16x8 b1 = kI8 ? fmt_dequant<FMT>(cw[cur][m].z, cw[cur][m].w, sc) : fmt_dequant<FMT>(cw[cur][m].y, 0u, sc);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i < NB) {
          acc[m][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(read_a(cur, i, 0), b0, acc[m][i], 0, 0, 0);
          acc[m][i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(read_a(cur, i, 1), b1, acc[m][i], 0, 0, 0);
        }
      }
    }
    // the next stage's A rows have landed (issued before its B loads), and every
    // wave is done with this stage's buffer
    if (st + 1 < n_st) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NM));
    __builtin_amdgcn_s_barrier();
  };
  for (int st = 0; st < n_st; st += 2) {
    stage(st, B0{});
    if (st + 1 < n_st) stage(st + 1, B1{});
  }
  // epilogue: lane holds D[row = 4 (lane / 16) + v][col = lane % 16] of each 16 x 16 block
  if (MODE == 0) {
    uint16_t* hws = reinterpret_cast<uint16_t*>(a.ws + W.h);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i * 16 + 4 * q + v;
        if (i < NB && row < td.rows) {
          const float g = acc[0][i][v] * glob[0], u = acc[NM - 1][i][v] * glob[NM - 1];
          const float hv = blob ? silu(g) * u : 0.0f;
          if (!(fabsf(hv) < 65520.0f)) bad = true;  // h does not fit the fp16 operand
          hws[(size_t)(td.row0 + row) * I + wr] = __builtin_bit_cast(uint16_t, (_Float16)hv);
        }
      }
    }
  } else {
    _Float16* ows = reinterpret_cast<_Float16*>(a.ws + W.o);
    // the rows' pair indices in one batch before the stores (as in the int4 GEMM)
    int prow[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i * 16 + 4 * q + v;
        prow[i][v] = sorted[td.row0 + (row < td.rows ? row : 0)];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i * 16 + 4 * q + v;
        if (i < NB && row < td.rows) {
          const float ov = acc[0][i][v] * glob[0];
          bad |= !(fabsf(ov) < 65520.0f);  // o does not fit its fp16 store
          ows[(size_t)prow[i][v] * H + wr] = (_Float16)ov;
        }
      }
    }
  }
  if (bad) *a.status = MOE_EUNSUP;
}

// ------------------------------------------------------------------ combine
// Thread: 8 consecutive columns of one token; the token's o rows (fp16, 16 bytes
// each) are loaded eight at a time before the sums, which run in rank order.
__global__ void __launch_bounds__(256) grouped_combine_kernel(FfnArgs a) {
  const int H = a.H, T = a.T, K = a.K;
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(T, H, a.I, a.E, K, has_shared);
  const uint4* o8 = reinterpret_cast<const uint4*>(a.ws + W.o);  // 8 fp16 per uint4
  const int P = T * K;
  const int H8 = H / 8;
  const size_t n8 = (size_t)T * H8;
  const bool check = a.mode & kModeCheckDone;
  const int32_t* done = reinterpret_cast<const int32_t*>(a.ws + W.done);
  if (check && blockIdx.x == 0 && threadIdx.x == 0 && done[a.E + 1] != kSession)
    *a.status = MOE_EINVAL;  // no first pass (MOE_FFN_PARTIAL_FIRST) since the last combine
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < n8; idx += (size_t)gridDim.x * 256) {
    const int t = (int)(idx / H8);
    const int c8 = (int)(idx % H8);
    if (check && c8 == 0) {
      // every pair of the token (and the shared term) must come from a pass of this chunk
      bool missing = has_shared && done[a.E] != 1;
      for (int k = 0; k < K; ++k) {
        const int e = a.ids[(size_t)t * K + k];
        missing |= e < 0 || e >= a.E || done[e] != 1;
      }
      if (missing) *a.status = MOE_ENOTRES;
    }
    float acc[8];
    if (has_shared) {
      const uint4 v = o8[(size_t)(P + t) * H8 + c8];
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[2 * e] = f16_lo_f(d[e]), acc[2 * e + 1] = f16_hi_f(d[e]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
    }
    for (int k0 = 0; k0 < K; k0 += 8) {
      uint4 ov[8];
      float wv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = k0 + j < K ? k0 + j : K - 1;
        ov[j] = o8[(size_t)(t * K + k) * H8 + c8];
        wv[j] = a.w[t * K + k];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (k0 + j < K) {
          const uint32_t d[4] = {ov[j].x, ov[j].y, ov[j].z, ov[j].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[2 * e] = fmaf(wv[j], f16_lo_f(d[e]), acc[2 * e]);
            acc[2 * e + 1] = fmaf(wv[j], f16_hi_f(d[e]), acc[2 * e + 1]);
          }
        }
      }
    }
    reinterpret_cast<uint4*>(a.y)[idx] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                    pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

inline int round8(int v) { return (v + 7) / 8 * 8; }

}  // namespace

bool grouped_shape_ok(int H, int I) { return H % kTK == 0 && I % kTK == 0; }  // H % 8 for the combine

// the GEMM addresses x and h with 32-bit byte offsets (and 32-bit buffer sizes,
// h's rounded up to 256 bytes)
static bool grouped_offsets_fit(int T, int H, int I, int K, int has_shared) {
  const size_t PA = (size_t)T * K + (has_shared ? (size_t)T : 0);
  return (size_t)T * H * 2 <= 0xFFFFFF00u && PA * I * 2 <= 0xFFFFFF00u;
}

// The plan in three launches: counts (with the fp16 conversion of x in the same
// grid, a 16-byte piece per thread and round, at most 256 workgroups), the
// one-workgroup plan, the scatter.
inline hipError_t launch_grouped_plan(const FfnArgs& a, hipStream_t s) {
  const int nb = hist_blocks((size_t)a.T * a.K);
  const size_t n8 = (size_t)a.T * a.H / 8;
  const size_t cb = (n8 + (size_t)kPlanThreads * kConvRound - 1) / ((size_t)kPlanThreads * kConvRound);
  hipLaunchKernelGGL(grouped_hist_kernel, dim3(nb + (int)(cb < 256 ? cb : 256)), dim3(kPlanThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(grouped_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(grouped_scatter_kernel, dim3(nb), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

size_t grouped_workspace_bytes(int T, int H, int I, int E, int K, int has_shared) {
  if (!grouped_offsets_fit(T, H, I, K, has_shared)) return 0;  // unsupported: the caller reports it
  return grouped_ws(T, H, I, E, K, has_shared).bytes;
}

hipError_t launch_ffn_grouped(const FfnArgs& a, int stage, hipStream_t s) {
  if (!grouped_shape_ok(a.H, a.I)) return hipErrorNotSupported;
  const bool has_shared = a.shared_blob != nullptr;
  if (!grouped_offsets_fit(a.T, a.H, a.I, a.K, has_shared)) return hipErrorNotSupported;
  const GroupedWs W = grouped_ws(a.T, a.H, a.I, a.E, a.K, has_shared);
  hipError_t e;
  if (stage == 0) {
    if ((e = launch_grouped_plan(a, s)) != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_gemm_kernel<0>), dim3(round8(W.max_mt * gemm_n_tiles<0>(a.H, a.I))), dim3(kGThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((grouped_gemm_kernel<1>), dim3(round8(W.max_mt * gemm_n_tiles<1>(a.H, a.I))), dim3(kGThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.mode & kModePartial) return hipSuccess;  // the caller combines after the last pass
  return launch_grouped_combine(a, s);
}

bool grouped_fmt_shape_ok(int H, int I) { return H % kFN == 0 && I % kFN == 0; }  // K stages and N tiles of 64

size_t grouped_fmt_workspace_bytes(int T, int H, int I, int E, int K, int has_shared) {
  return grouped_fmt_shape_ok(H, I) ? grouped_workspace_bytes(T, H, I, E, K, has_shared) : 0;
}

hipError_t launch_ffn_grouped_fmt(int fmt, const FfnArgs& a, hipStream_t s) {
  if (!grouped_fmt_shape_ok(a.H, a.I) || (fmt != MOE_FMT_INT8_G32 && fmt != MOE_FMT_NVFP4))
    return hipErrorNotSupported;
  const bool has_shared = a.shared_blob != nullptr;
  if (!grouped_offsets_fit(a.T, a.H, a.I, a.K, has_shared)) return hipErrorNotSupported;
  const GroupedWs W = grouped_ws(a.T, a.H, a.I, a.E, a.K, has_shared);
  hipError_t e;
  if ((e = launch_grouped_plan(a, s)) != hipSuccess) return e;
  const int g0 = round8(W.max_mt * (a.I / kFN)), g1 = round8(W.max_mt * (a.H / kFN));
  if (fmt == MOE_FMT_INT8_G32) {
    hipLaunchKernelGGL((fmt_gemm_kernel<MOE_FMT_INT8_G32, 0>), dim3(g0), dim3(kGThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((fmt_gemm_kernel<MOE_FMT_INT8_G32, 1>), dim3(g1), dim3(kGThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL((fmt_gemm_kernel<MOE_FMT_NVFP4, 0>), dim3(g0), dim3(kGThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((fmt_gemm_kernel<MOE_FMT_NVFP4, 1>), dim3(g1), dim3(kGThreads), 0, s, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return launch_grouped_combine(a, s);
}

hipError_t launch_grouped_combine(const FfnArgs& a, hipStream_t s) {
  const size_t n8 = (size_t)a.T * a.H / 8;
  // one output piece per thread where the grid allows: a thread's second piece
  // would load after its first store and wait for it (the buffers might alias)
  const size_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(grouped_combine_kernel, dim3(blocks < (1u << 20) ? (int)blocks : (1 << 20)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !(a.mode & kModeCheckDone)) return e;
  // close the chunk's session: the next chunk must start with a first pass
  const GroupedWs W = grouped_ws(a.T, a.H, a.I, a.E, a.K, a.shared_blob != nullptr);
  return launch_status(reinterpret_cast<int32_t*>(a.ws + W.done) + a.E + 1, nullptr, s);
}

}  // namespace moe
