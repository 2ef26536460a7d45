// Prefill expert FFN: expert-grouped GEMMs on bf16 MFMA with LDS-staged
// dequantised weight tiles.
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
//   2. convert: x (bf16) -> fp16 in the workspace. bf16 carries 8 significant
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
//      down matrix; o is written in bf16 at the pair's own index (one
//      rounding, relative error <= 2^-9, of each routed term; bf16 rather than
//      fp16 because an expert's output row is not bounded by 65504).
//   5. combine: y[t] = o_shared[t] + sum_k w[t][k] * o[t][k] in rank order,
//      fp32, rounded once to bf16.
#include <type_traits>

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
  size_t n_mt, tiles, ublob, unit_mt0, sorted, xh, h, o, bytes;
  int max_units, max_mt;
};

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
  w.bytes = al256(w.o + PA * (size_t)H * 2);  // o: bf16
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

__global__ void __launch_bounds__(kPlanThreads) grouped_plan_kernel(FfnArgs a) {
  __shared__ int cnt[kMaxE];
  __shared__ int seg[kMaxE];
  __shared__ int cur[kMaxE];
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
  for (int e = tid; e < kMaxE; e += kPlanThreads) cnt[e] = 0;
  __syncthreads();
  // eight pairs per thread and round, their ids loaded before any is used
  for (int p0 = tid; p0 < P; p0 += 8 * kPlanThreads) {
    int ev[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + j * kPlanThreads;
      ev[j] = p < P ? a.ids[p] : 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (p0 + j * kPlanThreads < P) {
        const int e = ev[j];
        if (e >= 0 && e < E)
          atomicAdd(&cnt[e], 1);
        else
          *a.status = MOE_EINVAL;
      }
    }
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
  if (tid < E) {
    seg[tid] = row0;
    cur[tid] = 0;
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
  __syncthreads();
  for (int p0 = tid; p0 < P; p0 += 8 * kPlanThreads) {
    int ev[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + j * kPlanThreads;
      ev[j] = p < P ? a.ids[p] : -1;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e = ev[j];
      if (e >= 0 && e < E) sorted[seg[e] + atomicAdd(&cur[e], 1)] = p0 + j * kPlanThreads;
    }
  }
}

// ------------------------------------------------------------------ GEMM
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

__global__ void __launch_bounds__(256) to_f16_kernel(FfnArgs a) {
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(a.T, a.H, a.I, a.E, a.K, has_shared);
  uint32_t* xh = reinterpret_cast<uint32_t*>(a.ws + W.xh);
  const size_t n2 = (size_t)a.T * a.H / 2;
  const uint32_t* xb = reinterpret_cast<const uint32_t*>(a.x);
  bool bad = false;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n2; i += (size_t)gridDim.x * 256) {
    const uint32_t v = xb[i];
    const float lo = __uint_as_float(v << 16), hi = __uint_as_float(v & 0xFFFF0000u);
    bad |= !(fabsf(lo) < 65520.0f) || !(fabsf(hi) < 65520.0f);
    const f16x2 h = {(_Float16)lo, (_Float16)hi};
    xh[i] = __builtin_bit_cast(uint32_t, h);
  }
  if (bad) *a.status = MOE_EUNSUP;
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// MODE 0: gate/up with SwiGLU epilogue (writes h in segment order).
// MODE 1: down (writes o at the pair's index).
//
// Tile: 128 pair rows x 256 weight rows, K in stages of 64 (two quantisation
// groups). Wave w owns tile columns 64 w .. +63 for all 128 rows, so every
// dequantised B fragment feeds eight MFMAs (one per 16-row block). LDS holds,
// double buffered, the stage's A rows (fp16, rows padded to 144 bytes, which
// the lanes of a ds_read_b128 reach without bank conflicts) and the weights as
// int4 codes and fp16 scales, a quarter of their fp16 size. A lane
// dequantises the B operand of v_mfma_f32_16x16x32_f16 (8 consecutive k of
// one column) from one code dword: nibble pair p of the dword holds k 2p and
// 2p + 1 (bits 4p and 4p + 16); the pair OR-ed under an fp16 pattern gives
// 1024 + u (pairs 0, 2) or 64 + u (pairs 1, 3) exactly, a packed add of -1032
// or -72 gives q, a packed multiply by the scale rounds q * s once. The next stage's global loads are in flight while
// the current stage is computed (one barrier per stage). A tile with at most
// 64 rows computes only its first four 16-row blocks.
//
// Block -> tile: the n_mt * n_nt tiles are ordered (unit, N-tile, M-tile) and
// cut into 8 contiguous ranges, one per XCD (blocks are dispatched to XCDs
// round-robin by block id), so the M-tiles of one unit that share a weight
// N-tile run back to back on one XCD and meet its weight bytes in that XCD's
// L2.
constexpr int kTM = 128, kTN = 256, kTK = 64;
constexpr int kARow = kTK + 8;  // A row in LDS, fp16 elements (16 bytes of padding)

// Loads through the global address space. The blob addresses come from the
// workspace, so the compiler cannot tell they are global and would emit flat
// loads, which count against the LDS wait counter as well: every LDS wait of
// a stage would then also wait for the next stage's weights.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ inline uint4 ld_global16(const uint8_t* p) {
  const u32x4 v = *(const __attribute__((address_space(1))) u32x4*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ inline uint32_t ld_global2(const uint8_t* p) { return *(const __attribute__((address_space(1))) uint16_t*)(p); }

template <int MODE>
__host__ __device__ inline int gemm_n_tiles(int H, int I) {
  return MODE == 0 ? (I + 127) / 128 : (H + kTN - 1) / kTN;
}

// dword e of the 8 code dwords of LDS column c holds dword e ^ sw(c) of the
// column's two chunks: 16 lanes reading dword d of 16 consecutive columns meet
// 16 different banks; the four dwords of a chunk stay in its 16 bytes
__device__ inline int code_swz(int c) { return (c >> 2) & 3; }

template <int MODE>
__global__ void __launch_bounds__(kGThreads, 2) grouped_gemm_kernel(FfnArgs a) {
  __shared__ __align__(16) _Float16 As[2][kTM][kARow];
  __shared__ __align__(16) uint32_t Bc[2][kTN * 8];  // per column: 2 groups x 4 code dwords (swizzled)
  __shared__ uint32_t Bs[2][kTN];                    // per column: the 2 groups' fp16 scales
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(T, H, I, a.E, K, has_shared);
  const int n_nt = gemm_n_tiles<MODE>(H, I);
  const int* cnts = reinterpret_cast<const int*>(a.ws + W.n_mt);
  const int n_mt = cnts[0], n_units = cnts[1];
  const int N = n_mt * n_nt;
  const int chunk = (N + 7) / 8;
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  if (jx >= chunk) return;
  const int t = xcd * chunk + jx;
  if (t >= N) return;
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
  const int nt = rr / m_cnt, mt = m_first + rr % m_cnt;
  const TileDesc td = reinterpret_cast<const TileDesc*>(a.ws + W.tiles)[mt];
  const uint8_t* blob = reinterpret_cast<const uint8_t* const*>(a.ws + W.ublob)[td.unit];
  const int32_t* sorted = reinterpret_cast<const int32_t*>(a.ws + W.sorted);
  const int P = T * K;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int Kd = MODE == 0 ? H : I;  // reduced dimension
  const int G = Kd / kGroup;
  const int n_st = Kd / kTK;
  const bool half = td.rows <= 64;  // only the first four 16-row blocks hold pairs
  const BlobLayout BL = blob_layout(H, I);

  // Loaders. A: 16-byte chunk q = v * 256 + tid (v < 4) of the 128 x 64 stage is
  // row q / 8, columns 8 (q % 8) .. +7, so eight consecutive lanes fill one row's
  // 128 bytes in LDS and in memory; a padding row reads the tile's first row (its
  // products are never stored). B: chunk q = k * 256 + tid (k < 2) is tile column
  // q / 2, group q % 2 of the stage, so consecutive lanes fill consecutive 16 bytes.
  // (named scalars rather than arrays: a private array indexed before unrolling
  // would be moved to LDS)
  auto a_ptr = [&](int v) -> const _Float16* {
    const int q = v * kGThreads + tid;
    int row = q >> 3;
    row = row < td.rows ? row : 0;
    const int col8 = (q & 7) * 8;
    if (MODE == 0) {
      const int p = sorted[td.row0 + row];
      const int tok = p < P ? p / K : p - P;
      return reinterpret_cast<const _Float16*>(a.ws + W.xh) + (size_t)tok * H + col8;
    }
    return reinterpret_cast<const _Float16*>(a.ws + W.h) + (size_t)(td.row0 + row) * I + col8;
  };
  const _Float16* const a_src0 = a_ptr(0);
  const _Float16* const a_src1 = a_ptr(1);
  const _Float16* const a_src2 = a_ptr(2);
  const _Float16* const a_src3 = a_ptr(3);
  const int R = MODE == 0 ? kRowBlockGU : kRowBlockDN;
  // B chunk k: code chunk at bsrc + (2 st + g) * R * 16 bytes, scale at ssrc + (2 st + g) * R * 2
  struct BSrc {
    const uint8_t* codes;
    const uint8_t* scales;
  };
  auto b_src = [&](int k) -> BSrc {
    const int q = k * kGThreads + tid;
    const int c = q >> 1;
    int brow;
    size_t bcodes, bscales;
    if (MODE == 0) {
      const int mat = (c >> 4) & 1;  // gate and up alternate in blocks of 16 columns
      brow = nt * 128 + (c >> 5) * 16 + (c & 15);
      brow = brow < I ? brow : I - 1;  // past the last row of a partial tile: a real row, never stored
      bcodes = mat ? BL.up_codes : BL.gate_codes;
      bscales = mat ? BL.up_scales : BL.gate_scales;
    } else {
      brow = nt * kTN + c;
      brow = brow < H ? brow : H - 1;
      bcodes = BL.down_codes;
      bscales = BL.down_scales;
    }
    const uint8_t* base = blob ? blob : a.slots;  // any readable blob; its terms get scale 0
    return BSrc{base + bcodes + code_off(brow, 0, G, R) + (size_t)(q & 1) * R * 16,
                base + bscales + scale_off(brow, 0, G, R) + (size_t)(q & 1) * R * 2};
  };
  const BSrc bs0 = b_src(0), bs1 = b_src(1);
  const int bcol0 = tid >> 1, bcol1 = (kGThreads + tid) >> 1;
  const uint32_t scale_mask = blob ? 0xFFFFu : 0u;  // a unit without a blob contributes zeros
  const int bg = tid & 1;                          // group of both B chunks of this thread

  uint4 ra0, ra1, ra2, ra3;  // A of the next stage
  uint4 rb0, rb1;            // B codes of the next stage
  uint32_t rs0, rs1;         // B scales of the next stage
  auto gload = [&](int st) {
    ra0 = *reinterpret_cast<const uint4*>(a_src0 + st * kTK);
    ra1 = *reinterpret_cast<const uint4*>(a_src1 + st * kTK);
    ra2 = *reinterpret_cast<const uint4*>(a_src2 + st * kTK);
    ra3 = *reinterpret_cast<const uint4*>(a_src3 + st * kTK);
    rb0 = ld_global16(bs0.codes + (size_t)st * 2 * R * 16);
    rb1 = ld_global16(bs1.codes + (size_t)st * 2 * R * 16);
    rs0 = ld_global2(bs0.scales + (size_t)st * 2 * R * 2) & scale_mask;
    rs1 = ld_global2(bs1.scales + (size_t)st * 2 * R * 2) & scale_mask;
  };
  // B chunk of column c into LDS: dword e of the chunk's 16 bytes holds code
  // dword e ^ code_swz(c), a permutation inside the chunk
  auto put_b = [&](int buf, int c, const uint4& w, uint32_t sc) {
    const int cs = code_swz(c);
    const uint32_t x = cs & 1 ? w.y : w.x, y = cs & 1 ? w.x : w.y;
    const uint32_t z = cs & 1 ? w.w : w.z, u = cs & 1 ? w.z : w.w;
    const uint4 o = cs & 2 ? make_uint4(z, u, x, y) : make_uint4(x, y, z, u);
    reinterpret_cast<uint4*>(&Bc[buf][c * 8])[bg] = o;
    reinterpret_cast<uint16_t*>(&Bs[buf][c])[bg] = (uint16_t)sc;
  };
  auto sstore = [&](int buf) {
    *reinterpret_cast<uint4*>(&As[buf][tid >> 3][(tid & 7) * 8]) = ra0;
    *reinterpret_cast<uint4*>(&As[buf][(kGThreads + tid) >> 3][(tid & 7) * 8]) = ra1;
    *reinterpret_cast<uint4*>(&As[buf][(2 * kGThreads + tid) >> 3][(tid & 7) * 8]) = ra2;
    *reinterpret_cast<uint4*>(&As[buf][(3 * kGThreads + tid) >> 3][(tid & 7) * 8]) = ra3;
    put_b(buf, bcol0, rb0, rs0);
    put_b(buf, bcol1, rb1, rs1);
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

  // one stage on LDS buffer buf; NB = 16-row blocks computed (8, or 4 for a half tile)
  auto compute = [&](auto NBC, int buf) {
    constexpr int NB = decltype(NBC)::value;
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // k-half = one quantisation group
      f16x8 fb[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const int col = wave * 64 + n * 16 + (lane & 15);
        const uint32_t cw = Bc[buf][col * 8 + h * 4 + ((lane >> 4) ^ code_swz(col))];
        const uint32_t sw = Bs[buf][col];
        const _Float16 sc = __builtin_bit_cast(_Float16, (uint16_t)(h ? sw >> 16 : sw));
        const f16x2 s2 = {sc, sc};
        const uint32_t w8 = cw >> 8;
        const uint32_t m0 = (cw & k_mlo) | k_elo, m1 = (cw & k_mhi) | k_ehi;
        const uint32_t m2 = (w8 & k_mlo) | k_elo, m3 = (w8 & k_mhi) | k_ehi;
        uint32_t bq[4];
        bq[0] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m0) + off_lo) * s2);
        bq[1] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m1) + off_hi) * s2);
        bq[2] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m2) + off_lo) * s2);
        bq[3] = __builtin_bit_cast(uint32_t, (__builtin_bit_cast(f16x2, m3) + off_hi) * s2);
        fb[n] = __builtin_bit_cast(f16x8, make_uint4(bq[0], bq[1], bq[2], bq[3]));
      }
      // A fragments one block ahead: block i + 1's is read before block i's MFMAs
      // are issued, so its LDS latency runs under them
      auto read_a = [&](int i) {
        return *reinterpret_cast<const f16x8*>(&As[buf][i * 16 + (lane & 15)][h * 32 + 8 * (lane >> 4)]);
      };
      f16x8 fa_next = read_a(0);
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const f16x8 fa = fa_next;
        if (i + 1 < NB) fa_next = read_a(i + 1);
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fb[n], acc[i][n], 0, 0, 0);
        asm volatile("" ::: "memory");  // no A fragment further ahead (register pressure)
      }
    }
  };

  using NB8 = std::integral_constant<int, 8>;
  using NB4 = std::integral_constant<int, 4>;
  // the stage loop, one copy per block count (one loop body each keeps the
  // register allocation simple)
  auto run = [&](auto NBC) {
    gload(0);
    sstore(0);
    __syncthreads();
    for (int st = 0; st < n_st; ++st) {
      const int buf = st & 1;
      // the next stage's loads (past the last stage: the last stage again, so the
      // count of loads in flight is the same on every path)
      gload(st + 1 < n_st ? st + 1 : st);
      compute(NBC, buf);
      sstore(buf ^ 1);  // buffer buf ^ 1 was last read in stage st - 1, before the barrier below it
      __syncthreads();
    }
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
    uint16_t* ows = reinterpret_cast<uint16_t*>(a.ws + W.o);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = i * 16 + 4 * (lane >> 4) + v;
        if (i < nb_live && row < td.rows) {
          const int p = sorted[td.row0 + row];
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int col = nt * kTN + wave * 64 + n * 16 + (lane & 15);
            if (col < H) ows[(size_t)p * H + col] = __builtin_bit_cast(uint16_t, (__bf16)acc[i][n][v]);
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ combine
// Thread: 8 consecutive columns of one token; every o row of the token is
// loaded (16 bytes each) before the sums, which run in rank order.
__device__ inline float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ inline float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__global__ void __launch_bounds__(256) grouped_combine_kernel(FfnArgs a) {
  const int H = a.H, T = a.T, K = a.K;
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(T, H, a.I, a.E, K, has_shared);
  const uint4* o8 = reinterpret_cast<const uint4*>(a.ws + W.o);  // 8 bf16 per uint4
  const int P = T * K;
  const int H8 = H / 8;
  const size_t n8 = (size_t)T * H8;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < n8; idx += (size_t)gridDim.x * 256) {
    const int t = (int)(idx / H8);
    const int c8 = (int)(idx % H8);
    float acc[8];
    {
      const uint4 v = has_shared ? o8[(size_t)(P + t) * H8 + c8] : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] = bf16_lo(d[e]);
        acc[2 * e + 1] = bf16_hi(d[e]);
      }
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
            acc[2 * e] = fmaf(wv[j], bf16_lo(d[e]), acc[2 * e]);
            acc[2 * e + 1] = fmaf(wv[j], bf16_hi(d[e]), acc[2 * e + 1]);
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

size_t grouped_workspace_bytes(int T, int H, int I, int E, int K, int has_shared) {
  return grouped_ws(T, H, I, E, K, has_shared).bytes;
}

hipError_t launch_ffn_grouped(const FfnArgs& a, int stage, hipStream_t s) {
  if (!grouped_shape_ok(a.H, a.I)) return hipErrorNotSupported;
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(a.T, a.H, a.I, a.E, a.K, has_shared);
  hipError_t e;
  if (stage == 0) {
    hipLaunchKernelGGL(grouped_plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const size_t n2 = (size_t)a.T * a.H / 2;
    const size_t cb = (n2 + 255) / 256;
    hipLaunchKernelGGL(to_f16_kernel, dim3(cb < 4096 ? (int)cb : 4096), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((grouped_gemm_kernel<0>), dim3(round8(W.max_mt * gemm_n_tiles<0>(a.H, a.I))), dim3(kGThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((grouped_gemm_kernel<1>), dim3(round8(W.max_mt * gemm_n_tiles<1>(a.H, a.I))), dim3(kGThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.mode & kModePartial) return hipSuccess;  // the caller combines after the last pass
  return launch_grouped_combine(a, s);
}

hipError_t launch_grouped_combine(const FfnArgs& a, hipStream_t s) {
  const size_t n8 = (size_t)a.T * a.H / 8;
  const size_t blocks = (n8 + 255) / 256;
  hipLaunchKernelGGL(grouped_combine_kernel, dim3(blocks < 8192 ? (int)blocks : 8192), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
