// Expert FFN for the INT8 group-32 and NVFP4 experts of the "Strata" README
// (Models: INT8 group-32 linears; NVFP4 experts, E2M1 pairs with group-16 E4M3
// scales and an FP32 per-tensor global scale; both with 16-bit activations):
// the same layer as moe_expert_ffn,
//   y[t] = shared(x[t]) + sum_k w[t][k] * FFN_{ids[t][k]}(x[t]),
//   FFN(x) = Wd (silu(Wg x) * (Wu x)),
//   int8:  W[n][j] = q[n][j] * s[n][j / 32]      (fp16 s),
//   NVFP4: W[n][j] = e2m1(c[n][j]) * e4m3(s[n][j / 16]) * global,
// for T <= 32. (INT4 group-128 experts need no kernel of their own: they are
// packed as group-32 blobs with repeated scales.)
//
// Blob (FmtLayout): gate codes [I] rows, up codes [I], down codes [H] rows, each
// row contiguous, then the scales [rows][cols / g] of the three matrices (and
// for NVFP4 the three fp32 global scales). int8 rows are 16-byte chunks of 16
// columns (offset binary u = q + 128, column order); NVFP4 rows are 16-byte
// chunks of 32 columns (two E2M1 codes per byte, the even column in the low
// nibble, as delivered).
//
// Dequantisation is exact and lives in the fp16 dot products. int8: the pairs
// (0x64 << 8 | u) = 1024 + u = q + 1152 come from one v_perm_b32 per two codes,
// and sum_c q_c x_c = D - 1152 sum_c x_c with the x sums per chunk staged once.
// NVFP4: v_cvt_scalef32_pk_f16_fp4 turns a code byte into the fp16 pair of its
// two columns (the E2M1 values are exact in fp16). Each group's dot product is
// scaled in fp32 by its scale (fp16, or E4M3 decoded exactly), and an NVFP4 row
// by its global scale. x (and
// h for the down projection) are staged as fp16 (a value past the fp16 range
// sets MOE_EUNSUP).
//
// Work: an expert's bytes are read once per token that uses it (the
// single-token decode reads each chosen expert once). Kernel 1: item = (pair,
// 8 rows of I), wave w the rows 2w, 2w + 1 of gate and up, lanes the chunks of
// a row; h = silu(g) * u in fp32, handed on rounded to fp16. Down and combine:
// for up to 9 units per token and h rows of up to 128 chunks one kernel, item =
// (token, 8 or 16 rows of H) over all of the token's units, y added in rank
// order and rounded once to bf16; otherwise item = (pair, 8 rows of H) with o
// in fp32, then the combine kernel in the same order. No atomics: the
// reduction order depends only on (T, K, the format).
#include "moe_internal.h"
#include "wave_ops.h"

namespace moe {
namespace {

constexpr int kFThreads = 256;
constexpr int kRowsPerItem = 8;

template <int FMT>
struct Fmt;
template <>
struct Fmt<MOE_FMT_INT8_G32> {
  static constexpr int kCols = 16;  // columns per 16-byte chunk
  static constexpr int kG = 32;     // columns per scale
};
template <>
struct Fmt<MOE_FMT_NVFP4> {
  static constexpr int kCols = 32;
  static constexpr int kG = 16;
};

// Byte SEL of w as E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
// no infinities, S.1111.111 is NaN and never stored) in fp32, exactly: gfx950's
// v_cvt_f32_fp8 decodes the OCP E4M3 format (checked on all 256 bytes against
// the format's definition).
template <int SEL>
__device__ inline float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

__host__ __device__ inline size_t fmt_al256(size_t v) { return (v + 255) & ~(size_t)255; }

struct FmtWs {
  size_t h, o, bytes;
};
__host__ __device__ inline FmtWs fmt_ws(int T, int H, int I, int K, int has_shared) {
  const size_t PA = (size_t)T * K + (has_shared ? T : 0);
  FmtWs w;
  w.h = 0;  // fp16 h [PA][I]
  w.o = fmt_al256(PA * I * 2);
  w.bytes = fmt_al256(w.o + PA * H * 4);
  return w;
}

// Blob of pair p (the shared expert for p >= T K), or nullptr with the status set.
__device__ inline const uint8_t* fmt_pair_blob(const FfnArgs& a, int p) {
  const int P = a.T * a.K;
  if (p >= P) return a.shared_blob;
  const int e = a.ids[p];
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

// Activation staging in two halves, so that a workgroup's weight loads are in
// flight while its activations are converted: act_load fetches one chunk of C
// activations into registers, act_stage writes them into xs as fp16 pairs and,
// per chunk, the sum of its fp16 values times the code offset 1152 (int8).
// Sources: bf16 x (converted, a value past the fp16 range sets MOE_EUNSUP) or
// the fp16 h that the gate/up kernel wrote (copied).
template <int FMT>
struct ActChunk {
  static constexpr int kWords = Fmt<FMT>::kCols * 2 / 16;  // 16-byte words per chunk of 16-bit values
  uint4 v[kWords];
};
static_assert(kFThreads == 256, "one activation chunk per thread covers 256 chunks");

// chunk c of the row at src (c is a real chunk)
template <int FMT>
__device__ inline void act_load(const uint16_t* src, int c, ActChunk<FMT>& ch) {
  const uint4* q = reinterpret_cast<const uint4*>(src + (size_t)c * Fmt<FMT>::kCols);
#pragma unroll
  for (int i = 0; i < ActChunk<FMT>::kWords; ++i) ch.v[i] = q[i];
}

// chunk c into xs (fp16 pairs of the row) and corr[c]
template <int FMT, bool F16>
__device__ inline void act_stage(const ActChunk<FMT>& ch, int c, uint32_t* xs, float* corr, bool* bad) {
  constexpr int C = Fmt<FMT>::kCols;
  const uint32_t* d = reinterpret_cast<const uint32_t*>(ch.v);  // the chunk's dwords, in order
  float ca = 0.0f;
#pragma unroll
  for (int j = 0; j < C; j += 2) {
    uint32_t hp;
    if constexpr (F16) {
      hp = d[j / 2];
    } else {
      const uint32_t b = d[j / 2];
      hp = to_f16_bits(__uint_as_float(b << 16), bad) | (to_f16_bits(__uint_as_float(b & 0xFFFF0000u), bad) << 16);
    }
    xs[(c * C + j) / 2] = hp;
    ca += f16_lo(hp) + f16_hi(hp);
  }
  corr[c] = FMT == MOE_FMT_INT8_G32 ? 1152.0f * ca : 0.0f;
}

// Workgroup barrier that orders LDS only: the weight loads still in flight are
// not waited for (a full fence would wait for every outstanding global load).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// NVFP4: the two groups' sums (columns 0..15 and 16..31 of the chunk). Byte b of
// a code dword holds columns 2b (low nibble) and 2b + 1; gfx950 converts it to
// the fp16 pair of those columns in one instruction (scale 1: the E4M3 and
// global scales are applied in fp32 to the group sums and the row).
__device__ inline void chunk_dot_nvfp4(const uint4& cw, const uint32_t* xp, float& d0, float& d1) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
  float d[2] = {0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // dword i: columns 8i .. 8i + 7
    const h2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 0);
    const h2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 1);
    const h2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 2);
    const h2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i], 1.0f, 3);
    d[i >> 1] = dot2h(__builtin_bit_cast(uint32_t, p0), xp[4 * i + 0], d[i >> 1]);
    d[i >> 1] = dot2h(__builtin_bit_cast(uint32_t, p1), xp[4 * i + 1], d[i >> 1]);
    d[i >> 1] = dot2h(__builtin_bit_cast(uint32_t, p2), xp[4 * i + 2], d[i >> 1]);
    d[i >> 1] = dot2h(__builtin_bit_cast(uint32_t, p3), xp[4 * i + 3], d[i >> 1]);
  }
  d0 = d[0];
  d1 = d[1];
}

// D for one 16-byte chunk against its fp16 activation pairs xp[0 .. C/2).
template <int FMT>
__device__ inline float chunk_dot(const uint4& cw, const uint32_t* xp) {
  static_assert(FMT == MOE_FMT_INT8_G32, "int8 codes here");
  const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
  float d = 0.0f;
  // bytes [b0, 0x64, b1, 0x64] and [b2, 0x64, b3, 0x64]: fp16 1024 + u of columns 4i .. 4i + 3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d = dot2h(__builtin_amdgcn_perm(0x64646464u, w[i], 0x04010400u), xp[2 * i], d);
    d = dot2h(__builtin_amdgcn_perm(0x64646464u, w[i], 0x04030402u), xp[2 * i + 1], d);
  }
  return d;
}

template <int FMT>
__host__ __device__ inline size_t row_bytes(int cols) {
  return (size_t)cols / Fmt<FMT>::kCols * 16;
}

// One wave: S row streams (codes rows, scale rows) over cols columns; lane l
// takes chunks l, l + 64, ... rows_load issues every code and scale load of the
// wave (codes with the non-temporal hint: an expert's weights are read once per
// token), rows_dot takes the dot products against the staged activations and
// returns them on every lane.
// (scales: fp16 [cols / 32] per row for int8, E4M3 bytes [cols / 16] for NVFP4)
typedef unsigned int FmtU32x4 __attribute__((ext_vector_type(4)));
template <int FMT, int S, int STEPS>
struct RowWords {
  uint4 cw[S][STEPS];
  uint32_t sr[S][STEPS];  // int8: the fp16 scale; NVFP4: the chunk's two E4M3 scales
};

template <int FMT, int S, int STEPS>
__device__ inline void rows_load(const uint8_t* const (&codes)[S], const uint8_t* const (&scales)[S], int cols,
                                 int lane, RowWords<FMT, S, STEPS>& rw) {
  constexpr int C = Fmt<FMT>::kCols;
  const int n_chunks = cols / C;
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int i = 0; i < STEPS; ++i) {
      int c = i * 64 + lane;
      c = c < n_chunks ? c : n_chunks - 1;  // a real chunk, scaled by 0 below
      const FmtU32x4 v = __builtin_nontemporal_load(reinterpret_cast<const FmtU32x4*>(codes[s] + (size_t)c * 16));
      rw.cw[s][i] = make_uint4(v.x, v.y, v.z, v.w);
      if (FMT == MOE_FMT_INT8_G32)
        rw.sr[s][i] = reinterpret_cast<const uint16_t*>(scales[s])[(size_t)c * C / Fmt<FMT>::kG];
      else
        rw.sr[s][i] = reinterpret_cast<const uint16_t*>(scales[s])[c];  // groups 2c, 2c + 1
    }
}

template <int FMT, int S, int STEPS>
__device__ inline void rows_dot(const RowWords<FMT, S, STEPS>& rw, int cols, const uint32_t* xs, const float* corr,
                                float scale_mask, int lane, float (&out)[S]) {
  constexpr int C = Fmt<FMT>::kCols;
  const int n_chunks = cols / C;
#pragma unroll
  for (int s = 0; s < S; ++s) out[s] = 0.0f;
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const int c = i * 64 + lane;
    const bool live = c < n_chunks;
    const int cc = live ? c : n_chunks - 1;
    const uint32_t* xp = xs + cc * (C / 2);
    const float k = live ? scale_mask : 0.0f;
    const float cr = corr[cc];
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if constexpr (FMT == MOE_FMT_INT8_G32) {
        const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)rw.sr[s][i]);
        out[s] = fmaf(sc * k, chunk_dot<FMT>(rw.cw[s][i], xp) - cr, out[s]);
      } else {
        float d0, d1;
        chunk_dot_nvfp4(rw.cw[s][i], xp, d0, d1);
        out[s] = fmaf(e4m3_to_f32<0>(rw.sr[s][i]) * k, d0, out[s]);
        out[s] = fmaf(e4m3_to_f32<1>(rw.sr[s][i]) * k, d1, out[s]);
      }
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s) out[s] = wave_sum_f32(out[s]);
}

template <int FMT, int STEPS>
__global__ void __launch_bounds__(kFThreads) fmt_gateup_kernel(FfnArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, K = a.K, P = a.T * a.K;
  uint32_t* xs = reinterpret_cast<uint32_t*>(smem);
  float* corr = reinterpret_cast<float*>(smem + (size_t)H * 2);
  const int n_rb = I / kRowsPerItem;
  const int p = blockIdx.x / n_rb, rb = blockIdx.x % n_rb;
  const int t = p < P ? p / K : p - P;
  // order of the loads: x (its chunk per thread), the pair's slot, every weight
  // load; x is converted into LDS while the weights stream
  // (every supported row has at most 256 chunks, one per thread: fmt_shape_ok)
  const int xc_i = (int)threadIdx.x < H / Fmt<FMT>::kCols ? (int)threadIdx.x : 0;
  ActChunk<FMT> xc;
  act_load<FMT>(a.x + (size_t)t * H, xc_i, xc);
  const uint8_t* blob = fmt_pair_blob(a, p);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const FmtLayout L = fmt_layout(FMT, H, I);
  const uint8_t* src = blob ? blob : a.slots;  // any readable blob; its terms get scale 0
  const int n0 = rb * kRowsPerItem + 2 * wave;
  const size_t rbytes = row_bytes<FMT>(H);
  const size_t sbytes = (size_t)H / Fmt<FMT>::kG * (FMT == MOE_FMT_INT8_G32 ? 2 : 1);  // scale bytes per row
  const uint8_t* const codes[4] = {src + L.gate_codes + n0 * rbytes, src + L.gate_codes + (n0 + 1) * rbytes,
                                   src + L.up_codes + n0 * rbytes, src + L.up_codes + (n0 + 1) * rbytes};
  const uint8_t* const scales[4] = {src + L.gate_scales + n0 * sbytes, src + L.gate_scales + (n0 + 1) * sbytes,
                                    src + L.up_scales + n0 * sbytes, src + L.up_scales + (n0 + 1) * sbytes};
  RowWords<FMT, 4, STEPS> rw;
  rows_load<FMT, 4, STEPS>(codes, scales, H, lane, rw);
  bool bad = false;
  if ((int)threadIdx.x < H / Fmt<FMT>::kCols) act_stage<FMT, false>(xc, threadIdx.x, xs, corr, &bad);
  lds_barrier();
  float r[4];
  rows_dot<FMT, 4, STEPS>(rw, H, xs, corr, blob ? 1.0f : 0.0f, lane, r);
  if (FMT == MOE_FMT_NVFP4) {  // per-tensor global scales of gate and up
    const float* gl = reinterpret_cast<const float*>(src + L.globals);
    const float gg = gl[0], gu = gl[1];
    r[0] *= gg;
    r[1] *= gg;
    r[2] *= gu;
    r[3] *= gu;
  }
  if (lane < 2) {  // h rounded to fp16 from its fp32 value, the operand of the down projection
    const float g = lane ? r[1] : r[0], u = lane ? r[3] : r[2];
    float hv = silu(g) * u;
    asm volatile("" : "+v"(hv));  // keeps the fp32 rounding of the product (no fused fp32->fp16 multiply)
    if (!(fabsf(hv) < 65520.0f)) bad = true;  // h does not fit fp16
    reinterpret_cast<_Float16*>(a.ws)[(size_t)p * I + n0 + lane] = (_Float16)hv;
  }
  if (bad) *a.status = MOE_EUNSUP;
}

template <int FMT, int STEPS>
__global__ void __launch_bounds__(kFThreads) fmt_down_kernel(FfnArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I;
  const bool has_shared = a.shared_blob != nullptr;
  const FmtWs W = fmt_ws(a.T, H, I, a.K, has_shared);
  uint32_t* hs = reinterpret_cast<uint32_t*>(smem);
  float* corr = reinterpret_cast<float*>(smem + (size_t)I * 2);
  const int n_rb = H / kRowsPerItem;
  const int p = blockIdx.x / n_rb, rb = blockIdx.x % n_rb;
  const int hc_i = (int)threadIdx.x < I / Fmt<FMT>::kCols ? (int)threadIdx.x : 0;
  ActChunk<FMT> hc;
  act_load<FMT>(reinterpret_cast<const uint16_t*>(a.ws + W.h) + (size_t)p * I, hc_i, hc);
  const uint8_t* blob = fmt_pair_blob(a, p);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const FmtLayout L = fmt_layout(FMT, H, I);
  const uint8_t* src = blob ? blob : a.slots;
  const int n0 = rb * kRowsPerItem + 2 * wave;
  const size_t rbytes = row_bytes<FMT>(I);
  const size_t sbytes = (size_t)I / Fmt<FMT>::kG * (FMT == MOE_FMT_INT8_G32 ? 2 : 1);
  const uint8_t* const codes[2] = {src + L.down_codes + n0 * rbytes, src + L.down_codes + (n0 + 1) * rbytes};
  const uint8_t* const scales[2] = {src + L.down_scales + n0 * sbytes, src + L.down_scales + (n0 + 1) * sbytes};
  RowWords<FMT, 2, STEPS> rw;
  rows_load<FMT, 2, STEPS>(codes, scales, I, lane, rw);
  if ((int)threadIdx.x < I / Fmt<FMT>::kCols) act_stage<FMT, true>(hc, threadIdx.x, hs, corr, nullptr);
  lds_barrier();
  float r[2];
  rows_dot<FMT, 2, STEPS>(rw, I, hs, corr, blob ? 1.0f : 0.0f, lane, r);
  if (FMT == MOE_FMT_NVFP4) {
    const float gd = reinterpret_cast<const float*>(src + L.globals)[2];
    r[0] *= gd;
    r[1] *= gd;
  }
  if (lane < 2) reinterpret_cast<float*>(a.ws + W.o)[(size_t)p * H + n0 + lane] = lane ? r[1] : r[0];
}

// Down projection and combine in one kernel for the decode sizes (U = K units,
// plus the shared expert, of at most kFusedUnits; h rows of at most 128 chunks):
// one item per (token, 4 RPW rows of H), wave w the rows RPW w .. RPW w + RPW - 1
// of every unit of the token, RPW = 4 when a row's h is one step of 64 chunks
// (NVFP4 at the decode shape: each workgroup's h staging then serves 16 rows),
// else 2 (the registers of two steps' loads for every unit). The h of all U units goes to LDS; every weight load of the wave is
// issued first (the units' slots before them). Each unit's sums are those of
// fmt_down_kernel, and y = o_shared + sum_k w[k] * o_k is added in rank order
// and rounded once, as fmt_combine_kernel does: the same bits.
constexpr int kFusedUnits = 9;

template <int FMT, int STEPS, int U>
__global__ void __launch_bounds__(kFThreads) fmt_down_fused_kernel(FfnArgs a) {
  constexpr int C = Fmt<FMT>::kCols;
  constexpr int CH = (U * 64 * STEPS + kFThreads - 1) / kFThreads;  // h chunks per thread, at most
  constexpr int RPW = STEPS == 1 ? 4 : 2, RPI = 4 * RPW;  // rows per wave, per item
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H, I = a.I, K = a.K, P = a.T * K;
  const bool has_shared = a.shared_blob != nullptr;
  const FmtWs W = fmt_ws(a.T, H, I, K, has_shared);
  const int n_chunks = I / C;
  uint32_t* hs = reinterpret_cast<uint32_t*>(smem);                   // [U][I / 2] fp16 pairs
  float* corr = reinterpret_cast<float*>(smem + (size_t)U * I * 2);  // [U][n_chunks]
  const int n_rb = H / RPI;
  const int t = blockIdx.x / n_rb, rb = blockIdx.x % n_rb;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // unit u: the shared expert first when present, then ranks 0 .. K-1 (the combine's order)
  auto pair_of = [&](int u) { return has_shared ? (u == 0 ? P + t : t * K + u - 1) : t * K + u; };
  const uint16_t* hg = reinterpret_cast<const uint16_t*>(a.ws + W.h);
  // 1. this thread's h chunks q = tid + 256 j of the U x n_chunks
  ActChunk<FMT> hc[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int q = (int)threadIdx.x + kFThreads * j;
    const int qq = q < U * n_chunks ? q : 0;
    act_load<FMT>(hg + (size_t)pair_of(qq / n_chunks) * I, qq % n_chunks, hc[j]);
  }
  // 2. the units' slots (ids, then the slot table), then every weight load
  int32_t eu[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int pu = pair_of(u);
    eu[u] = a.ids[pu < P ? pu : 0];
  }
  int32_t su[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool ok = eu[u] >= 0 && eu[u] < a.E;
    su[u] = a.slot_table[ok ? eu[u] : 0];
  }
  const FmtLayout L = fmt_layout(FMT, H, I);
  const int n0 = rb * RPI + RPW * wave;
  const size_t rbytes = row_bytes<FMT>(I);
  const size_t sbytes = (size_t)I / Fmt<FMT>::kG * (FMT == MOE_FMT_INT8_G32 ? 2 : 1);
  const uint8_t* src[U];
  bool live[U];
  RowWords<FMT, RPW, STEPS> rw[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool shared_u = has_shared && u == 0;
    const bool id_ok = eu[u] >= 0 && eu[u] < a.E;
    live[u] = shared_u || (id_ok && su[u] >= 0);
    if (!shared_u && !live[u]) *a.status = id_ok ? MOE_ENOTRES : MOE_EINVAL;
    src[u] = shared_u ? a.shared_blob : (live[u] ? a.slots + (size_t)su[u] * a.stride : a.slots);
    const uint8_t* codes[RPW];
    const uint8_t* scales[RPW];
#pragma unroll
    for (int rr = 0; rr < RPW; ++rr) {
      codes[rr] = src[u] + L.down_codes + (n0 + rr) * rbytes;
      scales[rr] = src[u] + L.down_scales + (n0 + rr) * sbytes;
    }
    rows_load<FMT, RPW, STEPS>(codes, scales, I, lane, rw[u]);
  }
  // 3. h into LDS while the weights stream
#pragma unroll
  for (int j = 0; j < CH; ++j) {
    const int q = (int)threadIdx.x + kFThreads * j;
    if (q < U * n_chunks) {
      const int u = q / n_chunks;
      act_stage<FMT, true>(hc[j], q % n_chunks, hs + (size_t)u * (I / 2), corr + (size_t)u * n_chunks, nullptr);
    }
  }
  lds_barrier();
  // 4. per unit, the sums of fmt_down_kernel; combined in rank order
  float acc[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) acc[rr] = 0.0f;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float r[RPW];
    rows_dot<FMT, RPW, STEPS>(rw[u], I, hs + (size_t)u * (I / 2), corr + (size_t)u * n_chunks, live[u] ? 1.0f : 0.0f,
                            lane, r);
    if (FMT == MOE_FMT_NVFP4) {
      const float gd = reinterpret_cast<const float*>(src[u] + L.globals)[2];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) r[rr] *= gd;
    }
    if (has_shared && u == 0) {
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) acc[rr] = r[rr];
    } else {
      const float wk = a.w[t * K + (has_shared ? u - 1 : u)];
#pragma unroll
      for (int rr = 0; rr < RPW; ++rr) acc[rr] = fmaf(wk, r[rr], acc[rr]);
    }
  }
  float out = acc[0];
#pragma unroll
  for (int rr = 1; rr < RPW; ++rr) out = lane == rr ? acc[rr] : out;
  if (lane < RPW) a.y[(size_t)t * H + n0 + lane] = __builtin_bit_cast(uint16_t, (__bf16)out);
}

__global__ void __launch_bounds__(256) fmt_combine_kernel(FfnArgs a) {
  const int H = a.H, T = a.T, K = a.K, P = T * K;
  const bool has_shared = a.shared_blob != nullptr;
  const FmtWs W = fmt_ws(T, H, a.I, K, has_shared);
  const float* o = reinterpret_cast<const float*>(a.ws + W.o);
  const size_t n = (size_t)T * H;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int t = (int)(i / H), c = (int)(i % H);
    float acc = has_shared ? o[(size_t)(P + t) * H + c] : 0.0f;
    for (int k = 0; k < K; ++k) acc = fmaf(a.w[t * K + k], o[(size_t)(t * K + k) * H + c], acc);
    a.y[i] = __builtin_bit_cast(uint16_t, (__bf16)acc);
  }
}

template <int FMT>
hipError_t launch_fmt(const FfnArgs& a, hipStream_t s) {
  constexpr int C = Fmt<FMT>::kCols;
  const bool has_shared = a.shared_blob != nullptr;
  const int PA = a.T * a.K + (has_shared ? a.T : 0);
  const int steps_gu = (a.H / C + 63) / 64, steps_dn = (a.I / C + 63) / 64;
  const size_t lds_gu = (size_t)a.H * 2 + (size_t)a.H / C * 4, lds_dn = (size_t)a.I * 2 + (size_t)a.I / C * 4;
  const int grid_gu = PA * (a.I / kRowsPerItem), grid_dn = PA * (a.H / kRowsPerItem);
#define GU(N)                                                                                     \
  do {                                                                                            \
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&fmt_gateup_kernel<FMT, N>),          \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_gu);           \
    hipLaunchKernelGGL((fmt_gateup_kernel<FMT, N>), dim3(grid_gu), dim3(kFThreads), lds_gu, s, a); \
  } while (0)
#define DN(N)                                                                                   \
  do {                                                                                          \
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&fmt_down_kernel<FMT, N>),          \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_dn);         \
    hipLaunchKernelGGL((fmt_down_kernel<FMT, N>), dim3(grid_dn), dim3(kFThreads), lds_dn, s, a); \
  } while (0)
  if (steps_gu == 1) GU(1);
  else if (steps_gu == 2) GU(2);
  else if (steps_gu <= 4) GU(4);
  else return hipErrorNotSupported;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int U = a.K + (has_shared ? 1 : 0);
  const size_t lds_fused = (size_t)U * a.I * 2 + (size_t)U * (a.I / C) * 4;
  if (U <= kFusedUnits && steps_dn <= 2 && lds_fused <= 96 * 1024) {
    const int grid_f = a.T * (a.H / (steps_dn == 1 ? 16 : 8));  // 4 RPW rows per item
#define FU(ST, UU)                                                                                          \
  case UU:                                                                                                  \
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&fmt_down_fused_kernel<FMT, ST, UU>),           \
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_fused);                  \
    hipLaunchKernelGGL((fmt_down_fused_kernel<FMT, ST, UU>), dim3(grid_f), dim3(kFThreads), lds_fused, s, a); \
    break;
#define FU_ALL(ST) \
  switch (U) { FU(ST, 1) FU(ST, 2) FU(ST, 3) FU(ST, 4) FU(ST, 5) FU(ST, 6) FU(ST, 7) FU(ST, 8) FU(ST, 9) }
    if (steps_dn == 1) {
      FU_ALL(1)
    } else {
      FU_ALL(2)
    }
#undef FU_ALL
#undef FU
    return hipGetLastError();
  }
  if (steps_dn == 1) DN(1);
  else if (steps_dn == 2) DN(2);
  else if (steps_dn <= 4) DN(4);
  else return hipErrorNotSupported;
#undef GU
#undef DN
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t n = (size_t)a.T * a.H;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(fmt_combine_kernel, dim3(blocks < 4096 ? (int)blocks : 4096), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool fmt_shape_ok(int fmt, int H, int I) {
  // at most 4 steps of 64 chunks per row (16 columns per chunk for int8, 32 for
  // NVFP4), whole chunks and groups, whole row blocks
  if (fmt == MOE_FMT_INT8_G32) return H > 0 && I > 0 && H % 32 == 0 && I % 32 == 0 && H <= 4096 && I <= 4096;
  if (fmt == MOE_FMT_NVFP4) return H > 0 && I > 0 && H % 32 == 0 && I % 32 == 0 && H <= 8192 && I <= 8192;
  return false;
}

size_t fmt_workspace_bytes(int T, int H, int I, int K, int has_shared) {
  return fmt_ws(T, H, I, K, has_shared).bytes;
}

hipError_t launch_ffn_fmt(int fmt, const FfnArgs& a, hipStream_t s) {
  if (!fmt_shape_ok(fmt, a.H, a.I)) return hipErrorNotSupported;
  return fmt == MOE_FMT_INT8_G32 ? launch_fmt<MOE_FMT_INT8_G32>(a, s) : launch_fmt<MOE_FMT_NVFP4>(a, s);
}

}  // namespace moe
