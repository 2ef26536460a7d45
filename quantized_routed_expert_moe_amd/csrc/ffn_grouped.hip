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
//   2. gate/up GEMM: tile = 128 pair rows x (64 gate + 64 up) weight rows,
//      K = H in steps of 64. A rows are gathered from x; B holds the int4 codes
//      q themselves, exact in bf16; both are staged in LDS and double
//      buffered. Each 32-wide K step is one quantisation group: one
//      v_mfma_f32_16x16x32_bf16 per 16x16 block gives the exact partial
//      sum_k x q in fp32, which is multiplied by the group's fp16 scale and
//      added to the fp32 accumulator. No rounding of the weights at all. The
//      tile's columns interleave gate and up in blocks of 16, so each lane
//      holds matching g and u and writes h = silu(g) * u as bf16 (the A
//      operand of the next GEMM).
//   3. down GEMM: A = h rows, B = down codes, same group scaling; o is written
//      in fp32 at the pair's own index.
//   4. combine: y[t] = o_shared[t] + sum_k w[t][k] * o[t][k] in rank order,
//      fp32, rounded once to bf16.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kGThreads = 256;
constexpr int kRowE = kBK + 8;  // LDS row length in bf16 (16 bytes of padding)
constexpr int kPlanThreads = 1024;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct TileDesc {
  int unit, row0, rows, pad;
};

struct GroupedWs {
  size_t n_mt, tiles, ublob, sorted, h, o, bytes;
  int max_units, max_mt;
};

__host__ __device__ inline size_t al256(size_t v) { return (v + 255) & ~(size_t)255; }

__host__ __device__ inline GroupedWs grouped_ws(int T, int H, int I, int E, int K, int has_shared) {
  GroupedWs w;
  const size_t P = (size_t)T * K;
  const size_t PA = P + (has_shared ? T : 0);
  w.max_units = (int)((P < (size_t)E ? P : (size_t)E) + (has_shared ? 1 : 0));
  w.max_mt = (int)((PA + kBM - 1) / kBM) + w.max_units;
  w.n_mt = 0;
  w.tiles = al256(w.n_mt + 16);
  w.ublob = al256(w.tiles + (size_t)w.max_mt * sizeof(TileDesc));
  w.sorted = al256(w.ublob + (size_t)w.max_units * sizeof(void*));
  w.h = al256(w.sorted + PA * sizeof(int32_t));
  w.o = al256(w.h + PA * (size_t)I * 2);
  w.bytes = al256(w.o + PA * (size_t)H * 4);
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
  int32_t* sorted = reinterpret_cast<int32_t*>(a.ws + W.sorted);
  const int tid = threadIdx.x;
  const int P = T * K;
  for (int e = tid; e < kMaxE; e += kPlanThreads) cnt[e] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += kPlanThreads) {
    const int e = a.ids[p];
    if (e >= 0 && e < E)
      atomicAdd(&cnt[e], 1);
    else
      *a.status = MOE_EINVAL;
  }
  __syncthreads();
  const int base_rows = has_shared ? T : 0;  // the shared unit's rows come first
  const int base_unit = has_shared ? 1 : 0;
  // thread e: segment start and unit index of expert e (experts in id order)
  const int c = tid < E ? cnt[tid] : 0;
  const int row0 = block_exclusive_scan(c, wsum, &total) + base_rows;
  const int uidx = block_exclusive_scan(c > 0 ? 1 : 0, wsum, &total) + base_unit;
  const int n_units = total + base_unit;
  const int mt_here = (c + kBM - 1) / kBM;
  const int mt0 = block_exclusive_scan(mt_here, wsum, &total);
  const int shared_mt = has_shared ? (T + kBM - 1) / kBM : 0;
  if (tid < E) {
    seg[tid] = row0;
    cur[tid] = 0;
    if (c > 0) {
      const int slot = a.slot_table[tid];
      if (slot < 0) *a.status = MOE_ENOTRES;
      ublob[uidx] = slot < 0 ? nullptr : a.slots + (size_t)slot * a.stride;
      for (int m = 0; m < mt_here; ++m) {
        const int rows = c - m * kBM < kBM ? c - m * kBM : kBM;
        tiles[shared_mt + mt0 + m] = TileDesc{uidx, row0 + m * kBM, rows, 0};
      }
    }
  }
  if (has_shared) {
    if (tid == 0) ublob[0] = a.shared_blob;
    for (int m = tid; m < shared_mt; m += kPlanThreads) {
      const int rows = T - m * kBM < kBM ? T - m * kBM : kBM;
      tiles[m] = TileDesc{0, m * kBM, rows, 0};
    }
    for (int t = tid; t < T; t += kPlanThreads) sorted[t] = P + t;
  }
  if (tid == 0) *n_mt = shared_mt + total;
  (void)n_units;
  __syncthreads();
  for (int p = tid; p < P; p += kPlanThreads) {
    const int e = a.ids[p];
    if (e >= 0 && e < E) sorted[seg[e] + atomicAdd(&cur[e], 1)] = p;
  }
}

// ------------------------------------------------------------------ GEMM
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// 32 codes of one (row, group) -> the 32 integer codes q = u - 8 as bf16 (exact),
// in column order.
__device__ inline void codes_to_bf16(uint4 codes, uint32_t out[16]) {
  const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t lo = cw[d] & 0x0F0F0F0Fu;
    const uint32_t hi = (cw[d] >> 4) & 0x0F0F0F0Fu;
    // columns 8d + {0..7}: lo.b0, lo.b2, hi.b0, hi.b2, lo.b1, lo.b3, hi.b1, hi.b3
    const float v0 = (float)(lo & 0xFF) - 8.0f;
    const float v1 = (float)((lo >> 16) & 0xFF) - 8.0f;
    const float v2 = (float)(hi & 0xFF) - 8.0f;
    const float v3 = (float)((hi >> 16) & 0xFF) - 8.0f;
    const float v4 = (float)((lo >> 8) & 0xFF) - 8.0f;
    const float v5 = (float)(lo >> 24) - 8.0f;
    const float v6 = (float)((hi >> 8) & 0xFF) - 8.0f;
    const float v7 = (float)(hi >> 24) - 8.0f;
    out[4 * d + 0] = pack_bf16x2(v0, v1);
    out[4 * d + 1] = pack_bf16x2(v2, v3);
    out[4 * d + 2] = pack_bf16x2(v4, v5);
    out[4 * d + 3] = pack_bf16x2(v6, v7);
  }
}

__device__ inline float silu(float z) { return z / (1.0f + expf(-z)); }

// MODE 0: gate/up with SwiGLU epilogue (writes h in segment order).
// MODE 1: down (writes o at the pair's index).
template <int MODE>
__global__ void __launch_bounds__(kGThreads) grouped_gemm_kernel(FfnArgs a) {
  __shared__ __align__(16) uint16_t As[2][kBM][kRowE];
  __shared__ __align__(16) uint16_t Bs[2][kBN][kRowE];
  __shared__ float Ss[2][kBK / kGroup][kBN];
  const int H = a.H, I = a.I, T = a.T, K = a.K;
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(T, H, I, a.E, K, has_shared);
  const int n_nt = MODE == 0 ? I / 64 : H / kBN;
  const int mt = blockIdx.x / n_nt, nt = blockIdx.x % n_nt;
  if (mt >= *reinterpret_cast<const int*>(a.ws + W.n_mt)) return;
  const TileDesc td = reinterpret_cast<const TileDesc*>(a.ws + W.tiles)[mt];
  const uint8_t* blob = reinterpret_cast<const uint8_t* const*>(a.ws + W.ublob)[td.unit];
  const int32_t* sorted = reinterpret_cast<const int32_t*>(a.ws + W.sorted);
  uint16_t* hws = reinterpret_cast<uint16_t*>(a.ws + W.h);
  float* ows = reinterpret_cast<float*>(a.ws + W.o);
  const int P = T * K;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int Kd = MODE == 0 ? H : I;  // reduced dimension
  const int G = Kd / kGroup;
  const int Nmat = MODE == 0 ? I : H;  // rows of the weight matrix
  const BlobLayout BL = blob_layout(H, I);

  // A loader: thread -> (row ar, 32-element half ah)
  const int ar = tid >> 1, ah = tid & 1;
  const bool a_ok = ar < td.rows && blob != nullptr;
  const uint16_t* a_src = nullptr;
  if (a_ok) {
    if (MODE == 0) {
      const int p = sorted[td.row0 + ar];
      const int t = p < P ? p / K : p - P;
      a_src = a.x + (size_t)t * H;
    } else {
      a_src = hws + (size_t)(td.row0 + ar) * I;
    }
  }
  // B loader: thread -> (tile column bc, group-in-stage bg)
  const int bc = tid & (kBN - 1), bg = tid >> 7;
  int brow;  // weight row
  size_t bcodes, bscales;
  if (MODE == 0) {
    const int mat = (bc >> 4) & 1;
    brow = nt * 64 + (bc >> 5) * 16 + (bc & 15);
    bcodes = mat ? BL.up_codes : BL.gate_codes;
    bscales = mat ? BL.up_scales : BL.gate_scales;
  } else {
    brow = nt * kBN + bc;
    bcodes = BL.down_codes;
    bscales = BL.down_scales;
  }

  uint4 ra[4];
  uint4 rb;
  _Float16 rs;
  auto gload = [&](int k0) {
    if (a_ok) {
#pragma unroll
      for (int v = 0; v < 4; ++v) ra[v] = reinterpret_cast<const uint4*>(a_src + k0 + 32 * ah)[v];
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) ra[v] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (blob) {
      const int j = k0 / kGroup + bg;
      rb = *reinterpret_cast<const uint4*>(blob + bcodes + ((size_t)j * Nmat + brow) * 16);
      rs = *reinterpret_cast<const _Float16*>(
          blob + bscales + (((size_t)(brow / kScaleBlock) * G + j) * kScaleBlock + brow % kScaleBlock) * 2);
    } else {
      rb = make_uint4(0x88888888u, 0x88888888u, 0x88888888u, 0x88888888u);
      rs = (_Float16)0.0f;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int v = 0; v < 4; ++v) reinterpret_cast<uint4*>(&As[buf][ar][32 * ah])[v] = ra[v];
    uint32_t deq[16];
    codes_to_bf16(rb, deq);
    Ss[buf][bg][bc] = (float)rs;
#pragma unroll
    for (int v = 0; v < 4; ++v)
      reinterpret_cast<uint4*>(&Bs[buf][bc][32 * bg])[v] = make_uint4(deq[4 * v], deq[4 * v + 1], deq[4 * v + 2], deq[4 * v + 3]);
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int n_st = Kd / kBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int st = 0; st < n_st; ++st) {
    const int buf = st & 1;
    if (st + 1 < n_st) gload((st + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 32; ++ks) {
      bf16x8 fa[4], fb[4];
      const int kk = ks * 32 + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(&As[buf][wm * 64 + i * 16 + (lane & 15)][kk]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(&Bs[buf][wn * 64 + j * 16 + (lane & 15)][kk]);
      float sc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) sc[j] = Ss[buf][ks][wn * 64 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // exact group partial sum_k a q, then the group's scale in fp32
          const f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[i][j][v] = fmaf(sc[j], part[v], acc[i][j][v]);
        }
    }
    if (st + 1 < n_st) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds D[row = 4*(lane/16) + v][col = lane%16] of each 16x16 block
  if (MODE == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int col_i = nt * 64 + (2 * wn + q) * 16 + (lane & 15);  // intermediate index
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int row = wm * 64 + i * 16 + 4 * (lane >> 4) + v;
          if (row < td.rows) {
            const float g = acc[i][2 * q][v], u = acc[i][2 * q + 1][v];
            const float hv = blob ? silu(g) * u : 0.0f;
            hws[(size_t)(td.row0 + row) * I + col_i] = __builtin_bit_cast(uint16_t, (__bf16)hv);
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = wm * 64 + i * 16 + 4 * (lane >> 4) + v;
        if (row < td.rows) {
          const int p = sorted[td.row0 + row];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = nt * kBN + wn * 64 + j * 16 + (lane & 15);
            ows[(size_t)p * H + n] = acc[i][j][v];
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ combine
__global__ void __launch_bounds__(256) grouped_combine_kernel(FfnArgs a) {
  const int H = a.H, T = a.T, K = a.K;
  const bool has_shared = a.shared_blob != nullptr;
  const GroupedWs W = grouped_ws(T, H, a.I, a.E, K, has_shared);
  const float* ows = reinterpret_cast<const float*>(a.ws + W.o);
  const int P = T * K;
  const size_t n4 = (size_t)T * H / 4;
  for (size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x; idx < n4; idx += (size_t)gridDim.x * 256) {
    const int t = (int)(idx / (H / 4));
    const int c4 = (int)(idx % (H / 4));
    float4 acc = has_shared ? reinterpret_cast<const float4*>(ows + (size_t)(P + t) * H)[c4]
                            : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < K; ++k) {
      const float wk = a.w[t * K + k];
      const float4 v = reinterpret_cast<const float4*>(ows + (size_t)(t * K + k) * H)[c4];
      acc.x = fmaf(wk, v.x, acc.x);
      acc.y = fmaf(wk, v.y, acc.y);
      acc.z = fmaf(wk, v.z, acc.z);
      acc.w = fmaf(wk, v.w, acc.w);
    }
    reinterpret_cast<uint2*>(a.y)[idx] = make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
  }
}

}  // namespace

bool grouped_shape_ok(int H, int I) { return H % kBN == 0 && I % 64 == 0 && H % kBK == 0; }

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
    hipLaunchKernelGGL((grouped_gemm_kernel<0>), dim3(W.max_mt * (a.I / 64)), dim3(kGThreads), 0, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((grouped_gemm_kernel<1>), dim3(W.max_mt * (a.H / kBN)), dim3(kGThreads), 0, s, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const size_t n4 = (size_t)a.T * a.H / 4;
  const size_t blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL(grouped_combine_kernel, dim3(blocks < 8192 ? (int)blocks : 8192), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
