// Internal declarations shared by the host entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr int kGroup = 32;      // int4 quantisation group along the reduced dimension
constexpr int kRowBlockGU = 8;  // rows per block of the gate and up matrices in the blob
constexpr int kRowBlockDN = 4;  // rows per block of the down matrix in the blob
constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kGemvMaxT = 32;   // default path choice: GEMV for T <= 32, grouped MFMA above

// Blob layout of one expert (all offsets in bytes from the blob start).
//   codes of gate, up, down, then scales of gate, up, down.
// Codes of a matrix with N rows and C reduced columns (G = C / 32 groups), in
//   blocks of R rows (R = 8 for gate and up, 4 for down): [N/R][G][R][16 bytes];
//   the 16-byte chunk of (row n, group j) is chunk ((n/R)*G + j)*R + n%R, so a
//   block of R rows is one contiguous run and 1 KB of it covers R rows of
//   64/R consecutive groups (one wave-wide load). The chunk holds the 32 codes
//   of columns 32j .. 32j+31 as four dwords; dword d covers columns c0 = 32j +
//   8d .. c0+7 with nibble i (bits 4i..4i+3) = column c0 + 2i for i < 4 and
//   c0 + 2(i-4) + 1 for i >= 4; each nibble is the offset-binary code u = q + 8.
// Scales: [N/R][G][R] fp16, scale of (row n, group j) at ((n/R)*G + j)*R + n%R
//   (the same index as the code chunk).
struct BlobLayout {
  size_t gate_codes, up_codes, down_codes, gate_scales, up_scales, down_scales, bytes;
};

__host__ __device__ inline BlobLayout blob_layout(int H, int I) {
  BlobLayout L;
  const size_t mat_codes = (size_t)H * I / 2;
  const size_t mat_scales = (size_t)H * I / kGroup * 2;
  L.gate_codes = 0;
  L.up_codes = mat_codes;
  L.down_codes = 2 * mat_codes;
  L.gate_scales = 3 * mat_codes;
  L.up_scales = L.gate_scales + mat_scales;
  L.down_scales = L.up_scales + mat_scales;
  L.bytes = L.down_scales + mat_scales;
  return L;
}

// Blob of the int8 group-32 and NVFP4 formats (moe_pack_expert_fmt,
// moe_pack_expert_nvfp4; the kernels in ffn_formats.hip): per matrix the rows
// one after another (int8 codes in column order, offset binary u = q + 128;
// NVFP4: two E2M1 codes per byte, the even column in the low nibble), then the
// scales [rows][cols / g] (int8: fp16, g = 32; NVFP4: E4M3 bytes, g = 16), then
// (NVFP4) the fp32 global scales of gate, up and down; every region starts on
// 256 bytes.
struct FmtLayout {
  size_t gate_codes, up_codes, down_codes, gate_scales, up_scales, down_scales, globals, bytes;
};
__host__ __device__ inline FmtLayout fmt_layout(int fmt, int H, int I) {
  const bool nv = fmt == MOE_FMT_NVFP4;
  const int bits = nv ? 4 : 8, g = nv ? 16 : 32, sb = nv ? 1 : 2;
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t gu_codes = (size_t)I * H * bits / 8, dn_codes = (size_t)H * I * bits / 8;
  const size_t gu_scales = (size_t)I * (H / g) * sb, dn_scales = (size_t)H * (I / g) * sb;
  FmtLayout L;
  L.gate_codes = 0;
  L.up_codes = al(L.gate_codes + gu_codes);
  L.down_codes = al(L.up_codes + gu_codes);
  L.gate_scales = al(L.down_codes + dn_codes);
  L.up_scales = al(L.gate_scales + gu_scales);
  L.down_scales = al(L.up_scales + gu_scales);
  L.globals = al(L.down_scales + dn_scales);
  L.bytes = nv ? al(L.globals + 12) : L.globals;
  return L;
}
bool fmt_shape_ok(int fmt, int H, int I);
size_t fmt_workspace_bytes(int T, int H, int I, int K, int has_shared);

// Byte offset of the code chunk / the scale of (row n, group j) within a matrix
// of G groups stored in blocks of R rows.
__host__ __device__ inline size_t chunk_index(int n, int j, int G, int R) {
  return ((size_t)(n / R) * G + j) * R + n % R;
}
__host__ __device__ inline size_t code_off(int n, int j, int G, int R) { return chunk_index(n, j, G, R) * 16; }
__host__ __device__ inline size_t scale_off(int n, int j, int G, int R) { return chunk_index(n, j, G, R) * 2; }

__host__ __device__ inline bool shape_ok(int H, int I, int g) {
  return g == kGroup && H >= kGroup && I >= kGroup && H % kGroup == 0 && I % kGroup == 0 && H <= 65536 &&
         I <= 65536;
}

// ---- launchers (return a hipError_t) ----
hipError_t launch_router_gemv(const uint16_t* x, const float* wr, float* logits, int T, int H, int E,
                              hipStream_t s);
// score: MOE_SCORE_*; bias (nullable) and scale as in moe_route_scored
// slot_table / slots_out (softmax scoring, T = 1 only): also write slots_out[k] =
// slot_table[ids[k]]
hipError_t launch_route_select(const float* logits, int T, int E, int K, unsigned flags, int32_t* ids,
                               float* w, hipStream_t s, int score = MOE_SCORE_SOFTMAX, const float* bias = nullptr,
                               float scale = 1.0f, const int32_t* slot_table = nullptr, int32_t* slots_out = nullptr);

// One-pass routing (onepass.h): the hand-off region of one token's routing,
// 64-bit words [0] call number, [1 + e] logit of expert e, and kOnepassCopies
// copies of the slot of rank k at onepass_slot_word(E, k, c), each in a 128-byte
// line of its own: the gate/up workgroups of one expert poll copy (workgroup % 8),
// so about 1/8 of them share a line.
constexpr int kOnepassCopies = 8;
__host__ __device__ inline int onepass_slot_word(int E, int k, int c) {
  return ((1 + E + 15) & ~15) + 16 * (k * kOnepassCopies + c);
}
__host__ __device__ inline size_t onepass_region_bytes(int E, int K) {
  return ((size_t)onepass_slot_word(E, K, 0) * 8 + 255) & ~(size_t)255;
}
hipError_t launch_route_onepass(const uint16_t* x, const float* wr, float* logits, int H, int E, int K, unsigned flags,
                                int32_t* ids, float* w, uint64_t* words, int32_t* status, hipStream_t s);

struct FfnArgs {
  const uint16_t* x;
  const int32_t* ids;
  const float* w;
  int T, H, I, E, K;
  const int32_t* slot_table;
  const uint8_t* slots;
  size_t stride;
  const uint8_t* shared_blob;
  uint16_t* y;
  uint8_t* ws;
  size_t ws_bytes;
  int32_t* status;
  unsigned mode;  // kModePartial / kModePartialShared (grouped path only), else 0
  // single-token path only, else nullptr: slot of routed expert k (rank order),
  // already resolved through slot_table by the routing kernel
  const int32_t* pre_slots;
  // single-token down kernel after a one-pass route + gate/up dispatch: the
  // region whose call number it advances; else nullptr
  uint64_t* onepass;
  // batched path under moe_layer: the plan kernel selects the top-k from these
  // logits itself (writing ids and w) before it plans; else nullptr
  const float* route_logits;
  unsigned route_flags;  // MOE_ROUTE_RENORM
};
// The router side of moe_layer's one-pass single-token path.
struct OnepassRoute {
  const float* w_router;
  float* logits;
  int32_t* ids;  // ids and w written by the selector (FfnArgs ids / w are the same buffers)
  float* w;
  unsigned flags;  // MOE_ROUTE_RENORM
  uint64_t* words;
};
// one dispatch: router GEMV, selection and gate/up; then the down kernel
hipError_t launch_ffn_decode1_onepass(const FfnArgs& a, const OnepassRoute& r, hipStream_t s);
// A partial pass of the grouped path: only routed experts with a slot are
// computed (the others are skipped without error), the per-pair outputs stay in
// the workspace and y is not written; kModePartialShared: this pass also
// computes the shared expert; kModePartialFirst: the chunk's first pass (it
// resets the workspace's record of computed experts). kModeCheckDone (the
// combine of moe_ffn_combine): every pair must have been computed by a pass.
constexpr unsigned kModePartial = 1u, kModePartialShared = 2u, kModePartialFirst = 4u, kModeCheckDone = 8u;
hipError_t launch_grouped_combine(const FfnArgs& a, hipStream_t s);
// the other expert formats (ffn_formats.hip): gate/up, down and combine
hipError_t launch_ffn_fmt(int fmt, const FfnArgs& a, hipStream_t s);

// Each path launches in two stages: stage 0 = gate/up (h into the workspace),
// stage 1 = down + combine (y).
size_t gemv_workspace_bytes(int T, int H, int I, int K, int has_shared);
// single-token workspaces end with room for the K resolved slots (moe_layer)
size_t decode1_slots_offset(int H, int I, int K, int has_shared);
hipError_t launch_ffn_gemv(const FfnArgs& a, int stage, hipStream_t s);

// small-batch kernels (2 <= T <= 32, shapes batched_supported admits)
bool batched_supported(int T, int H, int I, int K);
// the batched plan kernel can also select the top-k (FfnArgs::route_logits) for E experts
bool batched_routes(int E);
size_t batched_workspace_bytes(int T, int H, int I, int E, int K, int has_shared);
hipError_t launch_ffn_batched(const FfnArgs& a, int stage, hipStream_t s);

// single-token decode kernels (a specialisation of the GEMV path)
bool decode1_supported(int T, int H, int I, int K, bool has_shared);
hipError_t launch_ffn_decode1(const FfnArgs& a, int stage, hipStream_t s);

size_t grouped_workspace_bytes(int T, int H, int I, int E, int K, int has_shared);
bool grouped_shape_ok(int H, int I);
hipError_t launch_ffn_grouped(const FfnArgs& a, int stage, hipStream_t s);
// INT8 group-32 / NVFP4 experts for prompts: the grouped plan, fp16 x, fp16 o and
// combine with the format's MFMA GEMM (H and I multiples of 64)
bool grouped_fmt_shape_ok(int H, int I);
size_t grouped_fmt_workspace_bytes(int T, int H, int I, int E, int K, int has_shared);
hipError_t launch_ffn_grouped_fmt(int fmt, const FfnArgs& a, hipStream_t s);

hipError_t launch_table_update(int32_t* table, const int32_t* idx, const int32_t* val, int n, hipStream_t s);
// one-thread status word kernel: src == nullptr clears *dst; otherwise a non-zero
// *src is copied into *dst if *dst is still zero (the first error is kept)
hipError_t launch_status(int32_t* dst, const int32_t* src, hipStream_t s);
// ids[0..n) to pinned host memory host[0..n), then host[n] = seq (system scope, released)
hipError_t launch_publish_ids(const int32_t* ids, int n, int32_t* host, int32_t seq, hipStream_t s);

#ifdef MOE_TIMELINE
// per-unit row buffers of the instrumented build (timeline.h, MOE_TL_UNIT)
bool tl_owns_route(int kernel);
bool tl_owns_decode(int kernel);
bool tl_owns_batched(int kernel);
hipError_t tl_read_route(int kernel, uint64_t* host, int blocks);
hipError_t tl_read_decode(int kernel, uint64_t* host, int blocks);
hipError_t tl_read_batched(int kernel, uint64_t* host, int blocks);
hipError_t tl_clear_route();
hipError_t tl_clear_decode();
hipError_t tl_clear_batched();
#endif

}  // namespace moe
