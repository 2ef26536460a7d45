// Expert blob packing (host code): plain int4 interchange format -> device blob layout.
//
// The blob keeps one expert's three matrices in one contiguous allocation, the
// "one read per expert instead of three" layout of "Strata on a Mac" (What you
// need). Inside it, codes and scales are blocked by rows ([N/R][G][R][16
// bytes], R = 8 for gate/up and 4 for down) so that a kernel walking the
// groups of a row block reads one contiguous run, the
// nibbles are in offset binary (u = q + 8) and interleaved so that one shift and
// one mask turn a code dword into 16-bit pairs of consecutive columns. The
// layout is documented in moe_internal.h.
#include <string.h>

#include <cmath>
#include <utility>
#include <vector>

#include "moe_internal.h"

namespace {

// Source dword v holds 8 consecutive codes c0..c7 (byte b = codes 2b, 2b+1 in
// its low/high nibble, two's complement). Result: low nibbles of the 4 bytes
// (codes c0, c2, c4, c6) in nibbles 0..3, high nibbles (c1, c3, c5, c7) in
// nibbles 4..7, each converted to offset binary by flipping bit 3.
inline uint32_t interleave_dword(uint32_t v) {
  uint32_t lo = v & 0x0F0F0F0Fu;
  uint32_t hi = (v >> 4) & 0x0F0F0F0Fu;
  lo = (lo | (lo >> 4)) & 0x00FF00FFu;
  lo = (lo | (lo >> 8)) & 0x0000FFFFu;
  hi = (hi | (hi >> 4)) & 0x00FF00FFu;
  hi = (hi | (hi >> 8)) & 0x0000FFFFu;
  return (lo | (hi << 16)) ^ 0x88888888u;
}

void pack_matrix(const uint8_t* q, const uint16_t* s, int N, int C, int R, uint8_t* codes, uint16_t* scales) {
  const int G = C / moe::kGroup;
  const size_t row_bytes = (size_t)C / 2;
  for (int n = 0; n < N; ++n) {
    const uint8_t* row = q + (size_t)n * row_bytes;
    for (int j = 0; j < G; ++j) {
      uint32_t src[4], dst[4];
      memcpy(src, row + (size_t)j * 16, 16);
      for (int d = 0; d < 4; ++d) dst[d] = interleave_dword(src[d]);
      memcpy(codes + moe::code_off(n, j, G, R), dst, 16);
      scales[moe::chunk_index(n, j, G, R)] = s[(size_t)n * G + j];
    }
  }
}

}  // namespace

extern "C" size_t moe_blob_bytes(int H, int I, int g) {
  if (!moe::shape_ok(H, I, g)) return 0;
  return moe::blob_layout(H, I).bytes;
}

extern "C" size_t moe_slot_stride(int H, int I, int g) {
  const size_t b = moe_blob_bytes(H, I, g);
  return (b + 4095) / 4096 * 4096;
}

extern "C" int moe_pack_expert(const uint8_t* qg, const uint8_t* qu, const uint8_t* qd, const uint16_t* sg,
                               const uint16_t* su, const uint16_t* sd, int H, int I, int g, void* blob_out) {
  if (!qg || !qu || !qd || !sg || !su || !sd || !blob_out) return MOE_EINVAL;
  if (!moe::shape_ok(H, I, g)) return MOE_EUNSUP;
  const moe::BlobLayout L = moe::blob_layout(H, I);
  uint8_t* b = static_cast<uint8_t*>(blob_out);
  pack_matrix(qg, sg, I, H, moe::kRowBlockGU, b + L.gate_codes, reinterpret_cast<uint16_t*>(b + L.gate_scales));
  pack_matrix(qu, su, I, H, moe::kRowBlockGU, b + L.up_codes, reinterpret_cast<uint16_t*>(b + L.up_scales));
  pack_matrix(qd, sd, H, I, moe::kRowBlockDN, b + L.down_codes, reinterpret_cast<uint16_t*>(b + L.down_scales));
  return MOE_OK;
}

// ------------------------------------------------------------------ other formats
namespace {

// one matrix of N rows and C columns into the row-major layout of the formats
// blob (moe_internal.h, FmtLayout)
// int8 matrix of N rows and C columns into the row-major layout of the int8 blob
// (moe_internal.h, FmtLayout)
void pack_matrix_int8(const uint8_t* q, const uint16_t* s, int N, int C, uint8_t* codes, uint16_t* scales) {
  for (size_t i = 0; i < (size_t)N * C; ++i) codes[i] = (uint8_t)(q[i] ^ 0x80u);  // two's complement -> q + 128
  memcpy(scales, s, (size_t)N * (C / 32) * 2);
}

// group-128 scales [N][C/128] -> group-32 scales [N][C/32], each repeated for the
// four 32-column groups it covers (the same W[n][j] = q[n][j] * s[n][j / 128])
std::vector<uint16_t> repeat_scales(const uint16_t* s, int N, int C) {
  std::vector<uint16_t> out((size_t)N * (C / 32));
  for (size_t i = 0; i < out.size(); ++i) out[i] = s[i / 4];
  return out;
}

bool g128_shape_ok(int H, int I) { return H % 128 == 0 && I % 128 == 0 && moe::shape_ok(H, I, moe::kGroup); }

}  // namespace

extern "C" size_t moe_fmt_blob_bytes(int fmt, int H, int I) {
  if (fmt == MOE_FMT_INT4_G32) return moe_blob_bytes(H, I, moe::kGroup);
  if (fmt == MOE_FMT_INT4_G128) return g128_shape_ok(H, I) ? moe_blob_bytes(H, I, moe::kGroup) : 0;
  if (!moe::fmt_shape_ok(fmt, H, I)) return 0;
  return moe::fmt_layout(fmt, H, I).bytes;
}

extern "C" size_t moe_fmt_slot_stride(int fmt, int H, int I) {
  const size_t b = moe_fmt_blob_bytes(fmt, H, I);
  return (b + 4095) / 4096 * 4096;
}

extern "C" int moe_pack_expert_fmt(int fmt, const uint8_t* qg, const uint8_t* qu, const uint8_t* qd,
                                   const uint16_t* sg, const uint16_t* su, const uint16_t* sd, int H, int I,
                                   void* blob_out) {
  if (fmt == MOE_FMT_INT4_G32) return moe_pack_expert(qg, qu, qd, sg, su, sd, H, I, moe::kGroup, blob_out);
  if (fmt != MOE_FMT_INT4_G128 && fmt != MOE_FMT_INT8_G32) return MOE_EINVAL;  // NVFP4: moe_pack_expert_nvfp4
  if (!qg || !qu || !qd || !sg || !su || !sd || !blob_out) return MOE_EINVAL;
  if (fmt == MOE_FMT_INT4_G128) {  // the group-32 blob with repeated scales
    if (!g128_shape_ok(H, I)) return MOE_EUNSUP;
    const std::vector<uint16_t> g = repeat_scales(sg, I, H), u = repeat_scales(su, I, H), d = repeat_scales(sd, H, I);
    return moe_pack_expert(qg, qu, qd, g.data(), u.data(), d.data(), H, I, moe::kGroup, blob_out);
  }
  if (!moe::fmt_shape_ok(fmt, H, I)) return MOE_EUNSUP;
  const moe::FmtLayout L = moe::fmt_layout(fmt, H, I);
  uint8_t* b = static_cast<uint8_t*>(blob_out);
  memset(b, 0, L.bytes);  // padding between regions
  pack_matrix_int8(qg, sg, I, H, b + L.gate_codes, reinterpret_cast<uint16_t*>(b + L.gate_scales));
  pack_matrix_int8(qu, su, I, H, b + L.up_codes, reinterpret_cast<uint16_t*>(b + L.up_scales));
  pack_matrix_int8(qd, sd, H, I, b + L.down_codes, reinterpret_cast<uint16_t*>(b + L.down_scales));
  return MOE_OK;
}

extern "C" int moe_pack_expert_nvfp4(const uint8_t* qg, const uint8_t* qu, const uint8_t* qd, const uint8_t* sg,
                                     const uint8_t* su, const uint8_t* sd, const float* global3, int H, int I,
                                     void* blob_out) {
  if (!qg || !qu || !qd || !sg || !su || !sd || !global3 || !blob_out) return MOE_EINVAL;
  if (!moe::fmt_shape_ok(MOE_FMT_NVFP4, H, I)) return MOE_EUNSUP;
  for (int m = 0; m < 3; ++m)
    if (!std::isfinite(global3[m])) return MOE_EINVAL;
  const size_t n_gu = (size_t)I * (H / 16), n_dn = (size_t)H * (I / 16);
  for (const auto& sc : {std::make_pair(sg, n_gu), std::make_pair(su, n_gu), std::make_pair(sd, n_dn)})
    for (size_t i = 0; i < sc.second; ++i)
      if ((sc.first[i] & 0x7Fu) == 0x7Fu) return MOE_EINVAL;  // the E4M3 NaN
  const moe::FmtLayout L = moe::fmt_layout(MOE_FMT_NVFP4, H, I);
  uint8_t* b = static_cast<uint8_t*>(blob_out);
  memset(b, 0, L.bytes);
  memcpy(b + L.gate_codes, qg, (size_t)I * H / 2);  // E2M1 pairs as delivered
  memcpy(b + L.up_codes, qu, (size_t)I * H / 2);
  memcpy(b + L.down_codes, qd, (size_t)H * I / 2);
  memcpy(b + L.gate_scales, sg, n_gu);
  memcpy(b + L.up_scales, su, n_gu);
  memcpy(b + L.down_scales, sd, n_dn);
  memcpy(b + L.globals, global3, 12);
  return MOE_OK;
}
