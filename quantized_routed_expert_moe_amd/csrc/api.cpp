// C-ABI entry points: argument checks and dispatch to the HIP kernels.
//
// Exact or explicit failure ("Strata" README, execution rules: exact mode
// completes the exact computation or reports a failure; top-k and precision are
// never changed silently): every unsupported shape returns MOE_EUNSUP and no
// call falls back to another computation.
#include <cmath>

#include "moe_internal.h"
#include "moe_timeline.h"

namespace {

bool ffn_uses_grouped(int T, unsigned flags) {
  if (flags & MOE_FORCE_GEMV) return false;
  if (flags & (MOE_FORCE_GROUPED | MOE_FFN_PARTIAL)) return true;
  return T > moe::kGemvMaxT;
}

bool gemv_shape_ok(int T, int H, int I, int K) {
  // register-resident code slices: gate/up up to 16 groups per slice, down up to 16
  return T <= moe::kGemvMaxT && K <= moe::kMaxK && H <= 16 * 16 * moe::kGroup && I <= 16 * 8 * moe::kGroup;
}

}  // namespace

extern "C" const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK:
      return "ok";
    case MOE_EINVAL:
      return "invalid argument";
    case MOE_ENOSLOT:
      return "no free slot: more distinct experts requested than the arena has slots";
    case MOE_ENOTRES:
      return "an expert used by the layer is not resident in the arena";
    case MOE_EHIP:
      return "HIP runtime call or kernel launch failed";
    case MOE_EUNSUP:
      return "shape or option not supported by the kernels";
    case MOE_EWS:
      return "workspace missing or too small";
    default:
      return "unknown status";
  }
}

extern "C" int moe_version(void) { return 100; }

namespace {
// moe_route's argument checks, true when it would enqueue work (T > 0, valid arguments).
bool shape_ok_for_route(int T, int H, int E, int K, unsigned flags, const float* w_router, const uint16_t* x,
                        const float* logits, const int32_t* ids, const float* w) {
  if (T <= 0 || E <= 0 || K <= 0 || K > E || !logits || !ids || !w) return false;
  if (flags & ~(unsigned)(MOE_ROUTE_RENORM | MOE_ROUTE_BITONIC)) return false;
  if (E > moe::kMaxE || K > moe::kMaxK) return false;
  if (w_router && (!x || H <= 0 || H % moe::kGroup || H > 8192)) return false;
  return true;
}
}  // namespace

extern "C" int moe_route(const uint16_t* x, const float* w_router, float* logits, int T, int H, int E, int K,
                         unsigned flags, int32_t* ids, float* w, moe_stream_t stream) {
  if (T < 0 || E <= 0 || K <= 0 || K > E || !logits || !ids || !w) return MOE_EINVAL;
  if (flags & ~(unsigned)(MOE_ROUTE_RENORM | MOE_ROUTE_BITONIC)) return MOE_EINVAL;
  if (E > moe::kMaxE || K > moe::kMaxK) return MOE_EUNSUP;
  if (w_router) {
    if (!x || H <= 0) return MOE_EINVAL;
    if (H % moe::kGroup || H > 8192) return MOE_EUNSUP;
  }
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w_router && moe::launch_router_gemv(x, w_router, logits, T, H, E, s) != hipSuccess) return MOE_EHIP;
  if (moe::launch_route_select(logits, T, E, K, flags, ids, w, s) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

extern "C" int moe_route_scored(const uint16_t* x, const float* w_router, float* logits, int T, int H, int E, int K,
                                int score, const float* bias, float routed_scale, unsigned flags, int32_t* ids,
                                float* w, moe_stream_t stream) {
  if (T < 0 || E <= 0 || K <= 0 || K > E || !logits || !ids || !w) return MOE_EINVAL;
  if (flags & ~(unsigned)MOE_ROUTE_RENORM) return MOE_EINVAL;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID && score != MOE_SCORE_SQRTSOFTPLUS) return MOE_EINVAL;
  if (score == MOE_SCORE_SOFTMAX && bias) return MOE_EINVAL;
  if (!std::isfinite(routed_scale)) return MOE_EINVAL;
  if (E > moe::kMaxE || K > moe::kMaxK) return MOE_EUNSUP;
  if (w_router) {
    if (!x || H <= 0) return MOE_EINVAL;
    if (H % moe::kGroup || H > 8192) return MOE_EUNSUP;
  }
  if (T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (w_router && moe::launch_router_gemv(x, w_router, logits, T, H, E, s) != hipSuccess) return MOE_EHIP;
  if (moe::launch_route_select(logits, T, E, K, flags, ids, w, s, score, bias, routed_scale) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

extern "C" size_t moe_ffn_workspace_bytes(int T, int H, int I, int E, int K, int has_shared, unsigned flags) {
  if (T <= 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0) return 0;
  if (ffn_uses_grouped(T, flags)) return moe::grouped_workspace_bytes(T, H, I, E, K, has_shared);
  if (moe::batched_supported(T, H, I, K)) return moe::batched_workspace_bytes(T, H, I, E, K, has_shared);
  return moe::gemv_workspace_bytes(T, H, I, K, has_shared);
}

namespace {

// Whether expert_ffn_stage takes the batched path for these arguments.
bool ffn_uses_batched(int T, int H, int I, int K, unsigned flags, bool has_shared) {
  return !ffn_uses_grouped(T, flags) && gemv_shape_ok(T, H, I, K) &&
         !moe::decode1_supported(T, H, I, K, has_shared) && moe::batched_supported(T, H, I, K);
}

// Shared argument checks and dispatch of one stage (0 = gate/up, 1 = down +
// combine, 2 = both) of the expert FFN. route_logits (batched path only): the
// plan kernel selects the top-k from them and writes ids and w itself.
int expert_ffn_stage(const uint16_t* x, const int32_t* ids, const float* w, int T, int H, int I, int E, int K, int g,
                     const int32_t* slot_table, const void* slots, size_t stride, const void* shared_blob,
                     uint16_t* y, void* ws, size_t ws_bytes, int32_t* dev_status, unsigned flags,
                     moe_stream_t stream, int stage, const int32_t* pre_slots = nullptr,
                     const float* route_logits = nullptr, unsigned route_flags = 0) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || K > E) return MOE_EINVAL;
  if (flags & ~(unsigned)(MOE_FORCE_GEMV | MOE_FORCE_GROUPED | MOE_FFN_PARTIAL | MOE_FFN_PARTIAL_SHARED |
                          MOE_FFN_PARTIAL_FIRST))
    return MOE_EINVAL;
  if ((flags & MOE_FORCE_GEMV) && (flags & (MOE_FORCE_GROUPED | MOE_FFN_PARTIAL))) return MOE_EINVAL;
  if ((flags & MOE_FFN_PARTIAL_SHARED) && (!(flags & MOE_FFN_PARTIAL) || !shared_blob)) return MOE_EINVAL;
  if ((flags & MOE_FFN_PARTIAL_FIRST) && !(flags & MOE_FFN_PARTIAL)) return MOE_EINVAL;
  if (!moe::shape_ok(H, I, g) || E > moe::kMaxE || K > moe::kMaxK) return MOE_EUNSUP;
  if (T == 0) return MOE_OK;
  if (!x || !ids || !w || !slot_table || !slots || !y || !dev_status) return MOE_EINVAL;
  const size_t blob = moe_blob_bytes(H, I, g);
  if (stride < blob || stride % 256) return MOE_EINVAL;
  const bool grouped = ffn_uses_grouped(T, flags);
  if (!grouped && !gemv_shape_ok(T, H, I, K)) return MOE_EUNSUP;
  if (grouped && !moe::grouped_shape_ok(H, I)) return MOE_EUNSUP;
  const size_t need = moe_ffn_workspace_bytes(T, H, I, E, K, shared_blob != nullptr, flags);
  if (need == 0) return MOE_EUNSUP;
  if (!ws || ws_bytes < need) return MOE_EWS;
  moe::FfnArgs a{};
  a.x = x;
  a.ids = ids;
  a.w = w;
  a.T = T;
  a.H = H;
  a.I = I;
  a.E = E;
  a.K = K;
  a.slot_table = slot_table;
  a.slots = static_cast<const uint8_t*>(slots);
  a.stride = stride;
  a.shared_blob = static_cast<const uint8_t*>(shared_blob);
  a.y = y;
  a.ws = static_cast<uint8_t*>(ws);
  a.ws_bytes = ws_bytes;
  a.status = dev_status;
  a.mode = (flags & MOE_FFN_PARTIAL ? moe::kModePartial : 0u) |
           (flags & MOE_FFN_PARTIAL_SHARED ? moe::kModePartialShared : 0u) |
           (flags & MOE_FFN_PARTIAL_FIRST ? moe::kModePartialFirst : 0u);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool dec1 = !grouped && moe::decode1_supported(T, H, I, K, shared_blob != nullptr);
  if (dec1) a.pre_slots = pre_slots;
  const bool bat = !grouped && moe::batched_supported(T, H, I, K);
  if (route_logits) {
    if (!bat || dec1 || stage != 2) return MOE_EINVAL;  // callers check ffn_uses_batched first
    a.route_logits = route_logits;
    a.route_flags = route_flags;
  }
  for (int st = 0; st < 2; ++st) {
    if (stage != 2 && stage != st) continue;
    hipError_t err;
    if (grouped)
      err = moe::launch_ffn_grouped(a, st, s);
    else if (dec1)
      err = moe::launch_ffn_decode1(a, st, s);
    else if (bat)
      err = moe::launch_ffn_batched(a, st, s);
    else
      err = moe::launch_ffn_gemv(a, st, s);
    if (err == hipErrorNotSupported) return MOE_EUNSUP;
    if (err != hipSuccess) return MOE_EHIP;
  }
  return MOE_OK;
}

}  // namespace

extern "C" int moe_expert_ffn(const uint16_t* x, const int32_t* ids, const float* w, int T, int H, int I, int E,
                              int K, int g, const int32_t* slot_table, const void* slots, size_t stride,
                              const void* shared_blob, uint16_t* y, void* ws, size_t ws_bytes,
                              int32_t* dev_status, unsigned flags, moe_stream_t stream) {
  return expert_ffn_stage(x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
                          dev_status, flags, stream, 2);
}

extern "C" int moe_ffn_gate_up(const uint16_t* x, const int32_t* ids, const float* w, int T, int H, int I, int E,
                               int K, int g, const int32_t* slot_table, const void* slots, size_t stride,
                               const void* shared_blob, uint16_t* y, void* ws, size_t ws_bytes,
                               int32_t* dev_status, unsigned flags, moe_stream_t stream) {
  return expert_ffn_stage(x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
                          dev_status, flags, stream, 0);
}

extern "C" int moe_ffn_down(const uint16_t* x, const int32_t* ids, const float* w, int T, int H, int I, int E,
                            int K, int g, const int32_t* slot_table, const void* slots, size_t stride,
                            const void* shared_blob, uint16_t* y, void* ws, size_t ws_bytes, int32_t* dev_status,
                            unsigned flags, moe_stream_t stream) {
  return expert_ffn_stage(x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
                          dev_status, flags, stream, 1);
}

extern "C" size_t moe_route_onepass_ws_bytes(int E, int K) {
  if (E <= 0 || K <= 0 || E > moe::kMaxE || K > moe::kMaxK) return 0;
  return moe::onepass_region_bytes(E, K);
}

extern "C" int moe_route_onepass(const uint16_t* x, const float* w_router, float* logits, int H, int E, int K,
                                 unsigned flags, int32_t* ids, float* w, void* ws, size_t ws_bytes, int32_t* dev_status,
                                 moe_stream_t stream) {
  if (!x || !w_router || !logits || !ids || !w || !dev_status || H <= 0 || E <= 0 || K <= 0 || K > E)
    return MOE_EINVAL;
  if (flags & ~(unsigned)MOE_ROUTE_RENORM) return MOE_EINVAL;
  if (E > moe::kMaxE || K > moe::kMaxK || H % moe::kGroup || H > 8192) return MOE_EUNSUP;
  if (!ws || ws_bytes < moe::onepass_region_bytes(E, K)) return MOE_EWS;
  if (moe::launch_route_onepass(x, w_router, logits, H, E, K, flags, ids, w, static_cast<uint64_t*>(ws), dev_status,
                                static_cast<hipStream_t>(stream)) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

extern "C" int moe_layer(const uint16_t* x, const float* w_router, float* logits, int T, int H, int I, int E, int K,
                         int g, unsigned route_flags, int32_t* ids, float* w, const int32_t* slot_table,
                         const void* slots, size_t stride, const void* shared_blob, uint16_t* y, void* ws,
                         size_t ws_bytes, int32_t* dev_status, unsigned ffn_flags, moe_stream_t stream) {
  const bool onepass = (route_flags & MOE_ROUTE_ONEPASS) != 0;
  route_flags &= ~(unsigned)MOE_ROUTE_ONEPASS;
  // One token on the single-token path: the routing kernel also resolves the
  // chosen experts' slots into the end of the workspace (same results, one
  // dependent load less in each FFN kernel). Everything the FFN call checks is
  // checked here first, so that nothing is enqueued on an argument error.
  const bool dec1 = T == 1 && !ffn_uses_grouped(T, ffn_flags) && moe::shape_ok(H, I, g) && E <= moe::kMaxE &&
                    K <= moe::kMaxK && K <= E && moe::decode1_supported(T, H, I, K, shared_blob != nullptr) &&
                    !(ffn_flags & ~(unsigned)(MOE_FORCE_GEMV)) && slot_table && slots && y && dev_status && ws &&
                    ws_bytes >= moe_ffn_workspace_bytes(T, H, I, E, K, shared_blob != nullptr, ffn_flags) &&
                    stride >= moe_blob_bytes(H, I, g) && stride % 256 == 0 && w_router && x && H <= 8192 && logits && ids &&
                    w &&
                    !(route_flags & ~(unsigned)MOE_ROUTE_RENORM);
  if (onepass && !dec1) {
    // one-pass routing covers one token with a router GEMV on the single-token path;
    // anything else is reported, never run another way
    if (!x || !logits || !ids || !w || !slot_table || !slots || !y || !dev_status || K <= 0 || E <= 0 || K > E)
      return MOE_EINVAL;
    if (route_flags & ~(unsigned)MOE_ROUTE_RENORM) return MOE_EINVAL;
    if (T != 1 || !w_router || (ffn_flags & ~(unsigned)MOE_FORCE_GEMV) || !moe::shape_ok(H, I, g) ||
        E > moe::kMaxE || K > moe::kMaxK || H > 8192 || !moe::decode1_supported(T, H, I, K, shared_blob != nullptr))
      return MOE_EUNSUP;
    if (stride < moe_blob_bytes(H, I, g) || stride % 256) return MOE_EINVAL;
    return MOE_EWS;  // every other condition holds: the workspace is missing or short
  }
  if (dec1) {
    int32_t* pre = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) +
                                              moe::decode1_slots_offset(H, I, K, shared_blob != nullptr));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (onepass) {
      moe::FfnArgs a{};
      a.x = x;
      a.ids = ids;
      a.w = w;
      a.T = T;
      a.H = H;
      a.I = I;
      a.E = E;
      a.K = K;
      a.slot_table = slot_table;
      a.slots = static_cast<const uint8_t*>(slots);
      a.stride = stride;
      a.shared_blob = static_cast<const uint8_t*>(shared_blob);
      a.y = y;
      a.ws = static_cast<uint8_t*>(ws);
      a.ws_bytes = ws_bytes;
      a.status = dev_status;
      a.pre_slots = pre;
      moe::OnepassRoute r{w_router, logits, ids, w, route_flags,
                          reinterpret_cast<uint64_t*>(reinterpret_cast<uint8_t*>(pre) + 256)};
      return moe::launch_ffn_decode1_onepass(a, r, s) == hipSuccess ? MOE_OK : MOE_EHIP;
    }
    if (moe::launch_router_gemv(x, w_router, logits, T, H, E, s) != hipSuccess) return MOE_EHIP;
    if (moe::launch_route_select(logits, T, E, K, route_flags, ids, w, s, MOE_SCORE_SOFTMAX, nullptr, 1.0f, slot_table,
                                 pre) != hipSuccess)
      return MOE_EHIP;
    return expert_ffn_stage(x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
                            dev_status, ffn_flags, stream, 2, pre);
  }
  // The batched path (2..32 tokens): the plan kernel also does the selection (same
  // ids and weights as moe_route's), which saves a launch; the router GEMV, when
  // there is a router, runs first as in moe_route.
  if (T >= 2 && shape_ok_for_route(T, H, E, K, route_flags, w_router, x, logits, ids, w) &&
      !(route_flags & MOE_ROUTE_BITONIC) && moe::batched_routes(E) &&
      ffn_uses_batched(T, H, I, K, ffn_flags, shared_blob != nullptr)) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (w_router && moe::launch_router_gemv(x, w_router, logits, T, H, E, s) != hipSuccess) return MOE_EHIP;
    return expert_ffn_stage(x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
                            dev_status, ffn_flags, stream, 2, nullptr, logits, route_flags);
  }
  const int rs = moe_route(x, w_router, logits, T, H, E, K, route_flags, ids, w, stream);
  if (rs != MOE_OK) return rs;
  return expert_ffn_stage(x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
                          dev_status, ffn_flags, stream, 2);
}

extern "C" int moe_ffn_combine(const int32_t* ids, const float* w, int T, int H, int I, int E, int K, int has_shared,
                               uint16_t* y, void* ws, size_t ws_bytes, int32_t* dev_status, moe_stream_t stream) {
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || K > E || (has_shared != 0 && has_shared != 1))
    return MOE_EINVAL;
  if (!moe::shape_ok(H, I, 32) || E > moe::kMaxE || K > moe::kMaxK || !moe::grouped_shape_ok(H, I)) return MOE_EUNSUP;
  if (T == 0) return MOE_OK;
  if (!ids || !w || !y || !dev_status) return MOE_EINVAL;
  const size_t need = moe_ffn_workspace_bytes(T, H, I, E, K, has_shared, MOE_FFN_PARTIAL);
  if (need == 0) return MOE_EUNSUP;
  if (!ws || ws_bytes < need) return MOE_EWS;
  moe::FfnArgs a{};
  a.ids = ids;
  a.w = w;
  a.T = T;
  a.H = H;
  a.I = I;
  a.E = E;
  a.K = K;
  a.status = dev_status;
  a.mode = moe::kModeCheckDone;
  // the combine reads shared_blob only to test it for NULL (the workspace layout
  // and the shared term depend on it); it is never dereferenced
  a.shared_blob = has_shared ? static_cast<const uint8_t*>(ws) : nullptr;
  a.y = y;
  a.ws = static_cast<uint8_t*>(ws);
  a.ws_bytes = ws_bytes;
  if (moe::launch_grouped_combine(a, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

extern "C" size_t moe_fmt_workspace_bytes(int fmt, int T, int H, int I, int E, int K, int has_shared) {
  if (fmt == MOE_FMT_INT4_G32 || fmt == MOE_FMT_INT4_G128) {
    if (fmt == MOE_FMT_INT4_G128 && moe_fmt_blob_bytes(fmt, H, I) == 0) return 0;
    return moe_ffn_workspace_bytes(T, H, I, E, K, has_shared, 0);
  }
  if (T <= 0 || E <= 0 || K <= 0 || E > moe::kMaxE) return 0;
  if (T > moe::kGemvMaxT) {  // the grouped MFMA path
    if (fmt != MOE_FMT_INT8_G32 && fmt != MOE_FMT_NVFP4) return 0;
    return moe::grouped_fmt_workspace_bytes(T, H, I, E, K, has_shared);
  }
  if (!moe::fmt_shape_ok(fmt, H, I)) return 0;
  return moe::fmt_workspace_bytes(T, H, I, K, has_shared);
}

extern "C" int moe_expert_ffn_fmt(int fmt, const uint16_t* x, const int32_t* ids, const float* w, int T, int H, int I,
                                  int E, int K, const int32_t* slot_table, const void* slots, size_t stride,
                                  const void* shared_blob, uint16_t* y, void* ws, size_t ws_bytes,
                                  int32_t* dev_status, moe_stream_t stream) {
  if (fmt == MOE_FMT_INT4_G128 && T >= 0 && H > 0 && I > 0 && moe_fmt_blob_bytes(fmt, H, I) == 0) return MOE_EUNSUP;
  if (fmt == MOE_FMT_INT4_G32 || fmt == MOE_FMT_INT4_G128)  // group 128 is packed as group 32 (repeated scales)
    return moe_expert_ffn(x, ids, w, T, H, I, E, K, moe::kGroup, slot_table, slots, stride, shared_blob, y, ws,
                          ws_bytes, dev_status, 0, stream);
  if (fmt != MOE_FMT_INT8_G32 && fmt != MOE_FMT_NVFP4) return MOE_EINVAL;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || K > E) return MOE_EINVAL;
  const bool grouped = T > moe::kGemvMaxT;
  if (E > moe::kMaxE || K > moe::kMaxK) return MOE_EUNSUP;
  if (grouped ? !moe::grouped_fmt_shape_ok(H, I) : !moe::fmt_shape_ok(fmt, H, I)) return MOE_EUNSUP;
  if (T == 0) return MOE_OK;
  if (!x || !ids || !w || !slot_table || !slots || !y || !dev_status) return MOE_EINVAL;
  if (stride < moe_fmt_blob_bytes(fmt, H, I) || stride % 256) return MOE_EINVAL;
  const size_t need = moe_fmt_workspace_bytes(fmt, T, H, I, E, K, shared_blob != nullptr);
  if (need == 0) return MOE_EUNSUP;
  if (!ws || ws_bytes < need) return MOE_EWS;
  moe::FfnArgs a{};
  a.x = x;
  a.ids = ids;
  a.w = w;
  a.T = T;
  a.H = H;
  a.I = I;
  a.E = E;
  a.K = K;
  a.slot_table = slot_table;
  a.slots = static_cast<const uint8_t*>(slots);
  a.stride = stride;
  a.shared_blob = static_cast<const uint8_t*>(shared_blob);
  a.y = y;
  a.ws = static_cast<uint8_t*>(ws);
  a.ws_bytes = ws_bytes;
  a.status = dev_status;
  const hipError_t err = grouped ? moe::launch_ffn_grouped_fmt(fmt, a, static_cast<hipStream_t>(stream))
                                  : moe::launch_ffn_fmt(fmt, a, static_cast<hipStream_t>(stream));
  if (err == hipErrorNotSupported) return MOE_EUNSUP;
  return err == hipSuccess ? MOE_OK : MOE_EHIP;
}

#ifdef MOE_TIMELINE
// The instrumented build's row buffers (include/moe_timeline.h).
extern "C" int moe_timeline_read(int kernel, uint64_t* host, int max_blocks) {
  if (kernel < 0 || kernel >= MOE_TL_KERNELS || !host || max_blocks < 1 || max_blocks > MOE_TL_MAX_BLOCKS)
    return MOE_EINVAL;
  if (hipDeviceSynchronize() != hipSuccess) return MOE_EHIP;
  hipError_t err = hipErrorInvalidValue;
  if (moe::tl_owns_route(kernel)) err = moe::tl_read_route(kernel, host, max_blocks);
  if (moe::tl_owns_decode(kernel)) err = moe::tl_read_decode(kernel, host, max_blocks);
  if (moe::tl_owns_batched(kernel)) err = moe::tl_read_batched(kernel, host, max_blocks);
  return err == hipSuccess ? MOE_OK : MOE_EHIP;
}

extern "C" int moe_timeline_clear(void) {
  if (hipDeviceSynchronize() != hipSuccess) return MOE_EHIP;
  const bool ok = moe::tl_clear_route() == hipSuccess && moe::tl_clear_decode() == hipSuccess &&
                  moe::tl_clear_batched() == hipSuccess && hipDeviceSynchronize() == hipSuccess;
  return ok ? MOE_OK : MOE_EHIP;
}
#endif
