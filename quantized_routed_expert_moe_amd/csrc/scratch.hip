// moe_layer_noalloc: moe_layer for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). Its workspace is one file-scope device array per GPU, `scratch`,
// of kScratchBytes; the caller still passes every input and output.
//
// Host code never names `scratch` as an address (on the host the name is only a
// stand-in for the symbol): the first call on a device, with that device
// current, resolves the array's device address with hipGetSymbolAddress and
// keeps it per device; kernels get that address. Nothing here calls hipMalloc,
// hipFree or any routine that allocates.
//
// Every call on a GPU uses that GPU's one array: calls that overlap on one GPU
// (other streams, other host threads) race on it and must be serialised by the
// caller. The array keeps the last call's contents; moe_layer needs none of
// them (its workspace needs no initialisation), so nothing is cleared.
#include <mutex>

#include "moe_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU, held until the process ends
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` on each GPU, once resolved

// The device address of this GPU's array (resolved once per device), or nullptr.
void* scratch_ptr(int* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = MOE_EHIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *err = MOE_EHIP;
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace

extern "C" size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

extern "C" int moe_layer_noalloc(const uint16_t* x, const float* w_router, float* logits, int T, int H, int I, int E,
                                 int K, int g, unsigned route_flags, int32_t* ids, float* w,
                                 const int32_t* slot_table, const void* slots, size_t stride, const void* shared_blob,
                                 uint16_t* y, int32_t* dev_status, unsigned ffn_flags, moe_stream_t stream) {
  // partial passes keep their results in the workspace for moe_ffn_combine, which a
  // caller of this entry point cannot name
  if (ffn_flags & (MOE_FFN_PARTIAL | MOE_FFN_PARTIAL_SHARED | MOE_FFN_PARTIAL_FIRST)) return MOE_EINVAL;
  // one-pass routing keeps hand-off words in a workspace that must start at zero,
  // which a shared array reused by calls of every shape cannot promise
  if (route_flags & MOE_ROUTE_ONEPASS) return MOE_EINVAL;
  if (T < 0 || H <= 0 || I <= 0 || E <= 0 || K <= 0 || K > E) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  const size_t need = moe_ffn_workspace_bytes(T, H, I, E, K, shared_blob != nullptr, ffn_flags);
  if (need == 0) return MOE_EUNSUP;
  if (need > kScratchBytes) return MOE_EWS;  // larger than this entry point's fixed workspace
  int err = MOE_OK;
  void* ws = scratch_ptr(&err);
  if (!ws) return err;
  return moe_layer(x, w_router, logits, T, H, I, E, K, g, route_flags, ids, w, slot_table, slots, stride,
                   shared_blob, y, ws, kScratchBytes, dev_status, ffn_flags, stream);
}
