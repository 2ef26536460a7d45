// One layer of single-token paged decode, sequenced on the host in native code.
//
// "Strata on a Mac", What you need: experts that are not in the arena are read
// when a token needs them, and the experts the next layer will probably use are
// read ahead. Per call, on the compute stream `stream` and the copy stream
// `side`:
//
//   1. moe_route of x with the layer's router, or on the caller's logits (and,
//      with read-ahead, the top-P of the predictor on the same x: the next
//      layer's probable experts);
//   2. the ids to pinned host memory, event `ids_ready`; with
//      MOE_PAGED_HOST_POLL instead a one-wave kernel stores them there and then
//      a sequence word (system scope), which the host polls (no copy launch and
//      no event wake-up between the route and the fills);
//   3. with MOE_PAGED_SPECULATE: the expert FFN is enqueued at once, after the
//      last fills into this layer's arena, with its status word in the
//      workspace. It reads the slots the device table names when it runs;
//   4. the host waits for `ids_ready` (or the sequence word) only (not for the
//      FFN), maps the ids
//      (arena_map_slots) and enqueues the misses' copies on `side`, then the
//      read-ahead (arena_prefetch into the next layer's arena) after them;
//   5. if the layer missed any expert, or without speculation, the compute
//      stream waits for this arena's fills and runs the FFN (again).
//
// Exactness: a layer with misses always ends with an FFN that waited for every
// copy into its arena. A layer without misses keeps the speculative FFN and its
// status word (copied into dev_status after the decision, so an error the kept
// run raised, such as an activation outside the fp16 range, is reported): it ran
// after every fill that had been enqueued into this arena, none was enqueued
// since (the map made no fill), and every expert it reads was resident then,
// in the slot the table names. So every output equals the fully-resident run,
// bit for bit; the speculation and the prediction only move work earlier
// ("Strata" README: a predictor never changes what is computed).
//
// Hazards: the map and the prefetch may evict only experts that no enqueued
// compute still reads. The host waits for `ids_ready` of this layer, which
// follows every earlier launch on `stream`; the speculative FFN of this layer
// reads only its own requested experts, which this call's map protects; the
// prefetch writes another layer's arena (the same arena as the layer's own is
// rejected). A caller that runs several layers must call them in order on one
// compute stream.
#include <chrono>

#include "arena_internal.h"

namespace {

constexpr double kPollSeconds = 5.0;  // bound of the host's wait for the ids

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

bool arena_ready(const moe_arena* a) { return a && a->slots_dev && a->table_dev && a->host_src; }

}  // namespace

extern "C" size_t moe_paged_workspace_bytes(int H, int I, int E, int K, int has_shared) {
  const size_t ffn = moe_ffn_workspace_bytes(1, H, I, E, K, has_shared, 0);
  return ffn ? round256(ffn) + 256 : 0;
}

extern "C" int moe_paged_layer(const moe_paged_layer_t* cur, const moe_paged_layer_t* next, const float* w_predict,
                               int P, const uint16_t* x, int H, int I, int E, int K, int g, float* logits,
                               int32_t* ids, float* w, int32_t* ids_host, uint16_t* y, void* ws, size_t ws_bytes,
                               int32_t* dev_status, unsigned flags, moe_stream_t stream, moe_stream_t side,
                               moe_event_t ids_ready, int* n_misses, int* n_prefetched) {
  const bool poll = (flags & MOE_PAGED_HOST_POLL) != 0;
  if (!cur || !arena_ready(cur->arena) || !x || !logits || !ids || !w || !ids_host || !y || !ws || !dev_status ||
      (!ids_ready && !poll))
    return MOE_EINVAL;
  if (flags & ~(unsigned)(MOE_PAGED_SPECULATE | MOE_PAGED_HOST_POLL)) return MOE_EINVAL;
  moe_arena* A = cur->arena;
  if (E != A->E || K < 1 || K > A->S) return MOE_EINVAL;
  if (K > moe::kMaxK) return MOE_EUNSUP;
  const bool ahead = next != nullptr && w_predict != nullptr && P > 0;
  if (ahead && (!arena_ready(next->arena) || next->arena == A || next->arena->E != E || P > E ||
                P > next->arena->S))
    return MOE_EINVAL;
  const int has_shared = cur->shared_blob != nullptr;
  const size_t need = moe_paged_workspace_bytes(H, I, E, K, has_shared);
  if (need == 0) return MOE_EINVAL;
  if (ws_bytes < need) return MOE_EWS;
  const size_t ffn_ws = moe_ffn_workspace_bytes(1, H, I, E, K, has_shared, 0);
  int32_t* spec_status = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + round256(ffn_ws));
  hipStream_t s = static_cast<hipStream_t>(stream);

  // no router: logits already holds this layer's logits
  int rc = moe_route(cur->w_router ? x : nullptr, cur->w_router, logits, 1, H, E, K, 0, ids, w, stream);
  if (rc != MOE_OK) return rc;
  const int n_ids = K + (ahead ? P : 0);
  if (ahead) {
    rc = moe_route(x, w_predict, logits, 1, H, E, P, 0, ids + K, w + K, stream);
    if (rc != MOE_OK) return rc;
  }
  int32_t seq = 0;
  if (poll) {
    // the word after the ids: this call waits for the next value of whatever it holds
    seq = __atomic_load_n(ids_host + n_ids, __ATOMIC_ACQUIRE) + 1;
    if (seq == 0) seq = 1;
    if (moe::launch_publish_ids(ids, n_ids, ids_host, seq, s) != hipSuccess) return MOE_EHIP;
  } else {
    if (hipMemcpyAsync(ids_host, ids, sizeof(int32_t) * n_ids, hipMemcpyDeviceToHost, s) != hipSuccess)
      return MOE_EHIP;
    if (hipEventRecord(static_cast<hipEvent_t>(ids_ready), s) != hipSuccess) return MOE_EHIP;
  }

  const bool spec = (flags & MOE_PAGED_SPECULATE) != 0;
  auto run_ffn = [&](int32_t* status) -> int {
    if (hipEvent_t e = arena_fill_event(A))
      if (hipStreamWaitEvent(s, e, 0) != hipSuccess) return MOE_EHIP;
    return moe_expert_ffn(x, ids, w, 1, H, I, E, K, g, A->table_dev, A->slots_dev, A->stride, cur->shared_blob, y,
                          ws, ffn_ws, status, 0, stream);
  };
  if (spec) {
    // the speculative run reports into its own word, cleared first (the workspace
    // arrives uninitialised); it reaches dev_status only if its result is kept
    if (moe::launch_status(spec_status, nullptr, s) != hipSuccess) return MOE_EHIP;
    if ((rc = run_ffn(spec_status)) != MOE_OK) return rc;
  }

  if (poll) {
    const auto t0 = std::chrono::steady_clock::now();
    for (unsigned it = 1; __atomic_load_n(ids_host + n_ids, __ATOMIC_ACQUIRE) != seq; ++it)
      if ((it & 4095u) == 0 &&
          std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count() > kPollSeconds)
        return MOE_EHIP;  // the ids did not arrive (a failed launch upstream)
  } else if (hipEventSynchronize(static_cast<hipEvent_t>(ids_ready)) != hipSuccess) {
    return MOE_EHIP;
  }
  int32_t slots_of[moe::kMaxK];
  moe_fill fills[moe::kMaxK];
  int nf = 0;
  rc = arena_map_slots(A, ids_host, K, slots_of, fills, &nf);
  if (rc != MOE_OK) return rc;
  if (nf > 0 && (rc = arena_fill_async(A, fills, nf, side, nullptr)) != MOE_OK) return rc;
  int npf = 0;
  if (ahead) {
    std::vector<moe_fill> pf(P);
    rc = arena_prefetch(next->arena, ids_host + K, P, pf.data(), &npf);
    if (rc != MOE_OK) return rc;
    if (npf > 0 && (rc = arena_fill_async(next->arena, pf.data(), npf, side, nullptr)) != MOE_OK) return rc;
  }
  if (!spec || nf > 0) {
    if ((rc = run_ffn(dev_status)) != MOE_OK) return rc;
  } else if (moe::launch_status(dev_status, spec_status, s) != hipSuccess) {
    return MOE_EHIP;  // the speculative result is kept, and with it its status
  }
  if (n_misses) *n_misses = nf;
  if (n_prefetched) *n_prefetched = npf;
  return MOE_OK;
}
