/*
 * moe.h -- C ABI of the int4 routed-expert MoE layer for MI355X (gfx950).
 *
 * One MoE layer of a decode or prefill step: router logits, softmax + top-k
 * routing, resolution of the chosen experts through a fixed-slot expert arena,
 * a SwiGLU expert FFN whose int4 group-32 weights (fp16 scales) are
 * dequantised inside the kernels, and a routing-weighted combine.
 *
 * Sources (web pages on the "Strata" engines):
 *  - "Strata on a Mac (Apple Silicon, Metal)", "Switches": a router GEMV and a
 *    separate top-k routing dispatch (moe_route); "Status": an expert cache of
 *    64 slots; "What you need": an arena that keeps experts and reads the rest
 *    as each token needs them, one contiguous read per expert, and a
 *    "no free slot" failure;
 *  - "Strata" README (ro99/strata), "Models": 4-bit grouped integer experts run
 *    W4A16; "Architecture": a public C interface, routed experts leased into
 *    device memory per decode step through an LRU cache; the execution rules:
 *    top-k and precision never change silently, exact-or-explicit-failure;
 *  - "How these numbers are measured", "Fidelity": paged output equals the
 *    fully-resident output bit for bit.
 *
 * Conventions for every call:
 *  - Return value: MOE_OK (0) or a negative moe_status; moe_strerror() names it.
 *    No C++ exception crosses this interface.
 *  - Argument errors are detected before anything is enqueued. GPU work is
 *    enqueued on the stream given (a hipStream_t passed as moe_stream_t; NULL
 *    is the default stream) and runs asynchronously; a failed launch returns
 *    MOE_EHIP.
 *  - The caller owns every device buffer, pinned host buffer, stream and
 *    event. The library owns only the host metadata of an arena. Borrowed
 *    pointers must stay valid until the work using them has completed.
 *  - Shapes: T tokens, H hidden size, E routed experts, K experts per token,
 *    I expert intermediate size, g the quantisation group (only g = 32).
 *    H and I must be multiples of 32; 1 <= K <= min(E, 32); E <= 1024.
 *    A shape the kernels do not cover returns MOE_EUNSUP; there is no slower
 *    fallback path.
 *  - Calls on distinct streams are reentrant. An arena is single-threaded.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* a hipStream_t */
typedef void* moe_event_t;  /* a hipEvent_t */

enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = -1,  /* bad argument: NULL pointer, size, id out of range */
  MOE_ENOSLOT = -2, /* more distinct experts requested than the arena has slots */
  MOE_ENOTRES = -3, /* an expert was used that is not resident (device status word) */
  MOE_EHIP = -4,    /* a HIP runtime call or kernel launch failed */
  MOE_EUNSUP = -5,  /* shape or option outside what the kernels cover */
  MOE_EWS = -6      /* workspace missing or smaller than moe_ffn_workspace_bytes() */
};

/* Per-expert scoring of the router logits (moe_route_scored). */
enum moe_score {
  MOE_SCORE_SOFTMAX = 0,      /* softmax over all E experts (moe_route) */
  MOE_SCORE_SIGMOID = 1,      /* 1 / (1 + e^-l) */
  MOE_SCORE_SQRTSOFTPLUS = 2  /* sqrt(ln(1 + e^l)) */
};

/* Expert weight formats (moe_pack_expert_fmt, moe_expert_ffn_fmt). */
enum moe_format {
  MOE_FMT_INT4_G32 = 0,  /* int4, one fp16 scale per 32 columns: the blob of moe_pack_expert */
  MOE_FMT_INT4_G128 = 1, /* int4, one fp16 scale per 128 columns */
  MOE_FMT_INT8_G32 = 2,  /* int8, one fp16 scale per 32 columns */
  MOE_FMT_NVFP4 = 3      /* E2M1, one E4M3 scale per 16 columns, one fp32 scale per matrix */
};

enum moe_flags {
  MOE_ROUTE_RENORM = 1u << 0,  /* moe_route: divide the K selected weights by their sum */
  MOE_ROUTE_ONEPASS = 1u << 1, /* moe_layer (route_flags): one-pass routing fused with the gate/up dispatch */
  MOE_ROUTE_BITONIC = 1u << 2, /* moe_route: top-k by a wave-wide bitonic sort of all keys (same results) */
  MOE_FORCE_GEMV = 1u << 8,    /* moe_expert_ffn: use the per-expert GEMV path whatever T is */
  MOE_FORCE_GROUPED = 1u << 9, /* moe_expert_ffn: use the expert-grouped MFMA GEMM path */
  MOE_FFN_PARTIAL = 1u << 10,  /* moe_expert_ffn: one pass of a chunked paged run (see moe_ffn_combine) */
  MOE_FFN_PARTIAL_SHARED = 1u << 11, /* with MOE_FFN_PARTIAL: this pass also computes the shared expert */
  MOE_FFN_PARTIAL_FIRST = 1u << 12   /* with MOE_FFN_PARTIAL: the first pass of a chunk */
};

const char* moe_strerror(int status);
int moe_version(void); /* 100 * major + minor */

/* ------------------------------------------------------------------ experts
 * An expert is one contiguous blob in device memory ("one read per expert
 * instead of three": "Strata on a Mac", What you need): the int4 codes and the
 * fp16 group scales of gate [I x H], up [I x H] and down [H x I]. Its internal
 * layout belongs to the library; build it with moe_pack_expert().
 */

/* Bytes of one expert blob; 0 on an unsupported shape. */
size_t moe_blob_bytes(int H, int I, int g);
/* Slot stride: moe_blob_bytes rounded up to 4096. Slots of an arena and the
 * expert-major host source are laid out with this stride. */
size_t moe_slot_stride(int H, int I, int g);

/* Pack one expert (all pointers host memory) into blob_out (host, at least
 * moe_blob_bytes bytes). Inputs use the plain interchange format:
 *   qg, qu: uint8 [I][H/2]; qd: uint8 [H][I/2]. Row-major int4 codes; element j
 *           of a row is byte j/2, even j in the low nibble; each nibble is a
 *           two's-complement value in [-8, 7] (symmetric, no zero point).
 *   sg, su: fp16 bit patterns [I][H/g]; sd: fp16 bit patterns [H][I/g]; one
 *           scale per g consecutive elements of a row.
 * The dequantised weight is W[n][j] = q[n][j] * s[n][j/g]. Pure host code. */
int moe_pack_expert(const uint8_t* qg, const uint8_t* qu, const uint8_t* qd, const uint16_t* sg,
                    const uint16_t* su, const uint16_t* sd, int H, int I, int g, void* blob_out);

/* ------------------------------------------------------------------ routing
 * moe_route: router logits, then softmax + top-k ("Strata on a Mac", Switches:
 * router GEMV then moe_route).
 *   x        device bf16 [T][H] (bit patterns); read only when w_router != NULL.
 *   w_router device fp32 [E][H], or NULL when the logits are supplied.
 *   logits   device fp32 [T][E]. With w_router: written,
 *            logits[t][e] = fp32(sum_h x[t][h] * w_router[e][h]) accumulated in
 *            fp64 (exact products) and rounded once. Without: read.
 *   ids      device int32 [T][K], out: the K experts with the largest logits in
 *            rank order; equal logits rank the lower id first; -0.0 == +0.0.
 *            Logits must be finite.
 *   w        device fp32 [T][K], out: w[t][k] = softmax(logits[t][:])[ids[t][k]]
 *            over all E experts; with MOE_ROUTE_RENORM divided by sum_k w[t][k].
 *   flags    MOE_ROUTE_RENORM; MOE_ROUTE_BITONIC selects the K by a wave-wide
 *            bitonic sort of all (logit, id) keys instead of the default K
 *            rounds of a wave-wide maximum over per-lane sorted keys (the
 *            keys are distinct, so ids and w are the same bits either way).
 * Deterministic: the same inputs give the same bits on every run. */
int moe_route(const uint16_t* x, const float* w_router, float* logits, int T, int H, int E, int K,
              unsigned flags, int32_t* ids, float* w, moe_stream_t stream);

/* moe_route_scored: the router variants the "Strata" README names under
 * "Models" (sqrtsoftplus/noaux_tc routing, sigmoid/noaux_tc top-8, sigmoid
 * top-10 with a correction bias and a 2.5x routed scale). The page names them
 * only; this is the plain reading:
 *   score    MOE_SCORE_SOFTMAX: as moe_route, w times routed_scale; bias must
 *            be NULL (softmax probabilities are not fixed to the last bit, so
 *            they cannot key a bit-exact selection).
 *            MOE_SCORE_SIGMOID / MOE_SCORE_SQRTSOFTPLUS: s[t][e] = score of
 *            logits[t][e], evaluated in fp64 and rounded once to fp32
 *            (softplus as l + ln(1 + e^-l) for l > 0, so e^l never overflows).
 *   bias     device fp32 [E] correction added to the score for selection only,
 *            or NULL. Must be finite.
 *   ids      the K experts with the largest c = fp32(s + bias) in rank order;
 *            equal c rank the lower id first; -0.0 == +0.0.
 *   w        s[t][ids[t][k]] (the bias is not included), divided by the sum
 *            over the K selected with MOE_ROUTE_RENORM, times routed_scale
 *            (finite). The other arguments are as in moe_route.
 * Deterministic; argument errors return MOE_EINVAL before anything is
 * enqueued. */
int moe_route_scored(const uint16_t* x, const float* w_router, float* logits, int T, int H, int E, int K, int score,
                     const float* bias, float routed_scale, unsigned flags, int32_t* ids, float* w,
                     moe_stream_t stream);

/* moe_route_onepass: moe_route of one token with a router GEMV (T = 1), the
 * router GEMV and the softmax top-k in ONE dispatch ("Strata on a Mac",
 * Switches: the router GEMV and moe_route fused into one dispatch; the page
 * reports that its relaxed-atomics hand-off to the last threadgroup read stale
 * logits). Workgroup e computes logit e and publishes it in its own 64-bit word
 * (a 32-bit call number with the value); the last workgroup waits until all E
 * words carry this call's number, then selects. No word depends on another's
 * ordering, so no cache writeback or invalidation is needed, and the bits of
 * logits, ids and w equal moe_route's.
 *   ws        device, ws_bytes >= moe_route_onepass_ws_bytes(E, K). It must be
 *             all zero before its first one-pass call (zero it once; the calls
 *             keep it consistent), and zeroed again after it is used for
 *             anything else or a call reported an error. One-pass calls on one
 *             workspace must not overlap (one stream, or ordered).
 *   dev_status device int32, zeroed by the caller: MOE_EHIP when the words did
 *             not arrive within a bounded wait (workspace not zeroed, or
 *             overlapping calls); the outputs are then unspecified.
 * Other arguments as moe_route with T = 1; H <= 8192. */
size_t moe_route_onepass_ws_bytes(int E, int K); /* 0 on an unsupported E or K */
int moe_route_onepass(const uint16_t* x, const float* w_router, float* logits, int H, int E, int K, unsigned flags,
                      int32_t* ids, float* w, void* ws, size_t ws_bytes, int32_t* dev_status, moe_stream_t stream);

/* ------------------------------------------------------------------ expert FFN
 * moe_expert_ffn: y[t] = shared(x[t]) + sum_{k=0..K-1} w[t][k] * FFN_{ids[t][k]}(x[t])
 * with FFN(x) = Wd (silu(Wg x) * (Wu x)), silu(z) = z / (1 + e^-z), the terms
 * added in rank order, fp32 accumulation and one bf16 rounding (nearest even)
 * of y. Expert e's blob is at slots + slot_table[e] * stride.
 * Passages: top-k routed experts plus one shared expert ("Strata" README,
 * the models table: 256 experts + 1 shared, top-10 / top-8 / top-6); 4-bit
 * group-quantised experts executed W4A16, i.e. dequantised inside the matrix
 * products against 16-bit activations ("Strata" README, the models table and
 * Kernels: native INT4 group kernels); the prompt's expert GEMMs ("Strata on
 * a Mac", Switches). The SwiGLU form of each expert is this library's reading
 * of the expert FFN, which the pages name but do not write out. Arithmetic of the
 * paths: codes become exact fp16 values; x and h are fp16 operands (bf16 x
 * converts exactly for |x| in [2^-17, 65504], a value past fp16 sets
 * MOE_EUNSUP); the single-token path applies each group's fp16 scale in fp32,
 * the batched and grouped paths multiply it into an fp16 operand fp16(q * s)
 * (one rounding, relative error <= 2^-11).
 *   x          device bf16 [T][H].
 *   ids, w     device [T][K] as written by moe_route.
 *   slot_table device int32 [E]; -1 marks an expert that is not resident.
 *   slots      device base of the slot array; stride = moe_slot_stride().
 *   shared_blob device blob of an always-on shared expert (weight 1), or NULL.
 *   y          device bf16 [T][H], out.
 *   ws         device workspace of ws_bytes >= moe_ffn_workspace_bytes(); its
 *              contents need no initialisation.
 *   dev_status device int32, written only on error: MOE_ENOTRES when a used
 *              expert has slot_table[e] < 0, MOE_EINVAL when an id is outside
 *              [0, E). The caller zeroes it and checks it after the stream
 *              completes; a layer that flags an error has unspecified y.
 *   flags      MOE_FORCE_GEMV / MOE_FORCE_GROUPED select a path; by default the
 *              GEMV path serves T <= 32 and the grouped MFMA path larger T.
 * The reduction order depends only on (T, K, E, flags), never on slot
 * addresses or on which experts are resident, so a paged run gives the same
 * bits as a fully-resident one. */
size_t moe_ffn_workspace_bytes(int T, int H, int I, int E, int K, int has_shared, unsigned flags);
/* The two stages of moe_expert_ffn, with the same arguments, for callers that
 * time or schedule them separately: moe_ffn_gate_up computes h = silu(Wg x) *
 * (Wu x) of every (token, expert) pair into ws (y is not touched);
 * moe_ffn_down then applies Wd and the combine and writes y. They must run in
 * this order on one stream with the same arguments and workspace.
 * moe_expert_ffn(...) is exactly moe_ffn_gate_up(...) then moe_ffn_down(...). */
int moe_ffn_gate_up(const uint16_t* x, const int32_t* ids, const float* w, int T, int H, int I, int E, int K,
                    int g, const int32_t* slot_table, const void* slots, size_t stride, const void* shared_blob,
                    uint16_t* y, void* ws, size_t ws_bytes, int32_t* dev_status, unsigned flags,
                    moe_stream_t stream);
int moe_ffn_down(const uint16_t* x, const int32_t* ids, const float* w, int T, int H, int I, int E, int K, int g,
                 const int32_t* slot_table, const void* slots, size_t stride, const void* shared_blob, uint16_t* y,
                 void* ws, size_t ws_bytes, int32_t* dev_status, unsigned flags, moe_stream_t stream);
int moe_expert_ffn(const uint16_t* x, const int32_t* ids, const float* w, int T, int H, int I, int E, int K,
                   int g, const int32_t* slot_table, const void* slots, size_t stride, const void* shared_blob,
                   uint16_t* y, void* ws, size_t ws_bytes, int32_t* dev_status, unsigned flags,
                   moe_stream_t stream);

/* ------------------------------------------------------------------ other expert formats
 * The other expert formats of the "Strata" README (Models: INT8 group-32
 * linears; Kernels: INT4 group-128 and INT8 group-32 kernels, 16-bit
 * activations). W[n][j] = q[n][j] * s[n][j / g] as for the int4 group-32
 * experts; the layer and every argument are as in moe_expert_ffn, with
 * fmt in moe_format:
 *   MOE_FMT_INT4_G32  the blob of moe_pack_expert; moe_expert_ffn_fmt is
 *                     moe_expert_ffn(..., g = 32, flags = 0) and the two
 *                     functions below return moe_blob_bytes / moe_slot_stride;
 *   MOE_FMT_INT4_G128 codes as for moe_pack_expert (uint8 [rows][cols/2],
 *                     two's-complement nibbles, even column in the low nibble),
 *                     fp16 scales [rows][cols/128]; H, I multiples of 128. Packed
 *                     as a group-32 blob with each scale repeated for its four
 *                     32-column groups (the same weights), so every path of
 *                     moe_expert_ffn serves it (moe_expert_ffn_fmt calls it);
 *   MOE_FMT_INT8_G32  codes int8 [rows][cols] (two's complement, passed as
 *                     uint8), fp16 scales [rows][cols/32]; H, I multiples of 32
 *                     and at most 4096. T <= 32: each (token, expert) pair reads
 *                     its expert's rows (one read per chosen expert for one
 *                     token), the scales applied in fp32. T > 32 (prompts): the
 *                     grouped plan with the format's MFMA GEMM, H and I
 *                     multiples of 64 (else MOE_EUNSUP, no fallback), operand
 *                     fp16(q * s) rounded once, a scale of magnitude >= 512
 *                     sets MOE_EUNSUP in dev_status. x, the intermediate h and,
 *                     for T > 32, each routed term must fit fp16 (else
 *                     MOE_EUNSUP in dev_status).
 *   MOE_FMT_NVFP4     ("Strata" README, the models table: E2M1 pairs, group-16
 *                     E4M3 scales, FP32 per-tensor global scale): W[n][j] =
 *                     e2m1(c[n][j]) * e4m3(s[n][j / 16]) * global; packed with
 *                     moe_pack_expert_nvfp4; H, I multiples of 32 and at most
 *                     8192; for T > 32 the operand e2m1 * e4m3 is exact in fp16
 *                     and the global scale applies to the fp32 sums; otherwise
 *                     as MOE_FMT_INT8_G32.
 * The layout of these blobs belongs to the library. */
size_t moe_fmt_blob_bytes(int fmt, int H, int I);  /* 0 on an unsupported format or shape */
size_t moe_fmt_slot_stride(int fmt, int H, int I); /* moe_fmt_blob_bytes rounded up to 4096 */
int moe_pack_expert_fmt(int fmt, const uint8_t* qg, const uint8_t* qu, const uint8_t* qd, const uint16_t* sg,
                        const uint16_t* su, const uint16_t* sd, int H, int I, void* blob_out);
/* NVFP4 expert (all pointers host memory): qg, qu uint8 [I][H/2], qd [H][I/2],
 * two E2M1 codes per byte (1 sign, 2 exponent bits with bias 1, 1 mantissa
 * bit; the even column in the low nibble); sg, su uint8 [I][H/16], sd
 * [H][I/16], E4M3 scales (bias 7, no infinities; the NaN pattern is rejected
 * with MOE_EINVAL); global3 = the fp32 global scales of gate, up, down. */
int moe_pack_expert_nvfp4(const uint8_t* qg, const uint8_t* qu, const uint8_t* qd, const uint8_t* sg,
                          const uint8_t* su, const uint8_t* sd, const float* global3, int H, int I, void* blob_out);
size_t moe_fmt_workspace_bytes(int fmt, int T, int H, int I, int E, int K, int has_shared);
int moe_expert_ffn_fmt(int fmt, const uint16_t* x, const int32_t* ids, const float* w, int T, int H, int I, int E,
                       int K, const int32_t* slot_table, const void* slots, size_t stride, const void* shared_blob,
                       uint16_t* y, void* ws, size_t ws_bytes, int32_t* dev_status, moe_stream_t stream);

/* Chunked paged prefill ("Strata on a Mac", Measured, the UD-Q4/Q5/Q6_K_XL
 * part: each prompt chunk makes one pass over the experts it uses that are not
 * in the arena). When a
 * chunk of T tokens uses more experts than the arena holds, its FFN runs as
 * several passes over one workspace, each pass with the experts that are
 * resident for it, then one combine:
 *   moe_expert_ffn(..., flags = MOE_FFN_PARTIAL [| MOE_FFN_PARTIAL_SHARED]
 *                  [| MOE_FFN_PARTIAL_FIRST])
 *     computes the routed experts e with slot_table[e] >= 0 (the others are
 *     skipped, not flagged) for their (token, pick) pairs, keeps the per-pair
 *     outputs in ws and does not write y; MOE_FFN_PARTIAL_SHARED also computes
 *     the shared expert (shared_blob must be non-NULL; exactly one pass sets it).
 *     The first pass of every chunk sets MOE_FFN_PARTIAL_FIRST (it starts the
 *     workspace's record of which experts the chunk's passes computed).
 *     MOE_FFN_PARTIAL selects the grouped path (with MOE_FORCE_GEMV: MOE_EINVAL).
 *   moe_ffn_combine then writes y from ws: the shared output (when has_shared)
 *     plus sum_k w[t][k] * out[t][k], as moe_expert_ffn does.
 * Every pass and the combine use the same x, ids, w, T, H, I, E, K, g, the same
 * shared_blob (non-NULL in every pass, has_shared = 1 in the combine, or NULL
 * and 0 throughout), the same ws and one stream order. When each routed expert
 * that ids use has a slot in at least one pass, y is bit-identical to
 * moe_expert_ffn(..., MOE_FORCE_GROUPED) with every expert resident; an
 * expert computed in two passes gives the same bits twice.
 * Exact or explicit failure ("Strata" README, the execution rules): the combine
 * sets *dev_status (device int32, zeroed by the caller; the first error stays)
 * to MOE_ENOTRES when a pair's expert, or the shared expert, was computed in no
 * pass since the chunk's first pass, and to MOE_EINVAL when no pass with
 * MOE_FFN_PARTIAL_FIRST ran since the previous combine on this workspace; y is
 * then unspecified. ids: device int32 [T][K], the ids the passes used.
 * ws_bytes >= moe_ffn_workspace_bytes(T, H, I, E, K, has_shared, MOE_FFN_PARTIAL). */
int moe_ffn_combine(const int32_t* ids, const float* w, int T, int H, int I, int E, int K, int has_shared,
                    uint16_t* y, void* ws, size_t ws_bytes, int32_t* dev_status, moe_stream_t stream);

/* ------------------------------------------------------------------ whole layer
 * moe_layer: moe_route(x, w_router, logits, T, H, E, K, route_flags, ids, w)
 * then moe_expert_ffn(x, ids, w, ..., ffn_flags) in one call on one stream,
 * with the same arguments, checks and results ("Strata on a Mac", Switches:
 * the router GEMV and moe_route run before the expert FFN); ids and w are
 * outputs. A route error returns before the FFN is enqueued. For a resident
 * arena: a paged caller needs ids on the host before the FFN and uses
 * moe_route, arena_map_slots and arena_fill_async, then moe_expert_ffn.
 * route_flags may add MOE_ROUTE_ONEPASS for one token (T = 1) with a router
 * GEMV on the single-token path: the router GEMV, the selection and the gate/up
 * stage run as one dispatch (as moe_route_onepass; the gate/up workgroups wait
 * for their expert's slot word), then the down stage; the same bits as
 * without it. Its hand-off words live in ws, which must then be all zero
 * before the first such call on it, zeroed again after it is used for
 * anything else or a call reported an error, and not shared by overlapping
 * calls; a hand-off that does not complete within a bounded wait sets
 * *dev_status = MOE_EHIP. Other cases with MOE_ROUTE_ONEPASS return
 * MOE_EUNSUP. */
int moe_layer(const uint16_t* x, const float* w_router, float* logits, int T, int H, int I, int E, int K, int g,
              unsigned route_flags, int32_t* ids, float* w, const int32_t* slot_table, const void* slots,
              size_t stride, const void* shared_blob, uint16_t* y, void* ws, size_t ws_bytes,
              int32_t* dev_status, unsigned ffn_flags, moe_stream_t stream);

/* moe_layer_noalloc: moe_layer for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). It allocates nothing: its workspace is the library's own static
 * device array of moe_noalloc_scratch_bytes() bytes (64 MiB) on each GPU, held
 * from the first call on that GPU until the process ends. Arguments, results
 * and errors are those of moe_layer without ws and ws_bytes; in addition
 * MOE_EWS when moe_ffn_workspace_bytes(T, H, I, E, K, has_shared, ffn_flags)
 * exceeds that size, and MOE_EINVAL for the MOE_FFN_PARTIAL* flags (a partial
 * pass leaves its results in a workspace the caller cannot pass on to
 * moe_ffn_combine) and for MOE_ROUTE_ONEPASS (its workspace must start at
 * zero). All calls on one GPU share its array: calls that overlap on one GPU
 * (on other streams or host threads) race and must be serialised by the
 * caller. */
size_t moe_noalloc_scratch_bytes(void);
int moe_layer_noalloc(const uint16_t* x, const float* w_router, float* logits, int T, int H, int I, int E, int K,
                      int g, unsigned route_flags, int32_t* ids, float* w, const int32_t* slot_table,
                      const void* slots, size_t stride, const void* shared_blob, uint16_t* y, int32_t* dev_status,
                      unsigned ffn_flags, moe_stream_t stream);

/* ------------------------------------------------------------------ expert arena
 * A fixed-slot expert arena for one layer ("Strata on a Mac", Status: the
 * expert cache at 64 slots; "Strata" README, Architecture: an LRU lease per
 * decode step). Slot policy, deterministic:
 *   1. the requested ids are walked in order and de-duplicated;
 *   2. more distinct ids than slots -> MOE_ENOSLOT, an id outside [0, E) ->
 *      MOE_EINVAL; either way the arena is unchanged;
 *   3. a resident expert is a hit and is stamped with the call number;
 *   4. each miss, in first-occurrence order, takes the lowest empty slot, else
 *      evicts the expert with the oldest stamp among those not requested in
 *      this call (ties to the lower slot), and becomes a fill {expert, slot};
 *   5. the call number grows by one per successful call.
 */
typedef struct moe_arena moe_arena; /* opaque; host metadata only */
typedef struct {
  int32_t expert, slot;
} moe_fill;
typedef struct {
  uint64_t hits, misses, evictions, fills, h2d_bytes;
  /* arena_prefetch: fills it made (also counted in fills and h2d_bytes, not in
   * misses), and hits of arena_map_slots on an expert a prefetch filled and no
   * arena_map_slots call had requested since */
  uint64_t prefetch_fills, prefetch_hits;
} moe_arena_stats;

/* Create an arena of S slots for E experts.
 *   slots_dev      device, S * stride bytes (caller-owned), or NULL;
 *   slot_table_dev device int32 [E] (caller-owned), or NULL; its contents are
 *                  the caller's until arena_fill_async updates entries;
 *   host_src       pinned host memory, E * stride bytes, expert-major blobs
 *                  (caller-owned), or NULL.
 * With any of the three NULL the arena keeps book only and arena_fill_async
 * fails with MOE_EINVAL. An empty arena holds no expert. */
int arena_create(int E, int S, size_t blob_bytes, size_t stride, void* slots_dev, int32_t* slot_table_dev,
                 const void* host_src, moe_arena** out);
/* Resolve n requested ids (host int32) to slots (host int32 [n], out) and the
 * fills the misses need (host moe_fill, capacity n, out; count in *n_fills).
 * Precondition: no GPU work still reads a slot that may be evicted. */
int arena_map_slots(moe_arena* a, const int32_t* ids, int n, int32_t* slots, moe_fill* fills, int* n_fills);
/* Enqueue on `side`: one hipMemcpyAsync per fill (host_src + expert * stride ->
 * slots_dev + slot * stride, blob_bytes), then the slot_table_dev updates
 * (table[evicted] = -1, table[filled] = slot), then hipEventRecord(done) when
 * done != NULL. The compute stream must wait on `done` before using the
 * slots. Fills must come from the last arena_map_slots or arena_prefetch call. */
int arena_fill_async(moe_arena* a, const moe_fill* fills, int n_fills, moe_stream_t side, moe_event_t done);
/* Read-ahead ("Strata on a Mac", What you need: the experts the next layer
 * will probably use are read ahead; "Strata" README, the execution model: a
 * predictor may steer only what is fetched and when, never what is computed).
 * Maps n predicted ids (host int32) into the arena without counting hits or
 * misses; the fills they need go to fills (host, capacity n; count in
 * *n_fills), to be enqueued with arena_fill_async like those of
 * arena_map_slots:
 *   1. and 2. as arena_map_slots (MOE_EINVAL, MOE_ENOSLOT: arena unchanged);
 *   3. a predicted expert already resident is left as it is (its stamp too);
 *   4. each predicted expert not resident takes a slot by rule 4 of
 *      arena_map_slots (protected: the experts predicted in this call) and the
 *      call's stamp, and becomes a fill;
 *   5. the call number grows by one per successful call.
 * Precondition as arena_map_slots: no GPU work still reads a slot that may be
 * evicted. A later arena_map_slots that requests a prefetched expert finds it
 * resident; the compute stream must then wait for an event recorded on the
 * side stream after the prefetch's copies (arena_fill_async of that later
 * call, on the same side stream, records one). The predicted ids never change
 * a result: every output equals the run without read-ahead, bit for bit. */
int arena_prefetch(moe_arena* a, const int32_t* ids, int n, moe_fill* fills, int* n_fills);
/* Set-up placement: the caller has put expert's blob into slot (no copy, no
 * table write). An expert placed elsewhere before is moved. */
int arena_place(moe_arena* a, int expert, int slot);
/* Host view of the current placement: slot_of[E] (-1 when absent). */
int arena_slot_table(const moe_arena* a, int32_t* slot_of);
int arena_reset(moe_arena* a); /* empty every slot, zero the stamps and the stats */
int arena_stats(const moe_arena* a, moe_arena_stats* out);
void arena_destroy(moe_arena* a);
/* ------------------------------------------------------------------ paged decode layer
 * One layer of single-token decode whose experts page through an arena, with
 * the host hand-shake, the fills and the optional read-ahead sequenced in
 * native code ("Strata on a Mac", What you need: the rest of the experts are
 * read when a token needs them, and the ones the next layer will probably use
 * are read ahead). Per call, on `stream` (compute) and `side` (copies):
 *   1. moe_route(x, layer->w_router) -> ids[0..K), w[0..K), or, when
 *      layer->w_router is NULL, moe_route on the logits the caller put in
 *      logits; with read-ahead (next, w_predict and P > 0) also the top-P of
 *      w_predict on the same x -> ids[K..K+P), w[K..K+P) (which overwrites
 *      logits);
 *   2. the K (+ P) ids to ids_host, then hipEventRecord(ids_ready); with
 *      MOE_PAGED_HOST_POLL instead a one-wave kernel stores the ids into
 *      ids_host and then ids_host[K (+ P)] = s + 1, where s is the value that
 *      word held when the call began (system-scope stores, the word released
 *      last), and the host spins on that word;
 *   3. with MOE_PAGED_SPECULATE the expert FFN is enqueued at once, after the
 *      last fills into layer->arena, with its status word in the workspace;
 *   4. the host waits for ids_ready (or the word), arena_map_slots on the K ids, enqueues
 *      the misses on `side` (arena_fill_async), then arena_prefetch of the P
 *      predicted ids into next->arena and their fills, after the misses;
 *   5. if the map missed any expert, or without MOE_PAGED_SPECULATE, `stream`
 *      waits for this arena's fills and the expert FFN runs (again) with
 *      dev_status.
 * y (device bf16 [H]) then equals moe_expert_ffn on the fully-resident
 * experts, bit for bit, speculation and prediction or not ("Strata" README,
 * the execution model: a predictor changes only what is fetched and when).
 *   layer, next   the arena (its device slots, slot table and pinned host
 *                 source must be set), device fp32 router [E][H] and the
 *                 shared expert's blob (or NULL); next may be NULL and its
 *                 arena must differ from layer's;
 *   w_predict     device fp32 [E][H] predicting next's experts from x, or NULL;
 *   ids, w        device int32 / fp32, K + P entries; logits device fp32 [E];
 *   ids_host      pinned host int32, K + P entries (the ids, readable on
 *                 return), K + P + 1 with MOE_PAGED_HOST_POLL (the last is the
 *                 sequence word; the host spins on it for at most 5 s, then
 *                 returns MOE_EHIP);
 *   ws            device, ws_bytes >= moe_paged_workspace_bytes();
 *   ids_ready     a HIP event owned by the caller (may be NULL with
 *                 MOE_PAGED_HOST_POLL);
 *   n_misses, n_prefetched  (host, may be NULL) the fills of the map and of
 *                 the prefetch.
 * The call returns after step 5 is enqueued (it blocks only on the ids).
 * Calls for the layers of a token go in order on one compute stream; no other
 * GPU work may read an arena while these calls run. Arena rules and errors as
 * arena_map_slots / arena_prefetch / moe_expert_ffn; MOE_EINVAL also for an
 * arena without device buffers, E other than the arena's, K or P larger than
 * an arena, or next->arena == layer->arena; MOE_EWS for a short workspace. */
typedef struct {
  moe_arena* arena;
  const float* w_router;   /* device fp32 [E][H], or NULL: the caller supplies the logits */
  const void* shared_blob; /* device blob of the always-on shared expert, or NULL */
} moe_paged_layer_t;
#define MOE_PAGED_SPECULATE 1u
#define MOE_PAGED_HOST_POLL 2u /* the ids reach the host through a polled word, not an event */
size_t moe_paged_workspace_bytes(int H, int I, int E, int K, int has_shared); /* 0: unsupported shape */
int moe_paged_layer(const moe_paged_layer_t* layer, const moe_paged_layer_t* next, const float* w_predict, int P,
                    const uint16_t* x, int H, int I, int E, int K, int g, float* logits, int32_t* ids, float* w,
                    int32_t* ids_host, uint16_t* y, void* ws, size_t ws_bytes, int32_t* dev_status, unsigned flags,
                    moe_stream_t stream, moe_stream_t side, moe_event_t ids_ready, int* n_misses,
                    int* n_prefetched);

/* Passes of a chunked paged run (moe_ffn_combine): split the distinct experts
 * of n requested ids (host int32) into passes of at most max_per_pass experts.
 * The experts that are resident now come first (ascending id), then the
 * others (ascending id); the list is cut in order. Writes experts (host int32,
 * capacity n; the list), pass_end (host int32, capacity n; pass p is
 * experts[pass_end[p-1] .. pass_end[p]), with pass_end[-1] = 0), *n_distinct
 * and *n_passes; the arena is not changed. The caller then runs, per pass,
 * arena_map_slots on that pass's experts, arena_fill_async and one
 * MOE_FFN_PARTIAL pass whose slot table maps exactly those experts.
 * With max_per_pass <= S / 2 the misses of pass p + 1 evict no expert of pass
 * p, so the fills of pass p + 1 may run while pass p computes (they must still
 * wait for pass p - 1); with any max_per_pass <= S, no fill evicts an expert
 * that a later pass counts as resident.
 * MOE_EINVAL: an id outside [0, E), n < 0, max_per_pass < 1 or > S. */
int arena_chunk_passes(const moe_arena* a, const int32_t* ids, int n, int max_per_pass, int32_t* experts,
                       int32_t* pass_end, int* n_distinct, int* n_passes);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
