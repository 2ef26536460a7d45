"""fp64 CPU oracle of the int4 routed-expert MoE layer (test infrastructure only).

What the layer computes, written as plain definitions in float64. Sources:

* "Strata on a Mac (Apple Silicon, Metal)", section "Switches": the router is a
  GEMV producing one logit per expert, dispatched before a separate top-k
  routing step (``moe_route``); "Status": the 64-slot expert cache;
* "Strata" README (ro99/strata), "Models" table and "Architecture" / Kernels:
  4-bit grouped integer experts executed W4A16 (4-bit weights, 16-bit
  activations), checked against a CPU reference implementation;
* "How these numbers are measured", section "Fidelity": paged output must equal
  fully-resident output.

Where the pages leave a step open the plain reading is used (each is named at
the function): softmax over all experts, selection on logits with ties to the
lower expert id, no renormalisation of the selected weights, symmetric
two's-complement int4 with one fp16 scale per 32 consecutive inputs of a row,
SwiGLU with SiLU on the gate projection, an always-on shared expert of weight
1, and a combine summed in rank order.

Parity pins (tests/test_oracle_pins.py): router logits against exact rational
arithmetic; selection against brute-force rank counting; softmax against closed
forms; the scored router variants against closed forms (sigmoid(ln 3) = 3/4,
softplus(ln 3) = ln 4), monotonicity (unbiased selection equals the logit
selection) and bias / scale special cases; int4 decoding against hand-written bytes; dequantisation against an
element-by-element construction; the FFN against a closed form for an
identity-like expert (SiLU from torch); the layer against zero input,
linearity, permutation and relabelling invariances and the dense (K = E)
mixture. Parity unpinned: none of the pages prints a numeric example of this
layer, so no value here is pinned to a published number.
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------- formats


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64 exactly."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float16).astype(np.float64)


def unpack_int4(packed: np.ndarray, cols: int) -> np.ndarray:
    """Decode row-major packed int4 codes to int64 values in [-8, 7].

    Element j of a row is byte j // 2; even j uses the low nibble, odd j the
    high nibble; each nibble is two's complement (symmetric quantisation, no
    zero point).
    """
    p = np.asarray(packed, dtype=np.uint8)
    if p.shape[-1] * 2 != cols:
        raise ValueError("packed row length does not match cols")
    out = np.empty(p.shape[:-1] + (cols,), dtype=np.int64)
    lo = (p & 0x0F).astype(np.int64)
    hi = (p >> 4).astype(np.int64)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out


def dequantize(packed: np.ndarray, scales: np.ndarray, cols: int, g: int = 32) -> np.ndarray:
    """W[n, j] = q[n, j] * s[n, j // g] in float64 (exact: 4-bit times 11-bit significands)."""
    q = unpack_int4(packed, cols).astype(np.float64)
    s = f16_to_f64(scales)
    if s.shape[-1] * g != cols:
        raise ValueError("scale count does not match cols / g")
    return q * np.repeat(s, g, axis=-1)


def unpack_int8(codes: np.ndarray) -> np.ndarray:
    """Decode int8 codes held as bytes (uint8) to int64 values in [-128, 127]:
    two's complement, b - 256 for b >= 128 (the INT8 group-32 experts of the
    "Strata" README, Models and Kernels)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(b >= 128, b - 256, b)


def dequantize_int8(codes: np.ndarray, scales: np.ndarray, cols: int, g: int = 32) -> np.ndarray:
    """W[n, j] = q[n, j] * s[n, j // g] in float64 for int8 codes [rows, cols]."""
    q = unpack_int8(codes).astype(np.float64)
    if q.shape[-1] != cols:
        raise ValueError("code row length does not match cols")
    s = f16_to_f64(scales)
    if s.shape[-1] * g != cols:
        raise ValueError("scale count does not match cols / g")
    return q * np.repeat(s, g, axis=-1)


def decode_e2m1(nibbles: np.ndarray) -> np.ndarray:
    """E2M1 (FP4) codes 0..15 to float64: 1 sign bit, 2 exponent bits (bias 1),
    1 mantissa bit; exponent 0 is subnormal (0 or 0.5). The NVFP4 experts of the
    "Strata" README (Models) hold E2M1 pairs."""
    c = np.asarray(nibbles, dtype=np.int64)
    e, m = (c >> 1) & 3, c & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return np.where(c & 8, -mag, mag)


def decode_e4m3(b: np.ndarray) -> np.ndarray:
    """E4M3 (FP8) bytes to float64: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m * 2^-9); no infinities, S.1111.111 is NaN."""
    v = np.asarray(b, dtype=np.int64)
    e, m = (v >> 3) & 15, v & 7
    mag = np.where(e == 0, m * 2.0**-9, np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(v & 0x80, -mag, mag)


def dequantize_nvfp4(packed: np.ndarray, scales: np.ndarray, global_scale: float, cols: int) -> np.ndarray:
    """W[n, j] = e2m1(c[n, j]) * e4m3(s[n, j // 16]) * global in float64; codes two per
    byte, the even column in the low nibble (group 16, as the README gives NVFP4)."""
    p = np.asarray(packed, dtype=np.uint8)
    if p.shape[-1] * 2 != cols:
        raise ValueError("packed row length does not match cols")
    c = np.empty(p.shape[:-1] + (cols,), dtype=np.int64)
    c[..., 0::2] = p & 0x0F
    c[..., 1::2] = p >> 4
    s = decode_e4m3(scales)
    if s.shape[-1] * 16 != cols:
        raise ValueError("scale count does not match cols / 16")
    return decode_e2m1(c) * np.repeat(s, 16, axis=-1) * float(global_scale)


# ---------------------------------------------------------------- router


def _f32_round_exact(terms: list[float]) -> np.float32:
    """The float32 nearest (ties to even) to the exact sum of float64 ``terms``.

    ``math.fsum`` returns the float64 nearest to the exact sum. Rounding that to
    float32 equals rounding the exact sum to float32 except when the float64
    result sits exactly halfway between two float32 neighbours; then the sign
    of the exact residual (again from fsum, which keeps the sign of an exact
    value) decides.
    """
    s = math.fsum(terms)
    f = np.float32(s)
    if not np.isfinite(f):
        raise FloatingPointError("router logit overflows float32")
    fd = float(f)
    if fd == s:
        return f
    if fd < s:
        lo, hi = f, np.nextafter(f, np.float32(np.inf))
    else:
        lo, hi = np.nextafter(f, np.float32(-np.inf)), f
    mid = (float(lo) + float(hi)) / 2.0  # exact in float64
    if s != mid:
        return f
    r = math.fsum(list(terms) + [-s])
    if r > 0:
        return hi
    if r < 0:
        return lo
    return f  # exact tie: numpy's conversion already rounded to even


def router_logits(x_bits: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """l[t, e] = float32 rounding of the exact sum_h x[t, h] * Wr[e, h].

    The router GEMV of "Strata on a Mac", section "Switches". x is bf16, Wr is
    float32; each product is exact in float64 (8 + 24 significant bits), and the
    sum is rounded once, to the float32 nearest the exact value.
    """
    x = bf16_bits_to_f64(x_bits)
    w = np.asarray(w_router, dtype=np.float32).astype(np.float64)
    T, H = x.shape
    E = w.shape[0]
    if w.shape[1] != H:
        raise ValueError("router weight width must equal hidden size")
    out = np.empty((T, E), dtype=np.float32)
    for t in range(T):
        prods = x[t][None, :] * w  # exact products
        for e in range(E):
            out[t, e] = _f32_round_exact(prods[e].tolist())
    return out


def select_topk(logits: np.ndarray, K: int) -> np.ndarray:
    """ids[t, :] = the K experts with the largest logits, in rank order.

    The total order is (logit descending, expert id ascending): equal logits go
    to the lower id, and -0.0 equals +0.0. Selection is on logits, which ranks
    exactly like the softmax probabilities since softmax is strictly increasing.
    """
    l = np.asarray(logits, dtype=np.float32)
    if not np.all(np.isfinite(l)):
        raise ValueError("router logits must be finite")
    T, E = l.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    ids = np.empty((T, K), dtype=np.int32)
    for t in range(T):
        row = [float(v) for v in l[t]]
        order = sorted(range(E), key=lambda e: (-row[e], e))
        ids[t] = order[:K]
    return ids


def softmax_weights(logits: np.ndarray, ids: np.ndarray, renorm: bool = False) -> np.ndarray:
    """w[t, k] = softmax(l[t, :])[ids[t, k]] in float64.

    The probabilities are over all E experts (softmax, then top-k). By default
    the selected probabilities are used as they are; ``renorm`` divides them by
    their sum over the K selected experts.
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, K = ids.shape
    w = np.empty((T, K), dtype=np.float64)
    for t in range(T):
        m = l[t].max()
        ex = np.exp(l[t] - m)
        z = math.fsum(ex.tolist())
        w[t] = ex[ids[t]] / z
        if renorm:
            w[t] = w[t] / math.fsum(w[t].tolist())
    return w


def route(logits: np.ndarray, K: int, renorm: bool = False):
    ids = select_topk(logits, K)
    return ids, softmax_weights(logits, ids, renorm)


# ---------------------------------------------------------------- router variants

SCORE_SOFTMAX, SCORE_SIGMOID, SCORE_SQRTSOFTPLUS = 0, 1, 2


def expert_scores(logits: np.ndarray, score: int) -> np.ndarray:
    """s[t, e] for the per-expert scoring functions the "Strata" README names
    under "Models": sigmoid (GLM, Laguna) and sqrtsoftplus (DeepSeek).

    The page names the functions only; the plain readings are sigmoid(l) =
    1 / (1 + e^-l) and sqrtsoftplus(l) = sqrt(ln(1 + e^l)), each evaluated in
    float64 and rounded once to float32 (the precision of the selection key).
    softplus is taken as l + ln(1 + e^-l) for l > 0 so that e^l cannot overflow.
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    if score == SCORE_SIGMOID:
        s = 1.0 / (1.0 + np.exp(-l))
    elif score == SCORE_SQRTSOFTPLUS:
        sp = np.where(l > 0, l + np.log1p(np.exp(-np.abs(l))), np.log1p(np.exp(np.minimum(l, 0.0))))
        s = np.sqrt(sp)
    else:
        raise ValueError("score must be sigmoid or sqrtsoftplus")
    return s.astype(np.float32)


def route_scored(logits: np.ndarray, K: int, score: int, bias=None, routed_scale: float = 1.0, renorm: bool = False):
    """ids, w for the scored router variants of the "Strata" README, "Models"
    ("sigmoid/noaux_tc", "sqrtsoftplus/noaux_tc", "sigmoid top-10 routing with a
    correction bias and a 2.5x routed scale").

    Readings taken where the page only names the method: the experts are
    selected on c = float32(s + b), the score plus a per-expert correction bias
    (none when bias is None), with the same total order as ``select_topk``
    (c descending, equal values to the lower id); the bias steers selection
    only, so w[t, k] = s[t, ids[t, k]], divided by their sum over the K
    selected experts when ``renorm``, then multiplied by ``routed_scale``.
    With softmax scores no bias is defined (the softmax probabilities are not
    fixed to the last bit), and w is the softmax weight times the scale.
    """
    if score == SCORE_SOFTMAX:
        if bias is not None:
            raise ValueError("a correction bias needs sigmoid or sqrtsoftplus scores")
        ids, w = route(logits, K, renorm)
        return ids, w * float(routed_scale)
    s = expert_scores(logits, score)
    c = s if bias is None else (s + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32)
    ids = select_topk(c, K)
    T = s.shape[0]
    w = np.empty((T, K), dtype=np.float64)
    for t in range(T):
        w[t] = s[t, ids[t]].astype(np.float64)
        if renorm:
            w[t] = w[t] / math.fsum(w[t].tolist())
    return ids, w * float(routed_scale)


# ---------------------------------------------------------------- experts


def sigmoid(z: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-z))


def silu(z: np.ndarray) -> np.ndarray:
    return z * sigmoid(z)


class Expert:
    """One expert held as fp64 matrices: gate [I, H], up [I, H], down [H, I].

    bits = 4: packed int4 codes (group g = 32 or 128); bits = 8: int8 codes
    (group 32). W[n, j] = q[n, j] * s[n, j // g] either way. With a "global" entry
    the tensors are NVFP4 (dequantize_nvfp4)."""

    def __init__(self, tensors: dict, H: int, I: int, g: int = 32, bits: int = 4):
        self.H, self.I = H, I
        if "global" in tensors:  # NVFP4: E2M1 codes, E4M3 scales, fp32 global scales
            gl = tensors["global"]
            self.Wg = dequantize_nvfp4(tensors["qg"], tensors["sg"], gl[0], H)
            self.Wu = dequantize_nvfp4(tensors["qu"], tensors["su"], gl[1], H)
            self.Wd = dequantize_nvfp4(tensors["qd"], tensors["sd"], gl[2], I)
        else:
            deq = dequantize if bits == 4 else dequantize_int8
            self.Wg = deq(tensors["qg"], tensors["sg"], H, g)
            self.Wu = deq(tensors["qu"], tensors["su"], H, g)
            self.Wd = deq(tensors["qd"], tensors["sd"], I, g)
        if self.Wg.shape != (I, H) or self.Wu.shape != (I, H) or self.Wd.shape != (H, I):
            raise ValueError("expert tensor shapes do not match (H, I)")

    def __call__(self, x: np.ndarray) -> np.ndarray:
        """SwiGLU FFN: down( silu(gate(x)) * up(x) ) for x of shape [..., H]."""
        g = x @ self.Wg.T
        u = x @ self.Wu.T
        return (silu(g) * u) @ self.Wd.T


def moe_layer(x_bits, experts, K, logits=None, w_router=None, shared=None, renorm=False):
    """The whole layer for T tokens.

    ``experts`` maps an expert id to an ``Expert`` (a dict or a callable, so
    callers can build only the experts routing selects). Either ``logits``
    [T, E] or ``w_router`` [E, H] is given. Returns (y fp64 [T, H], ids, w, l).

    y[t] = shared(x[t]) + sum_{k=0..K-1} w[t, k] * expert_{ids[t, k]}(x[t]),
    accumulated in rank order.
    """
    x = bf16_bits_to_f64(x_bits)
    if logits is None:
        logits = router_logits(x_bits, w_router)
    ids, w = route(logits, K, renorm)
    get = experts if callable(experts) else experts.__getitem__
    T, H = x.shape
    y = np.zeros((T, H), dtype=np.float64)
    for t in range(T):
        acc = shared(x[t]) if shared is not None else np.zeros(H)
        for k in range(K):
            acc = acc + w[t, k] * get(int(ids[t, k]))(x[t])
        y[t] = acc
    return y, ids, w, np.asarray(logits, dtype=np.float32)


def expert_outputs(x_bits, experts, ids):
    """o[t, k] = expert_{ids[t, k]}(x[t]) for every (token, pick) pair, float64 [T, K, H].

    The same per-pair FFN as ``moe_layer``, evaluated one expert at a time over
    all the tokens that picked it (one batched product per expert instead of one
    vector product per pair). Only the summation order inside the products can
    differ from ``moe_layer``, so the two agree to float64 rounding."""
    x = bf16_bits_to_f64(x_bits)
    ids = np.asarray(ids)
    T, K = ids.shape
    get = experts if callable(experts) else experts.__getitem__
    o = np.empty((T, K, x.shape[1]), dtype=np.float64)
    for e in np.unique(ids):
        t_idx, k_idx = np.nonzero(ids == e)
        o[t_idx, k_idx] = get(int(e))(x[t_idx])
    return o


def combine(o, w, shared_out=None):
    """y[t] = shared_out[t] + sum_{k=0..K-1} w[t, k] * o[t, k], accumulated in rank order
    (the combine of ``moe_layer``); shared_out None means no shared expert."""
    T, K, H = o.shape
    y = np.zeros((T, H), dtype=np.float64) if shared_out is None else np.array(shared_out, dtype=np.float64)
    for k in range(K):
        y = y + w[:, k : k + 1] * o[:, k]
    return y


def moe_layer_expert_major(x_bits, experts, K, logits=None, w_router=None, shared=None, renorm=False):
    """``moe_layer`` evaluated expert by expert (``expert_outputs`` then ``combine``): the
    same routing and the same rank-ordered combine, for prompts too long to evaluate one
    pair at a time. Returns (y, ids, w, l) as ``moe_layer``."""
    x = bf16_bits_to_f64(x_bits)
    if logits is None:
        logits = router_logits(x_bits, w_router)
    ids, w = route(logits, K, renorm)
    o = expert_outputs(x_bits, experts, ids)
    y = combine(o, w, shared(x) if shared is not None else None)
    return y, ids, w, np.asarray(logits, dtype=np.float32)
