"""Seeded input generators (no layer arithmetic lives here).

Every tensor is a pure function of ``(seed, layer, expert, kind)`` through
NumPy's PCG64 seeded by ``SeedSequence([seed, layer, expert, kind])``, so any
expert of any layer can be regenerated without storing a model.

Interchange formats (shared by the library's packer and the CPU oracle):

* activations: bf16 bit patterns, ``uint16 [T, H]`` (drawn N(0,1) in fp32,
  rounded to nearest-even);
* router weight: ``float32 [E, H]`` drawn N(0, 0.02^2);
* router logits (when supplied instead of a router): ``float32 [T, E]``;
* int4 codes: row-major ``uint8 [rows, cols/2]``; element ``j`` of a row sits
  in byte ``j // 2``, even ``j`` in the low nibble, each nibble a two's
  complement value in [-8, 7]; drawn uniformly so every code occurs;
* group scales: ``float16 [rows, cols/g]``, one per ``g`` consecutive
  elements of a row, drawn U(0.005, 0.02).

Expert tensors: gate ``[I, H]``, up ``[I, H]``, down ``[H, I]`` (rows are
output features, columns the reduced input features).
"""

from __future__ import annotations

import dataclasses

import numpy as np

KIND_QG, KIND_QU, KIND_QD, KIND_SG, KIND_SU, KIND_SD = 0, 1, 2, 3, 4, 5
KIND_ROUTER, KIND_X, KIND_LOGITS, KIND_STREAM = 10, 11, 12, 13
SHARED_EXPERT = 1 << 20  # expert index used to seed the always-on shared expert


def _rng(seed: int, layer: int, expert: int, kind: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, expert, kind])))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def activations_bf16(seed: int, layer: int, T: int, H: int) -> np.ndarray:
    x = _rng(seed, layer, 0, KIND_X).standard_normal((T, H), dtype=np.float32)
    return bf16_bits_from_f32(x)


def router_weight(seed: int, layer: int, E: int, H: int) -> np.ndarray:
    return (_rng(seed, layer, 0, KIND_ROUTER).standard_normal((E, H), dtype=np.float32) * np.float32(0.02)).astype(
        np.float32
    )


def _codes(seed, layer, expert, kind, rows, cols):
    return _rng(seed, layer, expert, kind).integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)


def _scales(seed, layer, expert, kind, rows, cols, g):
    return _rng(seed, layer, expert, kind).uniform(0.005, 0.02, size=(rows, cols // g)).astype(np.float16)


def expert_tensors(seed: int, layer: int, expert: int, H: int, I: int, g: int = 32) -> dict:
    """Codes and scales of one expert (``expert=SHARED_EXPERT`` for the shared one)."""
    if H % g or I % g or g % 2:
        raise ValueError("H and I must be multiples of the group size")
    return {
        "qg": _codes(seed, layer, expert, KIND_QG, I, H),
        "qu": _codes(seed, layer, expert, KIND_QU, I, H),
        "qd": _codes(seed, layer, expert, KIND_QD, H, I),
        "sg": _scales(seed, layer, expert, KIND_SG, I, H, g),
        "su": _scales(seed, layer, expert, KIND_SU, I, H, g),
        "sd": _scales(seed, layer, expert, KIND_SD, H, I, g),
    }


# expert weight formats (the C enum moe_format)
FMT_INT4_G32, FMT_INT4_G128, FMT_INT8_G32, FMT_NVFP4 = 0, 1, 2, 3
FMT_BITS_G = {FMT_INT4_G32: (4, 32), FMT_INT4_G128: (4, 128), FMT_INT8_G32: (8, 32), FMT_NVFP4: (4, 16)}
KIND_GLOBAL = 97


def expert_tensors_fmt(seed: int, layer: int, expert: int, H: int, I: int, fmt: int) -> dict:
    """Codes and scales of one expert in format ``fmt``. int4: as expert_tensors with
    group 32 or 128. int8: uniform bytes (every code -128..127 occurs), scales
    U(0.005, 0.02) / 16 in fp16, so the weights span the int4 experts' range."""
    bits, g = FMT_BITS_G[fmt]
    if fmt == FMT_NVFP4:
        # uniform code bytes (every E2M1 code occurs); E4M3 scales with exponent
        # field 1 or 2 and any mantissa (2^-6 .. 2^-4.1); globals U(0.5, 1) in fp32
        def nv_scales(kind, rows, cols):
            r = _rng(seed, layer, expert, kind)
            return ((r.integers(1, 3, size=(rows, cols // 16)) << 3) | r.integers(0, 8, size=(rows, cols // 16))).astype(
                np.uint8)

        return {
            "qg": _codes(seed, layer, expert, KIND_QG, I, H),
            "qu": _codes(seed, layer, expert, KIND_QU, I, H),
            "qd": _codes(seed, layer, expert, KIND_QD, H, I),
            "sg": nv_scales(KIND_SG, I, H),
            "su": nv_scales(KIND_SU, I, H),
            "sd": nv_scales(KIND_SD, H, I),
            "global": _rng(seed, layer, expert, KIND_GLOBAL).uniform(0.5, 1.0, size=3).astype(np.float32),
        }
    if bits == 4:
        return expert_tensors(seed, layer, expert, H, I, g)

    def codes(kind, rows, cols):
        return _rng(seed, layer, expert, kind).integers(0, 256, size=(rows, cols), dtype=np.uint8)

    def scales(kind, rows, cols):
        return (_rng(seed, layer, expert, kind).uniform(0.005, 0.02, size=(rows, cols // g)) / 16).astype(np.float16)

    return {
        "qg": codes(KIND_QG, I, H),
        "qu": codes(KIND_QU, I, H),
        "qd": codes(KIND_QD, H, I),
        "sg": scales(KIND_SG, I, H),
        "su": scales(KIND_SU, I, H),
        "sd": scales(KIND_SD, H, I),
    }


def normal_logits(seed: int, layer: int, T: int, E: int) -> np.ndarray:
    return _rng(seed, layer, 0, KIND_LOGITS).standard_normal((T, E), dtype=np.float32)


def zipf_logits(seed: int, layer: int, T: int, E: int, s: float = 1.1) -> np.ndarray:
    """Logits whose top-k is a draw without replacement with P(expert) proportional to rank^-s.

    Each expert gets a rank from a seeded permutation; its logit is the log of its
    Zipf probability plus a standard Gumbel draw (the Gumbel-top-k construction),
    independently per token.
    """
    rng = _rng(seed, layer, 0, KIND_LOGITS)
    rank = np.empty(E, dtype=np.int64)
    rank[rng.permutation(E)] = np.arange(1, E + 1)
    logp = -s * np.log(rank.astype(np.float64))
    logp -= np.log(np.exp(logp).sum())
    u = rng.uniform(np.finfo(np.float64).tiny, 1.0, size=(T, E))
    return (logp[None, :] - np.log(-np.log(u))).astype(np.float32)


def locality_logits(seed: int, layers: int, steps: int, E: int, K: int, p_prev: float = 0.7) -> np.ndarray:
    """Single-token logits ``[steps, layers, E]`` with temporal locality of the chosen experts.

    Per layer and step, each of the K picks is, with probability ``p_prev``, drawn
    uniformly from the previous step's picks (same layer) not yet chosen, else
    uniformly from all experts not yet chosen. Picks get logits 3 + U(0,1); all
    other experts get min(N(0,1), 2.5), so the top-K are exactly the picks.
    """
    out = np.empty((steps, layers, E), dtype=np.float32)
    for layer in range(layers):
        rng = _rng(seed, layer, 0, KIND_LOGITS)
        prev: list[int] = []
        for step in range(steps):
            chosen: list[int] = []
            for _ in range(K):
                pool_prev = [e for e in prev if e not in chosen]
                if pool_prev and rng.uniform() < p_prev:
                    e = pool_prev[int(rng.integers(len(pool_prev)))]
                else:
                    pool = np.setdiff1d(np.arange(E), np.asarray(chosen, dtype=np.int64))
                    e = int(pool[int(rng.integers(len(pool)))])
                chosen.append(e)
            row = np.minimum(rng.standard_normal(E), 2.5)
            row[chosen] = 3.0 + rng.uniform(size=K)
            out[step, layer] = row.astype(np.float32)
            prev = chosen
    return out


def residual_stream(seed: int, steps: int, layers: int, H: int, a: float = 0.99, rho: float = 0.15) -> np.ndarray:
    """Layer inputs of a single-token decode, bf16 bits ``uint16 [steps, layers, H]``.

    A stand-in for a model's residual stream (no trained weights exist here):
    token t's first-layer input is b_t = a b_{t-1} + sqrt(1 - a^2) z (b_0 = z), and
    each layer adds an update, x_{l+1} = (x_l + rho z') / sqrt(1 + rho^2), with z, z'
    N(0, 1) in fp32. ``a`` sets how far consecutive tokens pick the same experts,
    ``rho`` how far consecutive layers' inputs differ. Every vector is N(0, I).
    """
    rng = _rng(seed, 0, 0, KIND_STREAM)
    out = np.empty((steps, layers, H), dtype=np.uint16)
    b = rng.standard_normal(H, dtype=np.float32)
    ca, cb = np.float32(a), np.float32(np.sqrt(1.0 - a * a))
    cn = np.float32(1.0 / np.sqrt(1.0 + rho * rho))
    for t in range(steps):
        if t:
            b = ca * b + cb * rng.standard_normal(H, dtype=np.float32)
        x = b
        for layer in range(layers):
            out[t, layer] = bf16_bits_from_f32(x)
            x = (x + np.float32(rho) * rng.standard_normal(H, dtype=np.float32)) * cn
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and input recipe of one synthetic MoE-layer workload."""

    name: str
    T: int  # tokens per layer call
    H: int  # hidden size
    E: int  # routed experts
    K: int  # experts per token
    I: int  # expert FFN intermediate size
    layers: int
    slots: int  # arena slots per layer
    router: str  # "gemv" (x @ Wr^T), "normal", "zipf" or "locality" (logits supplied), or
    # "residual" (x @ Wr^T on the layer inputs of residual_stream, one router per layer)
    seed: int
    shared: bool = False  # one always-on shared expert (weight 1)
    g: int = 32


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_t4_h256_e8_k2", 4, 256, 8, 2, 512, 1, 8, "gemv", 1),
        Workload("decode_t1_h4096_e256_k8_i1536_x48", 1, 4096, 256, 8, 1536, 48, 64, "gemv", 2),
        Workload("batched_t16_h2048_e128_k8_i768_zipf", 16, 2048, 128, 8, 768, 1, 128, "zipf", 3),
        Workload("prefill_t9940_h4096_e256_k8_i1536", 9940, 4096, 256, 8, 1536, 1, 256, "normal", 4),
        Workload("paged_t1_h4096_e256s1_k6_i2048_x43", 1, 4096, 256, 6, 2048, 43, 64, "locality", 5, shared=True),
        # a 4K prompt through one layer of the paged shape, streamed in chunks through the 64-slot arena
        Workload("chunked_t4096_h4096_e256s1_k6_i2048", 4096, 4096, 256, 6, 2048, 1, 64, "normal", 6, shared=True),
        # the paged shape routed by per-layer router GEMVs on a residual stream: the next
        # layer's router on this layer's input predicts what to read ahead
        Workload("readahead_t1_h4096_e256s1_k6_i2048_x43", 1, 4096, 256, 6, 2048, 43, 64, "residual", 7,
                 shared=True),
    )
}
