"""Pins of the CPU oracle to things other than itself (CPU only).

Each test pins one step of the layer to exact arithmetic, a closed form, a
brute-force count, a hand-written fixture, or an invariant, so that a dropped
term, a wrong sign or index or a transposed operand in the oracle fails here.
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers (test-side)


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack int codes [-8, 7] into the interchange nibble format (even index -> low nibble)."""
    c = (np.asarray(codes, dtype=np.int64) & 0xF).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def nearest_f32(fr: Fraction) -> np.float32:
    """Nearest float32 to an exact rational, ties to the even significand."""
    f = np.float32(float(fr))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - fr), int(np.float32(c).view(np.uint32)) & 1))


def bits_of(v: np.ndarray) -> np.ndarray:
    return gen.bf16_bits_from_f32(np.asarray(v, dtype=np.float32))


def identity_expert(H, I, sg, su, sd, g=32):
    """Gate/up rows i < H are unit vectors e_i, down rows j pick h_j; one scale per matrix."""
    qg = np.zeros((I, H), dtype=np.int64)
    qg[np.arange(min(I, H)), np.arange(min(I, H))] = 1
    qd = np.zeros((H, I), dtype=np.int64)
    qd[np.arange(min(I, H)), np.arange(min(I, H))] = 1
    return {
        "qg": pack_codes(qg),
        "qu": pack_codes(qg),
        "qd": pack_codes(qd),
        "sg": np.full((I, H // g), sg, dtype=np.float16),
        "su": np.full((I, H // g), su, dtype=np.float16),
        "sd": np.full((H, I // g), sd, dtype=np.float16),
    }


# ------------------------------------------------------------------ int4 format


def test_int4_golden_bytes():
    rows = 0
    with open(os.path.join(GOLDEN, "int4_nibbles.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            hexpart, codepart = line.split("|")
            packed = np.array([int(b, 16) for b in hexpart.split()], dtype=np.uint8)
            want = [int(c) for c in codepart.split()]
            got = R.unpack_int4(packed[None, :], 2 * packed.size)[0].tolist()
            assert got == want, (hexpart, got, want)
            rows += 1
    assert rows >= 5


def test_dequant_element_by_element():
    rng = np.random.default_rng(7)
    rows, cols, g = 3, 96, 32
    codes = rng.integers(-8, 8, size=(rows, cols))
    scales = rng.uniform(0.005, 0.02, size=(rows, cols // g)).astype(np.float16)
    W = R.dequantize(pack_codes(codes), scales, cols, g)
    for n in range(rows):
        for j in range(cols):
            assert W[n, j] == float(codes[n, j]) * float(scales[n, j // g])


def test_pack_roundtrip_every_code():
    codes = np.array([[(j % 16) - 8 for j in range(64)]])
    assert R.unpack_int4(pack_codes(codes), 64).tolist() == codes.tolist()


# ------------------------------------------------------------------ router logits


def exact_logits(x_bits, w):
    x = R.bf16_bits_to_f64(x_bits)
    T, E = x.shape[0], w.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    for t in range(T):
        for e in range(E):
            fr = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[t], w[e].astype(np.float64))), Fraction(0))
            out[t, e] = nearest_f32(fr)
    return out


def test_router_logits_exact_random():
    rng = np.random.default_rng(11)
    x_bits = bits_of(rng.standard_normal((3, 48)))
    w = (rng.standard_normal((5, 48)) * 0.02).astype(np.float32)
    got = R.router_logits(x_bits, w)
    assert np.array_equal(got.view(np.uint32), exact_logits(x_bits, w).view(np.uint32))


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_router_logits_double_rounding_midpoint(sign):
    # exact sum = 1 + 2^-24 + 2^-80: just above the float32 midpoint between 1 and 1 + 2^-23.
    # Its float64 rounding is exactly that midpoint, which ties-to-even would send to 1.0.
    x_bits = bits_of([[sign, sign, sign * 2.0**-40]])
    w = np.array([[1.0, 2.0**-24, 2.0**-40]], dtype=np.float32)
    got = R.router_logits(x_bits, w)[0, 0]
    assert got == np.float32(sign * (1.0 + 2.0**-23))
    assert got == exact_logits(x_bits, w)[0, 0]


def test_router_logits_exact_tie_goes_even():
    x_bits = bits_of([[1.0, 1.0]])
    w = np.array([[1.0, 2.0**-24]], dtype=np.float32)  # exactly the midpoint: even neighbour is 1.0
    assert R.router_logits(x_bits, w)[0, 0] == np.float32(1.0)
    w = np.array([[1.0 + 2.0**-23, 2.0**-24]], dtype=np.float32)  # midpoint above an odd significand
    assert R.router_logits(x_bits, w)[0, 0] == np.float32(1.0 + 2.0**-22)


# ------------------------------------------------------------------ selection


def brute_force_ids(row, K):
    E = len(row)
    rank = [sum(1 for f in range(E) if row[f] > row[e] or (row[f] == row[e] and f < e)) for e in range(E)]
    ids = [None] * K
    for e in range(E):
        if rank[e] < K:
            ids[rank[e]] = e
    return ids


def test_select_exhaustive_with_ties():
    values = [0.0, -0.0, 1.0, -1.5]
    E = 6
    n = 0
    for row in itertools.product(values, repeat=E):
        l = np.array([row], dtype=np.float32)
        for K in (1, 3, E):
            assert R.select_topk(l, K)[0].tolist() == brute_force_ids(row, K)
            n += 1
    assert n == 3 * 4**E


def test_select_random_large():
    rng = np.random.default_rng(3)
    l = rng.standard_normal((20, 256)).astype(np.float32)
    l[:, 10] = l[:, 200]  # exact ties across the board
    for t in range(20):
        assert R.select_topk(l[t : t + 1], 8)[0].tolist() == brute_force_ids(l[t].tolist(), 8)


def test_select_rejects_non_finite():
    with pytest.raises(ValueError):
        R.select_topk(np.array([[0.0, np.nan]], dtype=np.float32), 1)


# ------------------------------------------------------------------ softmax weights


def test_softmax_equal_logits():
    for E, K in ((8, 2), (256, 8), (5, 5)):
        ids, w = R.route(np.full((1, E), 0.37, dtype=np.float32), K)
        assert ids[0].tolist() == list(range(K))
        assert np.allclose(w, 1.0 / E, rtol=0, atol=1e-15)


def test_softmax_two_value_closed_form():
    E, delta = 16, 1.75
    l = np.zeros((1, E), dtype=np.float32)
    l[0, 9] = delta
    ids, w = R.route(l, 3)
    assert ids[0].tolist() == [9, 0, 1]
    p_top = 1.0 / (1.0 + (E - 1) * math.exp(-delta))
    p_rest = math.exp(-delta) * p_top
    assert abs(w[0, 0] - p_top) < 1e-15 and abs(w[0, 1] - p_rest) < 1e-15 and abs(w[0, 2] - p_rest) < 1e-15


def test_softmax_renorm():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((4, 32)).astype(np.float32)
    ids, w = R.route(l, 32, renorm=True)
    assert np.allclose(w.sum(1), 1.0, atol=1e-15)
    ids, w = R.route(l, 4, renorm=True)
    _, wp = R.route(l, 4, renorm=False)
    assert np.allclose(w, wp / wp.sum(1, keepdims=True), atol=1e-15)
    assert np.all(wp.sum(1) < 1.0)


# ------------------------------------------------------------------ scored router variants
# ("Strata" README, Models: sigmoid / sqrtsoftplus scoring, correction bias, routed scale)


def f32(v):
    return float(np.float32(v))


def test_scores_closed_forms():
    l = np.array([[0.0, math.log(3.0), -math.log(3.0), 1000.0, -1000.0]], dtype=np.float32)
    s = R.expert_scores(l, R.SCORE_SIGMOID)[0]
    assert s[0] == 0.5 and s[1] == 0.75 and s[2] == 0.25 and s[3] == 1.0 and s[4] == 0.0
    s = R.expert_scores(l, R.SCORE_SQRTSOFTPLUS)[0]
    assert s[0] == f32(math.sqrt(math.log(2.0)))  # softplus(0) = ln 2
    assert abs(float(s[1]) - math.sqrt(math.log(4.0))) <= 2 ** -23  # softplus(ln 3) = ln 4
    assert s[3] == f32(math.sqrt(1000.0))  # e^1000 would overflow: softplus(l) -> l
    assert s[4] == 0.0


def test_scored_unbiased_selection_equals_logit_selection():
    # both scores increase strictly with the logit, so without a bias they pick
    # the same experts in the same order as the logits (when no two scores round equal)
    rng = np.random.default_rng(11)
    l = (2.0 * rng.standard_normal((6, 64))).astype(np.float32)
    for score in (R.SCORE_SIGMOID, R.SCORE_SQRTSOFTPLUS):
        s = R.expert_scores(l, score)
        assert all(len(set(row.tolist())) == 64 for row in s)
        ids, w = R.route_scored(l, 8, score)
        assert np.array_equal(ids, R.select_topk(l, 8))
        assert np.all(np.diff(w, axis=1) <= 0)


def test_scored_bias_steers_selection_only():
    rng = np.random.default_rng(12)
    l = rng.standard_normal((1, 32)).astype(np.float32)
    low = int(np.argmin(l[0]))
    top = int(np.argmax(l[0]))
    bias = np.zeros(32, dtype=np.float32)
    bias[low] = 10.0  # the least likely expert is forced in, at rank 0
    bias[top] = -10.0  # the most likely is forced out
    for score in (R.SCORE_SIGMOID, R.SCORE_SQRTSOFTPLUS):
        s = R.expert_scores(l, score)[0]
        ids, w = R.route_scored(l, 4, score, bias=bias)
        assert ids[0, 0] == low and top not in ids[0].tolist()
        assert w[0, 0] == float(s[low])  # the weight is the score, not score + bias
        c = [float(np.float32(s[e] + bias[e])) for e in range(32)]
        assert ids[0].tolist() == brute_force_ids(c, 4)


def test_scored_renorm_and_routed_scale():
    rng = np.random.default_rng(13)
    l = rng.standard_normal((5, 48)).astype(np.float32)
    bias = (0.1 * rng.standard_normal(48)).astype(np.float32)
    for score in (R.SCORE_SIGMOID, R.SCORE_SQRTSOFTPLUS):
        s = R.expert_scores(l, score)
        ids, w1 = R.route_scored(l, 6, score, bias=bias)
        assert np.array_equal(w1, np.take_along_axis(s, ids, 1).astype(np.float64))
        _, w25 = R.route_scored(l, 6, score, bias=bias, routed_scale=2.5)
        assert np.array_equal(w25, 2.5 * w1)  # the scale is applied once
        _, wn = R.route_scored(l, 6, score, bias=bias, routed_scale=2.5, renorm=True)
        assert all(abs(math.fsum(row.tolist()) - 2.5) < 1e-15 for row in wn)


def test_scored_saturated_scores_tie_to_lower_id():
    # sigmoid rounds to 1.0f above l ~ 17: the scores tie and the lower id ranks first
    l = np.array([[30.0, 40.0, 25.0, 35.0, 0.0]], dtype=np.float32)
    ids, w = R.route_scored(l, 3, R.SCORE_SIGMOID)
    assert ids[0].tolist() == [0, 1, 2] and np.all(w == 1.0)


def test_scored_softmax_scale_and_bias_rule():
    rng = np.random.default_rng(14)
    l = rng.standard_normal((3, 16)).astype(np.float32)
    ids, w = R.route_scored(l, 4, R.SCORE_SOFTMAX, routed_scale=2.5)
    ids0, w0 = R.route(l, 4)
    assert np.array_equal(ids, ids0) and np.array_equal(w, 2.5 * w0)
    with pytest.raises(ValueError):
        R.route_scored(l, 4, R.SCORE_SOFTMAX, bias=np.zeros(16, dtype=np.float32))


# ------------------------------------------------------------------ expert FFN and layer


def test_identity_expert_closed_form():
    H, I = 256, 512
    sg, su, sd = np.float16(2.0), np.float16(0.5), np.float16(0.25)
    ex = R.Expert(identity_expert(H, I, sg, su, sd), H, I)
    rng = np.random.default_rng(9)
    x = R.bf16_bits_to_f64(bits_of(rng.standard_normal((4, H))))
    xt = torch.from_numpy(x)
    want = (float(sd) * float(su) * xt * torch.nn.functional.silu(float(sg) * xt)).numpy()
    got = ex(x)
    assert np.allclose(got, want, rtol=1e-14, atol=1e-300)
    # the single-expert layer (E = K = 1) has routing weight exactly 1
    y, ids, w, _ = R.moe_layer(bits_of(x), {0: ex}, 1, logits=np.zeros((4, 1), dtype=np.float32))
    assert ids.tolist() == [[0]] * 4 and np.all(w == 1.0)
    assert np.allclose(y, want, rtol=1e-14, atol=1e-300)


def tiny_experts(seed, E, H, I):
    return {e: R.Expert(gen.expert_tensors(seed, 0, e, H, I), H, I) for e in range(E)}


def test_zero_activation_gives_zero():
    T, H, E, K, I = 4, 256, 8, 2, 512
    experts = tiny_experts(1, E, H, I)
    wr = gen.router_weight(1, 0, E, H)
    y, ids, w, l = R.moe_layer(np.zeros((T, H), dtype=np.uint16), experts, K, w_router=wr)
    assert np.all(l == 0.0)
    assert ids.tolist() == [[0, 1]] * T
    assert np.all(w == 1.0 / E)
    assert np.all(y == 0.0)


def test_shared_expert_term():
    H, I, E = 256, 512, 4
    shared = R.Expert(identity_expert(H, I, np.float16(1.0), np.float16(1.0), np.float16(1.0)), H, I)
    zero = {"qg": np.zeros((I, H // 2), np.uint8), "qu": np.zeros((I, H // 2), np.uint8),
            "qd": np.zeros((H, I // 2), np.uint8), "sg": np.ones((I, H // 32), np.float16),
            "su": np.ones((I, H // 32), np.float16), "sd": np.ones((H, I // 32), np.float16)}
    experts = {e: R.Expert(zero, H, I) for e in range(E)}
    rng = np.random.default_rng(2)
    xb = bits_of(rng.standard_normal((3, H)))
    x = R.bf16_bits_to_f64(xb)
    y, *_ = R.moe_layer(xb, experts, 2, logits=rng.standard_normal((3, E)).astype(np.float32), shared=shared)
    want = (torch.from_numpy(x) * torch.nn.functional.silu(torch.from_numpy(x))).numpy()
    assert np.allclose(y, want, rtol=1e-14, atol=1e-300)


def test_linearity_in_down_scales():
    T, H, E, K, I = 3, 256, 8, 2, 512
    rng = np.random.default_rng(4)
    xb = bits_of(rng.standard_normal((T, H)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ts = {e: gen.expert_tensors(6, 0, e, H, I) for e in range(E)}
    y1, *_ = R.moe_layer(xb, {e: R.Expert(ts[e], H, I) for e in range(E)}, K, logits=logits)
    ts2 = {e: dict(ts[e], sd=(ts[e]["sd"].astype(np.float32) * 2).astype(np.float16)) for e in range(E)}
    y2, *_ = R.moe_layer(xb, {e: R.Expert(ts2[e], H, I) for e in range(E)}, K, logits=logits)
    assert np.array_equal(y2, 2.0 * y1)


def test_token_permutation_and_expert_relabelling():
    T, H, E, K, I = 5, 256, 8, 3, 512
    rng = np.random.default_rng(8)
    xb = bits_of(rng.standard_normal((T, H)))
    wr = gen.router_weight(2, 0, E, H)
    experts = tiny_experts(3, E, H, I)
    y, ids, w, _ = R.moe_layer(xb, experts, K, w_router=wr)
    perm = rng.permutation(T)
    yp, *_ = R.moe_layer(xb[perm], experts, K, w_router=wr)
    assert np.array_equal(yp, y[perm])
    sigma = rng.permutation(E)  # new id sigma[e] for old expert e
    wr2 = np.empty_like(wr)
    wr2[sigma] = wr
    experts2 = {int(sigma[e]): experts[e] for e in range(E)}
    y2, ids2, w2, _ = R.moe_layer(xb, experts2, K, w_router=wr2)
    assert np.array_equal(ids2, sigma[ids])
    assert np.array_equal(w2, w)
    assert np.allclose(y2, y, rtol=1e-13, atol=1e-15)


def test_dense_limit_is_softmax_mixture():
    T, H, E, I = 3, 256, 6, 512
    rng = np.random.default_rng(12)
    xb = bits_of(rng.standard_normal((T, H)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    experts = tiny_experts(4, E, H, I)
    y, ids, w, _ = R.moe_layer(xb, experts, E, logits=logits)
    p = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    x = R.bf16_bits_to_f64(xb)
    want = sum(p[:, e : e + 1] * experts[e](x) for e in range(E))
    assert np.allclose(y, want, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------------ other expert formats


def test_int8_decoding_all_bytes_against_numpy():
    b = np.arange(256, dtype=np.uint8)
    assert np.array_equal(R.unpack_int8(b), b.view(np.int8).astype(np.int64))


def test_int8_dequantize_hand_values():
    # two's complement bytes 0x00, 0x7F (scale 0.5) and 0x80, 0xFF (scale 0.125); g = 2
    # here to keep the fixture small
    codes = np.array([[0x00, 0x7F, 0x80, 0xFF]], dtype=np.uint8)
    s = np.array([[0.5, 0.125]], dtype=np.float16)
    assert R.dequantize_int8(codes, s, 4, g=2).tolist() == [[0.0, 63.5, -16.0, -0.125]]
    with pytest.raises(ValueError):
        R.dequantize_int8(codes, s, 4, g=4)


def test_group_128_equals_group_32_with_repeated_scales():
    rng = np.random.default_rng(12)
    packed = rng.integers(0, 256, size=(3, 128), dtype=np.uint8)  # 256 columns
    s128 = rng.uniform(0.005, 0.02, size=(3, 2)).astype(np.float16)
    w128 = R.dequantize(packed, s128, 256, g=128)
    w32 = R.dequantize(packed, np.repeat(s128, 4, axis=1), 256, g=32)
    assert np.array_equal(w128, w32)
    # and a different scale in one group changes exactly that group's 128 columns
    s2 = s128.copy()
    s2[1, 1] = np.float16(0.5)
    d = R.dequantize(packed, s2, 256, g=128) != w128
    assert not d[:, :128].any() and not d[0].any() and not d[2].any()


def test_int8_identity_expert_closed_form():
    H, I = 64, 96
    eye_gu = np.zeros((I, H), dtype=np.int64)
    eye_gu[np.arange(H), np.arange(H)] = 1
    eye_dn = np.zeros((H, I), dtype=np.int64)
    eye_dn[np.arange(H), np.arange(H)] = 1

    def as_bytes(q, mult):
        return ((q * mult) & 0xFF).astype(np.uint8)

    t = {
        "qg": as_bytes(eye_gu, 4), "qu": as_bytes(eye_gu, -3), "qd": as_bytes(eye_dn, 127),
        "sg": np.full((I, H // 32), 0.5, dtype=np.float16), "su": np.full((I, H // 32), 0.25, dtype=np.float16),
        "sd": np.full((H, I // 32), 0.125, dtype=np.float16),
    }
    ex = R.Expert(t, H, I, g=32, bits=8)
    rng = np.random.default_rng(13)
    x = R.bf16_bits_to_f64(bits_of(rng.standard_normal((3, H))))
    xt = torch.from_numpy(x)
    # gate = 4 * 0.5 x, up = -3 * 0.25 x, down = 127 * 0.125 h
    want = (127 * 0.125 * (-0.75 * xt) * torch.nn.functional.silu(2.0 * xt)).numpy()
    assert np.allclose(ex(x), want, rtol=1e-14, atol=1e-300)


def test_format_generator_ranges():
    t8 = gen.expert_tensors_fmt(3, 0, 5, 64, 96, gen.FMT_INT8_G32)
    q = R.unpack_int8(t8["qg"])
    assert q.shape == (96, 64) and q.min() == -128 and q.max() == 127
    assert t8["sg"].shape == (96, 2) and t8["sd"].shape == (64, 3)
    t128 = gen.expert_tensors_fmt(3, 0, 5, 256, 128, gen.FMT_INT4_G128)
    assert t128["sg"].shape == (128, 2) and t128["sd"].shape == (256, 1)
    assert np.array_equal(t128["qg"], gen.expert_tensors(3, 0, 5, 256, 128, 32)["qg"])


def test_e4m3_decoding_against_torch():
    b = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(b).view(torch.float8_e4m3fn).double().numpy()
    got = R.decode_e4m3(b)
    nan = np.isnan(want)
    assert np.array_equal(nan, np.isnan(got)) and nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(got[~nan], want[~nan])


def test_e2m1_decoding_against_torch_e4m3():
    # the E4M3 pattern with the same value: exponent + 6, mantissa bit at the top of the
    # three, the E2M1 subnormal 0.5 as 2^-1; decoded by torch, an independent routine
    c = np.arange(16)
    s, e, m = c >> 3, (c >> 1) & 3, c & 1
    pat = np.where(e > 0, (s << 7) | ((e + 6) << 3) | (m << 2), np.where(m == 1, (s << 7) | (6 << 3), s << 7))
    want = torch.from_numpy(pat.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(R.decode_e2m1(c), want)
    assert R.decode_e2m1(c).tolist()[:8] == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_nvfp4_dequantize_hand_values():
    # one row of 32 columns: code bytes 0x71 (columns 0, 1 = 0.5, 6.0), 0xF8 (columns 2, 3 =
    # -0.0, -6.0) and 0x2A (columns 16, 17 = -1.0, 1.0), the rest zero; scales 0x38 (1.0)
    # and 0x01 (2^-9); global 0.25
    packed = np.zeros((1, 16), dtype=np.uint8)
    packed[0, 0], packed[0, 1], packed[0, 8] = 0x71, 0xF8, 0x2A
    W = R.dequantize_nvfp4(packed, np.array([[0x38, 0x01]], dtype=np.uint8), 0.25, 32)
    assert W[0, :4].tolist() == [0.125, 1.5, -0.0, -1.5]
    assert W[0, 16] == -(2.0**-9) * 0.25 and W[0, 17] == 2.0**-9 * 0.25
    assert not W[0, 4:16].any() and not W[0, 18:].any()


def test_nvfp4_unit_scales_give_the_code_values():
    rng = np.random.default_rng(14)
    packed = rng.integers(0, 256, size=(5, 32), dtype=np.uint8)
    W = R.dequantize_nvfp4(packed, np.full((5, 4), 0x38, dtype=np.uint8), 1.0, 64)
    c = np.empty((5, 64), dtype=np.int64)
    c[:, 0::2], c[:, 1::2] = packed & 15, packed >> 4
    assert np.array_equal(W, R.decode_e2m1(c))
    t = gen.expert_tensors_fmt(3, 0, 5, 64, 96, gen.FMT_NVFP4)
    sc = R.decode_e4m3(t["sg"])
    assert sc.min() >= 2.0**-6 and sc.max() < 2.0**-4 and t["sg"].shape == (96, 4) and t["global"].dtype == np.float32


# ------------------------------------------------------------------ expert-major evaluation


@pytest.mark.parametrize("shared", [False, True])
def test_expert_major_equals_per_pair_layer(shared):
    """moe_layer_expert_major (one batched product per expert, then the rank-ordered
    combine) gives moe_layer's ids and weights exactly and its y to float64 rounding,
    with uneven expert loads, an expert nobody picks and repeated tokens."""
    T, H, E, K, I = 37, 256, 9, 3, 160
    rng = np.random.default_rng(31)
    xb = bits_of(rng.standard_normal((T, H)))
    xb[5] = xb[2]
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 4] = -50.0  # expert 4 never selected
    logits[:, 7] += 1.5  # expert 7 in most tokens
    experts = tiny_experts(9, E, H, I)
    sh = R.Expert(gen.expert_tensors(9, 0, gen.SHARED_EXPERT, H, I), H, I) if shared else None
    y1, ids1, w1, _ = R.moe_layer(xb, experts, K, logits=logits, shared=sh)
    y2, ids2, w2, _ = R.moe_layer_expert_major(xb, experts, K, logits=logits, shared=sh)
    assert np.array_equal(ids1, ids2) and np.array_equal(w1, w2)
    assert 4 not in ids1 and (ids1 == 7).any(axis=1).sum() > T // 2
    rms = np.sqrt(np.mean(y1**2))
    assert np.abs(y2 - y1).max() <= 1e-13 * rms


def test_expert_major_dense_limit_and_zero_input():
    """K = E gives the textbook softmax mixture (torch's softmax); x = 0 gives y = 0."""
    T, H, E, I = 4, 256, 5, 512
    rng = np.random.default_rng(13)
    xb = bits_of(rng.standard_normal((T, H)))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    experts = tiny_experts(5, E, H, I)
    y, *_ = R.moe_layer_expert_major(xb, experts, E, logits=logits)
    p = torch.softmax(torch.from_numpy(logits.astype(np.float64)), dim=1).numpy()
    x = R.bf16_bits_to_f64(xb)
    want = sum(p[:, e : e + 1] * experts[e](x) for e in range(E))
    assert np.allclose(y, want, rtol=1e-12, atol=1e-14)
    y0, *_ = R.moe_layer_expert_major(np.zeros((T, H), np.uint16), experts, 2, logits=logits)
    assert np.all(y0 == 0.0)


def test_combine_rank_order_and_shared_term():
    """combine adds the shared output and w[t, k] * o[t, k] for k = 0..K-1: checked on
    values where each term is exactly representable, and the order against a sum whose
    float64 result depends on it (1 + 2^-53 + 2^-53 rounds differently in the other order)."""
    o = np.zeros((1, 3, 2))
    o[0, :, 0] = [1.0, 2.0**-53, 2.0**-53]
    o[0, :, 1] = [3.0, 5.0, 7.0]
    w = np.array([[1.0, 1.0, 1.0]])
    y = R.combine(o, w, shared_out=np.array([[0.0, 0.5]]))
    assert y[0, 0] == 1.0  # (1 + 2^-53) rounds to 1, then again: rank order
    assert y[0, 1] == 15.5
    o2 = o[:, ::-1].copy()
    assert R.combine(o2, w)[0, 0] == 1.0 + 2.0**-52  # the other order keeps both small terms


def test_oracle_pool_expert_major_equals_oracle():
    """The worker-pool evaluation the full-size GPU tests use (tests/oracle_pool.py) gives
    moe_layer_expert_major's ids and weights exactly and its y to float64 rounding."""
    import oracle_pool as OP

    w = gen.Workload("pool_t50_h256_e6_k2_i128_shared", 50, 256, 6, 2, 128, 1, 6, "normal", 17, shared=True)
    xb = gen.activations_bf16(w.seed, 0, w.T, w.H)
    logits = gen.normal_logits(w.seed, 0, w.T, w.E)
    experts = {e: R.Expert(gen.expert_tensors(w.seed, 0, e, w.H, w.I), w.H, w.I) for e in range(w.E)}
    shared = R.Expert(gen.expert_tensors(w.seed, 0, gen.SHARED_EXPERT, w.H, w.I), w.H, w.I)
    y1, ids1, w1, _ = R.moe_layer_expert_major(xb, experts, w.K, logits=logits, shared=shared)
    with OP.pool(2) as ex:
        y2, ids2, w2 = OP.expert_major_layer(ex, w, 0, xb, logits)
        y3, ids3, w3, _ = ex.submit(OP.layer_ref, w, 0, xb, logits).result()
    assert np.array_equal(ids1, ids2) and np.array_equal(w1, w2) and np.array_equal(ids1, ids3)
    rms = np.sqrt(np.mean(y1**2))
    assert np.abs(y2 - y1).max() <= 1e-13 * rms
    assert np.abs(y3 - y1).max() <= 1e-13 * rms
