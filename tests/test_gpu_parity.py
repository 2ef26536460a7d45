"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars: expert ids bit-exact; routing weights within 1e-5; layer outputs within
max|y - y_ref| <= 2e-2 * rms(y_ref) of the fp64 oracle (parity_util.check_close);
paged and fully-resident runs bitwise equal.
"""

import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from quantized_routed_expert_moe_amd import harness, lib
from synth import gen

from parity_util import DEV, TOL, OracleExperts, check_close, oracle_layer, say, y_f64  # noqa: F401

pytestmark = pytest.mark.gpu


def small(name, **kw):
    return gen.Workload(name, **kw)


# ------------------------------------------------------------------ routing


@pytest.mark.parametrize("wname,layers", [("tiny_t4_h256_e8_k2", [0]), ("decode_t1_h4096_e256_k8_i1536_x48", [0, 1, 47])])
def test_route_gemv_matches_oracle(wname, layers):
    w = gen.WORKLOADS[wname]
    run = harness.LayerRunner(w, DEV)
    for layer in layers:
        say(f"route {wname} layer {layer}")
        xb = gen.activations_bf16(w.seed, layer, w.T, w.H)
        wr = gen.router_weight(w.seed, layer, w.E, w.H)
        x = harness.bf16_tensor(xb, DEV)
        wr_d = torch.from_numpy(wr).to(DEV)
        lg = torch.empty(w.T, w.E, dtype=torch.float32, device=DEV)
        lib.moe_route(x, wr_d, lg, w.T, w.H, w.E, w.K, 0, run.ids, run.wts)
        torch.cuda.synchronize()
        l_ref = R.router_logits(xb, wr)
        l_gpu = lg.cpu().numpy()
        ulp = np.abs(l_gpu.view(np.int32).astype(np.int64) - l_ref.view(np.int32).astype(np.int64))
        say(f"  logits differing from the correctly rounded value: {(ulp > 0).sum()} of {ulp.size}, max {ulp.max()} ulp")
        assert ulp.max() <= 1
        ids_ref, w_ref = R.route(l_ref, w.K)
        assert np.array_equal(run.ids.cpu().numpy(), ids_ref)
        assert np.abs(run.wts.cpu().numpy() - w_ref).max() <= 1e-5


@pytest.mark.parametrize("T,E,K,kind", [(16, 128, 8, "zipf"), (9940, 256, 8, "normal"), (7, 1024, 32, "normal"),
                                        (5, 3, 3, "normal"), (64, 64, 1, "normal")])
def test_route_logits_in(T, E, K, kind):
    say(f"route logits-in T={T} E={E} K={K} {kind}")
    lg = (gen.zipf_logits if kind == "zipf" else gen.normal_logits)(11, 0, T, E)
    d = torch.from_numpy(lg).to(DEV)
    ids = torch.empty(T, K, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, K, dtype=torch.float32, device=DEV)
    for renorm in (False, True):
        lib.moe_route(None, None, d, T, 0, E, K, lib.MOE_ROUTE_RENORM if renorm else 0, ids, wts)
        torch.cuda.synchronize()
        ids_ref, w_ref = R.route(lg, K, renorm)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        assert np.abs(wts.cpu().numpy() - w_ref).max() <= 1e-5


@pytest.mark.parametrize("score", [lib.MOE_SCORE_SIGMOID, lib.MOE_SCORE_SQRTSOFTPLUS])
@pytest.mark.parametrize("T,E,K", [(1, 256, 8), (37, 256, 6), (5, 384, 10), (3, 1024, 32), (4, 32, 32)])
def test_route_scored_matches_oracle(score, T, E, K):
    """Scored router variants: ids bit-exact, weights within 1e-5 of the fp64 oracle."""
    say(f"route scored score={score} T={T} E={E} K={K}")
    lg = (3.0 * gen.normal_logits(21, 0, T, E)).astype(np.float32)
    rng = np.random.default_rng(E + K)
    bias_np = (0.05 * rng.standard_normal(E)).astype(np.float32)
    d = torch.from_numpy(lg).to(DEV)
    bias = torch.from_numpy(bias_np).to(DEV)
    ids = torch.empty(T, K, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, K, dtype=torch.float32, device=DEV)
    for use_bias in (False, True):
        for renorm in (False, True):
            for scale in (1.0, 2.5):
                lib.moe_route_scored(None, None, d, T, 0, E, K, score, bias if use_bias else None, scale,
                                     lib.MOE_ROUTE_RENORM if renorm else 0, ids, wts)
                torch.cuda.synchronize()
                ids_ref, w_ref = R.route_scored(lg, K, score, bias=bias_np if use_bias else None, routed_scale=scale,
                                                renorm=renorm)
                assert np.array_equal(ids.cpu().numpy(), ids_ref), (use_bias, renorm, scale)
                assert np.abs(wts.cpu().numpy() - w_ref).max() <= 1e-5 * scale, (use_bias, renorm, scale)


def test_route_scored_saturated_ties_and_gemv():
    """fp32 saturation makes scores tie (lower id first); the router GEMV feeds the scored select."""
    T, E, K = 4, 64, 8
    lg = np.zeros((T, E), dtype=np.float32)
    lg[0, ::3] = 40.0  # sigmoid -> 1.0f for 22 experts
    lg[1, :] = -200.0  # both scores underflow to 0 for every expert
    lg[2, 5:20] = 18.5
    lg[3] = np.linspace(-30, 30, E, dtype=np.float32)
    d = torch.from_numpy(lg).to(DEV)
    ids = torch.empty(T, K, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, K, dtype=torch.float32, device=DEV)
    for score in (lib.MOE_SCORE_SIGMOID, lib.MOE_SCORE_SQRTSOFTPLUS):
        lib.moe_route_scored(None, None, d, T, 0, E, K, score, None, 2.5, 0, ids, wts)
        torch.cuda.synchronize()
        ids_ref, w_ref = R.route_scored(lg, K, score, routed_scale=2.5)
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        assert np.abs(wts.cpu().numpy() - w_ref).max() <= 2.5e-5
    # with the router GEMV: logits bit-exact, then the same selection
    w = gen.WORKLOADS["tiny_t4_h256_e8_k2"]
    xb = gen.activations_bf16(w.seed, 0, w.T, w.H)
    wr = gen.router_weight(w.seed, 0, w.E, w.H)
    x = harness.bf16_tensor(xb, DEV)
    wrd = torch.from_numpy(wr).to(DEV)
    logits = torch.empty(w.T, w.E, dtype=torch.float32, device=DEV)
    ids = torch.empty(w.T, w.K, dtype=torch.int32, device=DEV)
    wts = torch.empty(w.T, w.K, dtype=torch.float32, device=DEV)
    lib.moe_route_scored(x, wrd, logits, w.T, w.H, w.E, w.K, lib.MOE_SCORE_SIGMOID, None, 1.0, lib.MOE_ROUTE_RENORM,
                         ids, wts)
    torch.cuda.synchronize()
    l_ref = R.router_logits(xb, wr)
    l_gpu = logits.cpu().numpy()
    assert np.abs(l_gpu.view(np.int32).astype(np.int64) - l_ref.view(np.int32).astype(np.int64)).max() <= 1
    ids_ref, w_ref = R.route_scored(l_gpu, w.K, R.SCORE_SIGMOID, renorm=True)  # the selection on the same logits
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(wts.cpu().numpy() - w_ref).max() <= 1e-5


def test_route_scored_softmax_scale_and_argument_errors():
    T, E, K = 6, 128, 8
    lg = gen.normal_logits(23, 0, T, E)
    d = torch.from_numpy(lg).to(DEV)
    ids = torch.empty(T, K, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, K, dtype=torch.float32, device=DEV)
    ids0 = torch.empty_like(ids)
    w0 = torch.empty_like(wts)
    lib.moe_route_scored(None, None, d, T, 0, E, K, lib.MOE_SCORE_SOFTMAX, None, 2.5, 0, ids, wts)
    lib.moe_route(None, None, d, T, 0, E, K, 0, ids0, w0)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids0) and torch.equal(wts, w0 * 2.5)  # one exact scaling of the same weights
    bias = torch.zeros(E, dtype=torch.float32, device=DEV)
    for args in ((lib.MOE_SCORE_SOFTMAX, bias, 1.0), (3, None, 1.0), (lib.MOE_SCORE_SIGMOID, None, float("nan"))):
        with pytest.raises(lib.MoeError) as ei:
            lib.moe_route_scored(None, None, d, T, 0, E, K, args[0], args[1], args[2], 0, ids, wts)
        assert ei.value.status == lib.MOE_EINVAL


@pytest.mark.parametrize("E,K", [(8, 2), (70, 9), (128, 8), (256, 8), (256, 32), (1000, 32), (1024, 1)])
def test_route_bitonic_selection_equals_default(E, K):
    """MOE_ROUTE_BITONIC (a wave-wide bitonic sort of every key) selects the same ids with
    the same weights, bit for bit, as the default selection, and both equal the oracle's ids;
    the logits include ties and signed zeros."""
    T = 33
    rng = np.random.default_rng(E * 100 + K)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[1] = 0.0
    lg[2] = -0.0
    lg[3, ::3] = 1.5  # many equal logits
    lg[4] = np.round(lg[4] * 2) / 2  # coarse values: ties across the top
    d = torch.from_numpy(lg).to(DEV)
    out = {}
    for name, flags in (("default", 0), ("bitonic", lib.MOE_ROUTE_BITONIC), ("bitonic_renorm",
                                                                           lib.MOE_ROUTE_BITONIC | lib.MOE_ROUTE_RENORM),
                        ("renorm", lib.MOE_ROUTE_RENORM)):
        ids = torch.empty(T, K, dtype=torch.int32, device=DEV)
        wts = torch.empty(T, K, dtype=torch.float32, device=DEV)
        lib.moe_route(None, None, d, T, 0, E, K, flags, ids, wts)
        torch.cuda.synchronize()
        out[name] = (ids.cpu().numpy(), wts.cpu().numpy().view(np.int32))
    ids_ref, _ = R.route(lg, K)
    assert np.array_equal(out["default"][0], ids_ref)
    for a, b in (("default", "bitonic"), ("renorm", "bitonic_renorm")):
        assert np.array_equal(out[a][0], out[b][0]) and np.array_equal(out[a][1], out[b][1]), (a, b)


def test_route_ties_and_signed_zero():
    E, K = 70, 9
    rows = [np.zeros(E), -np.zeros(E), np.where(np.arange(E) % 3 == 0, 1.0, -0.0), np.full(E, -2.5),
            np.where(np.arange(E) > 60, 4.0, 0.0)]
    lg = np.array(rows, dtype=np.float32)
    T = lg.shape[0]
    d = torch.from_numpy(lg).to(DEV)
    ids = torch.empty(T, K, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, K, dtype=torch.float32, device=DEV)
    lib.moe_route(None, None, d, T, 0, E, K, 0, ids, wts)
    torch.cuda.synchronize()
    ids_ref, w_ref = R.route(lg, K)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.abs(wts.cpu().numpy() - w_ref).max() <= 1e-6


# ------------------------------------------------------------------ expert FFN vs oracle


def ffn_case(w, layer, flags=0, slots=None, place_seed=None, only_routed=False):
    say(f"ffn {w.name} layer {layer} flags={flags}")
    xb = gen.activations_bf16(w.seed, layer, w.T, w.H)
    logits = None
    if w.router != "gemv":
        logits = {"normal": gen.normal_logits, "zipf": gen.zipf_logits}[w.router](w.seed, layer, w.T, w.E)
    y_ref, ids_ref, w_ref, l_ref = oracle_layer(w, layer, xb, logits=logits)
    experts = sorted(set(ids_ref.ravel().tolist())) if only_routed else None
    L = harness.make_layer(w, layer, DEV, slots=slots, experts=experts, place_seed=place_seed, logits=logits,
                           x_bits=xb)
    run = harness.LayerRunner(w, DEV, flags)
    run(L)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    assert np.array_equal(run.ids.cpu().numpy(), ids_ref)
    check_close(y_f64(run.y), y_ref, f"  {w.name} layer {layer}")
    return L, run


def test_ffn_tiny():
    w = gen.WORKLOADS["tiny_t4_h256_e8_k2"]
    ffn_case(w, 0)
    ffn_case(w, 0, place_seed=3)


@pytest.mark.parametrize("layer", [0, 47])
def test_ffn_decode_full_size(layer):
    w = gen.WORKLOADS["decode_t1_h4096_e256_k8_i1536_x48"]
    ffn_case(w, layer, slots=64, place_seed=100 + layer, only_routed=True)


def test_ffn_batched_zipf_full_layer():
    w = gen.WORKLOADS["batched_t16_h2048_e128_k8_i768_zipf"]
    ffn_case(w, 0, only_routed=True)


def test_ffn_paged_shape_with_shared_expert():
    w = gen.WORKLOADS["paged_t1_h4096_e256s1_k6_i2048_x43"]
    w1 = gen.Workload("paged_one_layer", 1, w.H, w.E, w.K, w.I, 1, 64, "normal", w.seed, shared=True)
    ffn_case(w1, 0, slots=64, place_seed=7, only_routed=True)


@pytest.mark.parametrize(
    "w",
    [
        # ragged: down groups (3) fewer than slices, several token chunks, odd T
        gen.Workload("ragged_t7_h1024_e16_k3_i96", 7, 1024, 16, 3, 96, 1, 16, "gemv", 21),
        gen.Workload("ragged_t32_h512_e40_k5_i160_shared", 32, 512, 40, 5, 160, 1, 40, "normal", 22, shared=True),
        gen.Workload("ragged_t3_h8192_e4_k4_i64", 3, 8192, 4, 4, 64, 1, 4, "zipf", 23),
        gen.Workload("ragged_t2_h96_e6_k6_i4096", 2, 96, 6, 6, 4096, 1, 6, "normal", 24),
    ],
    ids=lambda w: w.name,
)
def test_ffn_ragged_shapes(w):
    ffn_case(w, 0, flags=lib.MOE_FORCE_GEMV)


@pytest.mark.parametrize(
    "w",
    [
        # 32 shared pairs (two M-tiles of 16), I 160: 32-row gate/up workgroups
        gen.Workload("bat_t32_h512_e40_k5_i160_shared", 32, 512, 40, 5, 160, 1, 40, "normal", 25, shared=True),
        # 3 groups in H and in I: one partial chunk each; H 96: 32-row down workgroups
        gen.Workload("bat_t7_h96_e16_k3_i96", 7, 96, 16, 3, 96, 1, 16, "normal", 26),
        # 32 chunks of gate/up codes per wave, 16 of down
        gen.Workload("bat_t3_h4096_e8_k4_i2048", 3, 4096, 8, 4, 2048, 1, 8, "zipf", 27),
        # two tokens, I 64 (one 64-row item), H 160 (5 groups)
        gen.Workload("bat_t2_h160_e6_k6_i64", 2, 160, 6, 6, 64, 1, 6, "normal", 28),
        # every expert takes all 24 tokens: 24 pairs per unit, two M-tiles everywhere
        gen.Workload("bat_t24_h1024_e8_k8_i512_shared", 24, 1024, 8, 8, 512, 1, 8, "normal", 29, shared=True),
    ],
    ids=lambda w: w.name,
)
def test_ffn_batched_shapes(w):
    """The small-batch path (default for 2 <= T <= 32) on partial chunks, each
    workgroup width and units with more pairs than one M-tile."""
    ffn_case(w, 0)


# ------------------------------------------------------------------ whole layer (moe_layer)


@pytest.mark.parametrize(
    "w,renorm",
    [
        (gen.WORKLOADS["decode_t1_h4096_e256_k8_i1536_x48"], False),
        (gen.Workload("paged_shape_t1_shared_logits_in", 1, 4096, 256, 6, 2048, 1, 64, "normal", 5, shared=True),
         True),
        (gen.Workload("dec_t1_h256_e64_k4_i512", 1, 256, 64, 4, 512, 1, 64, "gemv", 31), True),
        (gen.Workload("dec_t1_h512_e256_k32_i512_shared", 1, 512, 256, 32, 512, 1, 256, "gemv", 32, shared=True),
         False),
        (gen.Workload("dec_t1_h256_e512_k8_i512", 1, 256, 512, 8, 512, 1, 512, "normal", 33), False),
        (gen.Workload("t5_h256_e64_k4_i512", 5, 256, 64, 4, 512, 1, 64, "gemv", 34), False),
        # batched path (2..32 tokens): moe_layer selects inside the plan kernel
        (gen.Workload("bat_t16_h2048_e128_k8_i768", 16, 2048, 128, 8, 768, 1, 128, "normal", 35), False),
        (gen.Workload("bat_t16_h2048_e128_k8_i768", 16, 2048, 128, 8, 768, 1, 128, "normal", 35), True),
        (gen.Workload("bat_t32_h512_e512_k8_i256_shared", 32, 512, 512, 8, 256, 1, 512, "gemv", 36, shared=True),
         False),
        (gen.Workload("bat_t2_h256_e1024_k32_i256", 2, 256, 1024, 32, 256, 1, 1024, "normal", 37), True),
        (gen.Workload("bat_t7_h256_e40_k3_i512", 7, 256, 40, 3, 512, 1, 40, "gemv", 38), False),
    ],
    ids=lambda v: v.name if hasattr(v, "name") else f"renorm{int(v)}",
)
def test_layer_equals_route_then_ffn_bitwise(w, renorm):
    """moe_layer gives the bits of moe_route followed by moe_expert_ffn: logits,
    ids, w and y, for one token and for several, with and without renormalised
    weights, router GEMV or logits in, with and without a shared expert; on the
    batched path (2..32 tokens) moe_layer's plan kernel does the selection itself
    (E of 40 to 1024 experts, so every experts-per-lane width)."""
    layer = 3
    say(f"moe_layer {w.name} renorm={renorm}")
    xb = gen.activations_bf16(w.seed, layer, w.T, w.H)
    logits = None
    if w.router != "gemv":
        logits = gen.normal_logits(w.seed, layer, w.T, w.E)
        l_ref = logits
    else:
        l_ref = R.router_logits(xb, gen.router_weight(w.seed, layer, w.E, w.H))
    ids_ref, _ = R.route(l_ref, w.K, renorm)
    experts = sorted(set(ids_ref.ravel().tolist()))
    L = harness.make_layer(w, layer, DEV, slots=max(len(experts), min(w.E, 64)), experts=experts, place_seed=9,
                           logits=logits, x_bits=xb)
    run = harness.LayerRunner(w, DEV)
    run.route(L, renorm=renorm)
    run.ffn(L)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    y1, ids1, w1, lg1 = run.y.clone(), run.ids.clone(), run.wts.clone(), L.logits.clone()
    y2 = torch.empty_like(run.y)
    ids2 = torch.full_like(run.ids, -7)
    w2 = torch.full_like(run.wts, -7.0)
    lg2 = L.logits if L.wr is None else torch.full_like(L.logits, -7.0)
    lib.moe_layer(L.x, L.wr, lg2, w.T, w.H, w.I, w.E, w.K, w.g, lib.MOE_ROUTE_RENORM if renorm else 0, ids2, w2,
                  L.table, L.slots, L.stride, L.shared, y2, run.ws, run.ws_bytes, run.status)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    assert torch.equal(lg2.view(torch.int32), lg1.view(torch.int32))
    assert torch.equal(ids2, ids1)
    assert np.array_equal(ids2.cpu().numpy(), ids_ref)
    assert torch.equal(w2.view(torch.int32), w1.view(torch.int32))
    assert torch.equal(y2.view(torch.int16), y1.view(torch.int16))


def test_layer_decode_matches_oracle():
    w = gen.WORKLOADS["decode_t1_h4096_e256_k8_i1536_x48"]
    layer = 11
    xb = gen.activations_bf16(w.seed, layer, w.T, w.H)
    y_ref, ids_ref, w_ref, _ = oracle_layer(w, layer, xb)
    L = harness.make_layer(w, layer, DEV, slots=64, experts=sorted(set(ids_ref.ravel().tolist())), place_seed=4,
                           x_bits=xb)
    run = harness.LayerRunner(w, DEV)
    lib.moe_layer(L.x, L.wr, L.logits, w.T, w.H, w.I, w.E, w.K, w.g, 0, run.ids, run.wts, L.table, L.slots,
                  L.stride, L.shared, run.y, run.ws, run.ws_bytes, run.status)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    assert np.array_equal(run.ids.cpu().numpy(), ids_ref)
    assert np.abs(run.wts.cpu().numpy() - w_ref).max() <= 1e-5
    check_close(y_f64(run.y), y_ref, "  moe_layer decode layer 11")


# ------------------------------------------------------------------ edge cases and errors


def test_zero_tokens_is_a_noop():
    w = gen.WORKLOADS["tiny_t4_h256_e8_k2"]
    L = harness.make_layer(w, 0, DEV)
    y = torch.full((1, w.H), 7.0, dtype=torch.bfloat16, device=DEV)
    run = harness.LayerRunner(w, DEV)
    lib.moe_route(L.x, L.wr, L.logits, 0, w.H, w.E, w.K, 0, run.ids, run.wts)
    lib.moe_expert_ffn(L.x, run.ids, run.wts, 0, w.H, w.I, w.E, w.K, 32, L.table, L.slots, L.stride, None, y,
                       run.ws, run.ws_bytes, run.status)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


def test_zero_activation_gives_exact_zero():
    w = gen.WORKLOADS["tiny_t4_h256_e8_k2"]
    L = harness.make_layer(w, 0, DEV, x_bits=np.zeros((w.T, w.H), np.uint16))
    run = harness.LayerRunner(w, DEV)
    run(L)
    torch.cuda.synchronize()
    assert run.ids.cpu().numpy().tolist() == [[0, 1]] * w.T
    assert np.all(run.wts.cpu().numpy() == np.float32(1.0 / w.E))
    assert torch.all(run.y.float() == 0.0)


def test_not_resident_and_bad_id_set_status():
    w = gen.WORKLOADS["tiny_t4_h256_e8_k2"]
    L = harness.make_layer(w, 0, DEV)
    run = harness.LayerRunner(w, DEV)
    run.route(L)
    e0 = int(run.ids[0, 0].item())
    L.table[e0] = -1
    run.ffn(L)
    torch.cuda.synchronize()
    assert int(run.status.item()) == lib.MOE_ENOTRES
    run.status.zero_()
    run.ids[1, 1] = w.E  # out of range
    run.ffn(L)
    torch.cuda.synchronize()
    assert int(run.status.item()) in (lib.MOE_EINVAL, lib.MOE_ENOTRES)


def test_layer_single_token_not_resident_sets_status():
    """moe_layer on one token resolves the slots inside the routing kernel: a routed
    expert without a slot still sets MOE_ENOTRES, and with every slot back the
    output is that of moe_route then moe_expert_ffn again."""
    w = gen.Workload("dec_t1_h256_e64_k4_i512_status", 1, 256, 64, 4, 512, 1, 64, "gemv", 35, shared=True)
    L = harness.make_layer(w, 0, DEV, place_seed=8)
    run = harness.LayerRunner(w, DEV)
    run.layer(L)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    y0 = run.y.view(torch.int16).clone()
    for k in (0, w.K - 1):
        e = int(run.ids[0, k].item())
        saved = int(L.table[e].item())
        L.table[e] = -1
        run.layer(L)
        torch.cuda.synchronize()
        assert int(run.status.item()) == lib.MOE_ENOTRES, k
        run.status.zero_()
        L.table[e] = saved
    run.layer(L)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    assert torch.equal(run.y.view(torch.int16), y0)
    run.route(L)
    run.ffn(L)
    torch.cuda.synchronize()
    assert torch.equal(run.y.view(torch.int16), y0)


def test_argument_errors_return_status():
    w = gen.WORKLOADS["tiny_t4_h256_e8_k2"]
    L = harness.make_layer(w, 0, DEV)
    run = harness.LayerRunner(w, DEV)
    with pytest.raises(lib.MoeError) as e:
        lib.moe_expert_ffn(L.x, run.ids, run.wts, w.T, w.H, w.I, w.E, w.K, 32, L.table, L.slots, L.stride, None,
                           run.y, run.ws, 16, run.status)
    assert e.value.status == lib.MOE_EWS
    with pytest.raises(lib.MoeError) as e:
        lib.moe_route(L.x, L.wr, L.logits, w.T, w.H, w.E, w.E + 1, 0, run.ids, run.wts)
    assert e.value.status == lib.MOE_EINVAL
    with pytest.raises(lib.MoeError) as e:
        lib.moe_expert_ffn(L.x, run.ids, run.wts, w.T, w.H, w.I, w.E, w.K, 64, L.table, L.slots, L.stride, None,
                           run.y, run.ws, run.ws_bytes, run.status)
    assert e.value.status == lib.MOE_EUNSUP


# ------------------------------------------------------------------ fidelity: paged == resident, bitwise


def test_resident_layout_invariance_bitwise():
    """Same layer under the identity map, a permuted map and a routed-only arena: identical bits."""
    w = gen.Workload("fid_t5_h1024_e32_k4_i256_shared", 5, 1024, 32, 4, 256, 1, 32, "gemv", 31, shared=True)
    xb = gen.activations_bf16(w.seed, 0, w.T, w.H)
    outs = []
    for slots, place_seed, only in ((None, None, False), (None, 5, False), (64, 9, True)):
        L0 = harness.make_layer(w, 0, DEV, x_bits=xb)
        run = harness.LayerRunner(w, DEV)
        run.route(L0)
        routed = sorted(set(run.ids.cpu().numpy().ravel().tolist())) if only else None
        L = harness.make_layer(w, 0, DEV, slots=slots, experts=routed, place_seed=place_seed, x_bits=xb)
        for _ in range(2):  # run twice: same bits
            run(L)
            torch.cuda.synchronize()
            assert int(run.status.item()) == 0
            outs.append(run.y.view(torch.int16).cpu().numpy().copy())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def test_paged_equals_resident_at_budget_top_k():
    """Decode steps through an arena with S = K slots (maximum paging pressure) filled by
    arena_fill_async from pinned host memory: every step bitwise equal to the resident run."""
    w = gen.Workload("paged_t1_h1024_e32s1_k4_i512", 1, 1024, 32, 4, 512, 2, 4, "locality", 41, shared=True)
    steps = 24
    lg = gen.locality_logits(w.seed, w.layers, steps, w.E, w.K)
    stride = lib.moe_slot_stride(w.H, w.I)
    blob = lib.moe_blob_bytes(w.H, w.I)
    comp = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    run = harness.LayerRunner(w, DEV)
    y_res = torch.empty_like(run.y)
    for layer in range(w.layers):
        host = torch.empty(w.E * stride, dtype=torch.uint8, pin_memory=True)
        for e in range(w.E):
            host[e * stride : (e + 1) * stride].copy_(torch.from_numpy(harness.pack_expert(w.seed, layer, e, w.H, w.I)))
        resident = harness.make_layer(w, layer, DEV, logits=lg[0, layer][None, :])
        slots = torch.empty(w.K * stride, dtype=torch.uint8, device=DEV)
        table = torch.full((w.E,), -1, dtype=torch.int32, device=DEV)
        arena = lib.Arena(w.E, w.K, blob, stride, slots, table, host)
        ids_h = torch.empty(w.K, dtype=torch.int32, pin_memory=True)
        done = torch.cuda.Event()
        done.record(side)  # creates the HIP event
        for s in range(steps):
            resident.logits.copy_(torch.from_numpy(lg[s, layer][None, :]))
            run.route(resident)
            ids_h.copy_(run.ids.view(-1), non_blocking=True)
            comp.synchronize()  # the per-layer hand-shake: read the router's choice
            _, fills = arena.map_slots(ids_h.tolist())
            arena.fill_async(side, done)
            comp.wait_event(done)
            run.ffn(harness.DeviceLayer(w, layer, resident.x, None, resident.logits, slots, table, resident.shared,
                                        arena, stride))
            run.ffn(resident, y=y_res)
            torch.cuda.synchronize()
            assert int(run.status.item()) == 0
            assert torch.equal(run.y.view(torch.int16), y_res.view(torch.int16)), (layer, s)
        st = arena.stats()
        say(f"  layer {layer}: hits {st['hits']} misses {st['misses']} evictions {st['evictions']}")
        assert st["misses"] > 0 and st["hits"] + st["misses"] == steps * w.K


# ------------------------------------------------------------------ grouped (prefill) path


@pytest.mark.parametrize(
    "w",
    [
        gen.Workload("grouped_t300_h512_e16_k4_i256", 300, 512, 16, 4, 256, 1, 16, "normal", 51),
        gen.Workload("grouped_t77_h1024_e40_k6_i192_shared", 77, 1024, 40, 6, 192, 1, 40, "zipf", 52, shared=True),
        gen.Workload("grouped_t33_h256_e8_k2_i512", 33, 256, 8, 2, 512, 1, 8, "gemv", 53),
        gen.Workload("grouped_t5_h384_e3_k3_i128", 5, 384, 3, 3, 128, 1, 3, "normal", 54),
    ],
    ids=lambda w: w.name,
)
def test_grouped_matches_oracle(w):
    flags = lib.MOE_FORCE_GROUPED if w.T <= 32 else 0
    L, run = ffn_case(w, 0, flags=flags, place_seed=2)
    first = run.y.view(torch.int16).clone()
    run(L)  # same inputs again: identical bits although the pair scatter uses atomics
    torch.cuda.synchronize()
    assert torch.equal(run.y.view(torch.int16), first)


def test_grouped_equals_gemv_path_within_tolerance():
    """The two paths are separate kernels; on a shape both serve they agree to the oracle's bar."""
    w = gen.Workload("both_t24_h512_e12_k3_i256", 24, 512, 12, 3, 256, 1, 12, "normal", 55, shared=True)
    xb = gen.activations_bf16(w.seed, 0, w.T, w.H)
    logits = gen.normal_logits(w.seed, 0, w.T, w.E)
    y_ref, *_ = oracle_layer(w, 0, xb, logits=logits)
    L = harness.make_layer(w, 0, DEV, logits=logits, x_bits=xb)
    for flags in (lib.MOE_FORCE_GEMV, lib.MOE_FORCE_GROUPED):
        run = harness.LayerRunner(w, DEV, flags)
        run(L)
        torch.cuda.synchronize()
        assert int(run.status.item()) == 0
        check_close(y_f64(run.y), y_ref, f"  flags {flags}")


# ------------------------------------------------------------------ chunked paged prefill


def paged_arena(w, layer, S):
    stride = lib.moe_slot_stride(w.H, w.I)
    host = torch.empty(w.E * stride, dtype=torch.uint8, pin_memory=True)
    for e in range(w.E):
        host[e * stride : (e + 1) * stride].copy_(torch.from_numpy(harness.pack_expert(w.seed, layer, e, w.H, w.I)))
    slots = torch.empty(S * stride, dtype=torch.uint8, device=DEV)
    table = torch.full((w.E,), -1, dtype=torch.int32, device=DEV)
    arena = lib.Arena(w.E, S, lib.moe_blob_bytes(w.H, w.I), stride, slots, table, host)
    return arena, slots, stride


def resident_grouped(L, w, x, logits, T):
    """The chunk through the fully-resident layer on the grouped path (the bitwise reference)."""
    ids = torch.empty(T, w.K, dtype=torch.int32, device=DEV)
    wts = torch.empty(T, w.K, dtype=torch.float32, device=DEV)
    y = torch.empty(T, w.H, dtype=torch.bfloat16, device=DEV)
    nb = lib.moe_ffn_workspace_bytes(T, w.H, w.I, w.E, w.K, w.shared, lib.MOE_FORCE_GROUPED)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    lib.moe_route(None, None, logits, T, w.H, w.E, w.K, 0, ids, wts)
    lib.moe_expert_ffn(x, ids, wts, T, w.H, w.I, w.E, w.K, 32, L.table, L.slots, L.stride, L.shared, y, ws, nb, st,
                       lib.MOE_FORCE_GROUPED)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return y


@pytest.mark.parametrize("chunk,cap", [(40, 4), (40, 8), (100, 3), (7, 4), (1, 8)])
def test_chunked_paged_prefill_equals_resident(chunk, cap):
    """A 100-token prompt through an 8-slot arena of 32 experts (top-4, shared expert) in chunks:
    every chunk bitwise equal to its fully-resident grouped run, the prompt within the oracle's
    bar, and each chunk fills exactly the experts it uses that were not resident."""
    from quantized_routed_expert_moe_amd.paged import ChunkedPrefill

    w = gen.Workload("chunked_t100_h512_e32s1_k4_i256", 100, 512, 32, 4, 256, 1, 8, "normal", 61, shared=True)
    say(f"chunked paged prefill chunk={chunk} cap={cap}")
    xb = gen.activations_bf16(w.seed, 0, w.T, w.H)
    logits = gen.normal_logits(w.seed, 0, w.T, w.E)
    L = harness.make_layer(w, 0, DEV, logits=logits, x_bits=xb, place_seed=6)
    arena, slots, stride = paged_arena(w, 0, w.slots)
    cp = ChunkedPrefill(arena, slots, stride, w.H, w.I, w.E, w.K, chunk, cap, shared=L.shared, device=DEV)
    y = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=DEV)
    ids_all = R.route(logits, w.K)[0]
    for t0 in range(0, w.T, chunk):
        t1 = min(t0 + chunk, w.T)
        before = set(e for e, s in enumerate(arena.slot_table()) if s >= 0)
        st0 = arena.stats()
        cp.run_chunk(L.x[t0:t1], L.logits[t0:t1], y[t0:t1])
        torch.cuda.synchronize()
        assert int(cp.status.item()) == 0
        used = set(ids_all[t0:t1].ravel().tolist())
        assert sorted(e for p in cp.last_passes for e in p) == sorted(used)
        assert arena.stats()["fills"] - st0["fills"] == len(used - before)
        y_res = resident_grouped(L, w, L.x[t0:t1], L.logits[t0:t1], t1 - t0)
        assert torch.equal(y[t0:t1].view(torch.int16), y_res.view(torch.int16)), (t0, t1)
    y_ref, *_ = oracle_layer(w, 0, xb, logits=logits)
    check_close(y_f64(y), y_ref, f"  chunked prompt chunk={chunk} cap={cap}")


def test_partial_flags_and_combine_errors():
    w = gen.Workload("partial_t8_h256_e8_k2_i256", 8, 256, 8, 2, 256, 1, 8, "normal", 62, shared=True)
    L = harness.make_layer(w, 0, DEV)
    run = harness.LayerRunner(w, DEV, lib.MOE_FFN_PARTIAL)
    run.route(L)
    args = (L.x, run.ids, run.wts, w.T, w.H, w.I, w.E, w.K, 32, L.table, L.slots, L.stride)
    for flags, shared in ((lib.MOE_FFN_PARTIAL | lib.MOE_FORCE_GEMV, L.shared), (lib.MOE_FFN_PARTIAL_SHARED, L.shared),
                          (lib.MOE_FFN_PARTIAL | lib.MOE_FFN_PARTIAL_SHARED, None), (lib.MOE_FFN_PARTIAL_FIRST, L.shared)):
        with pytest.raises(lib.MoeError) as ex:
            lib.moe_expert_ffn(*args, shared, run.y, run.ws, run.ws_bytes, run.status, flags)
        assert ex.value.status == lib.MOE_EINVAL
    with pytest.raises(lib.MoeError) as ex:
        lib.moe_ffn_combine(run.ids, run.wts, w.T, w.H, w.I, w.E, w.K, 1, run.y, run.ws, run.ws_bytes - 1, run.status)
    assert ex.value.status == lib.MOE_EWS
    with pytest.raises(lib.MoeError) as ex:
        lib.moe_ffn_combine(None, run.wts, w.T, w.H, w.I, w.E, w.K, 1, run.y, run.ws, run.ws_bytes, run.status)
    assert ex.value.status == lib.MOE_EINVAL
    raw = lib.load().moe_ffn_combine  # the binding maps has_shared to 0 / 1; the C ABI takes only those
    assert raw(run.ids.data_ptr(), run.wts.data_ptr(), w.T, w.H, w.I, w.E, w.K, 2, run.y.data_ptr(),
               run.ws.data_ptr(), run.ws_bytes, run.status.data_ptr(), None) == lib.MOE_EINVAL
    lib.moe_ffn_combine(run.ids, run.wts, 0, w.H, w.I, w.E, w.K, 1, None, None, 0, None)  # T = 0: a no-op
    # one partial pass with every expert resident, then the combine: the plain grouped result
    first = lib.MOE_FFN_PARTIAL | lib.MOE_FFN_PARTIAL_SHARED | lib.MOE_FFN_PARTIAL_FIRST
    lib.moe_expert_ffn(*args, L.shared, run.y, run.ws, run.ws_bytes, run.status, first)
    lib.moe_ffn_combine(run.ids, run.wts, w.T, w.H, w.I, w.E, w.K, 1, run.y, run.ws, run.ws_bytes, run.status)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    y_res = resident_grouped(L, w, L.x, L.logits, w.T)
    assert torch.equal(run.y.view(torch.int16), y_res.view(torch.int16))


def test_combine_reports_pairs_no_pass_computed():
    """Exact or explicit failure for chunked passes: a pair whose expert no pass of the
    chunk computed, a shared expert no pass computed, and a combine with no first pass
    since the previous one each set the status word; the complete run still gives the
    resident bits afterwards on the same workspace."""
    w = gen.Workload("partial_t40_h256_e8_k2_i256_shared", 40, 256, 8, 2, 256, 1, 8, "normal", 63, shared=True)
    L = harness.make_layer(w, 0, DEV)
    run = harness.LayerRunner(w, DEV, lib.MOE_FFN_PARTIAL)
    run.route(L)
    torch.cuda.synchronize()
    used = sorted(set(run.ids.cpu().numpy().ravel().tolist()))
    assert len(used) >= 3
    args = (L.x, run.ids, run.wts, w.T, w.H, w.I, w.E, w.K, 32)
    full = L.table.clone()

    def table_of(experts):
        t = torch.full_like(full, -1)
        for e in experts:
            t[e] = full[e]
        return t

    def passes(tables, shared_pass=0, first=True):
        for p, tb in enumerate(tables):
            fl = lib.MOE_FFN_PARTIAL | (lib.MOE_FFN_PARTIAL_FIRST if first and p == 0 else 0)
            fl |= lib.MOE_FFN_PARTIAL_SHARED if p == shared_pass else 0
            lib.moe_expert_ffn(*args, tb, L.slots, L.stride, L.shared, run.y, run.ws, run.ws_bytes, run.status, fl)
        lib.moe_ffn_combine(run.ids, run.wts, w.T, w.H, w.I, w.E, w.K, 1, run.y, run.ws, run.ws_bytes, run.status)
        torch.cuda.synchronize()
        st = int(run.status.item())
        run.status.zero_()
        return st

    half = len(used) // 2
    # two passes covering every used expert: no error, and the resident bits
    assert passes([table_of(used[:half]), table_of(used[half:])]) == 0
    y_res = resident_grouped(L, w, L.x, L.logits, w.T)
    assert torch.equal(run.y.view(torch.int16), y_res.view(torch.int16))
    # the last used expert in no pass
    assert passes([table_of(used[:half]), table_of(used[half:-1])]) == lib.MOE_ENOTRES
    # every routed expert, but the shared expert in no pass
    assert passes([table_of(used)], shared_pass=-1) == lib.MOE_ENOTRES
    # a chunk whose first pass is not flagged: the marks of the previous chunk must not count
    assert passes([table_of(used)], first=False) == lib.MOE_EINVAL
    # and again complete: same bits as the resident run
    assert passes([table_of(used[half:]), table_of(used[:half])], shared_pass=1) == 0
    assert torch.equal(run.y.view(torch.int16), y_res.view(torch.int16))


# ------------------------------------------------------------------ other expert formats


def fmt_layer(fmt, w, layer=0, place_seed=None, experts=None, S=None):
    """Pack seeded experts of format fmt into slots (all E, or ``experts``), a table and a shared blob."""
    stride = lib.moe_fmt_slot_stride(fmt, w.H, w.I)
    ex = list(range(w.E)) if experts is None else list(experts)
    S = S or len(ex)
    order = np.random.default_rng(place_seed).permutation(S)[: len(ex)] if place_seed is not None else np.arange(len(ex))
    slots = torch.zeros(S * stride, dtype=torch.uint8, device=DEV)
    table = np.full(w.E, -1, dtype=np.int32)
    for e, s in zip(ex, order):
        slots[int(s) * stride : (int(s) + 1) * stride].copy_(
            torch.from_numpy(harness.pack_expert_fmt(w.seed, layer, int(e), w.H, w.I, fmt)))
        table[int(e)] = int(s)
    shared = None
    if w.shared:
        shared = torch.from_numpy(harness.pack_expert_fmt(w.seed, layer, gen.SHARED_EXPERT, w.H, w.I, fmt)).to(DEV)
    return slots, torch.from_numpy(table).to(DEV), shared, stride


def fmt_oracle_expert(fmt, w, layer, e):
    bits, g = gen.FMT_BITS_G[fmt]
    return R.Expert(gen.expert_tensors_fmt(w.seed, layer, e, w.H, w.I, fmt), w.H, w.I, g=g, bits=bits)


def fmt_run(fmt, w, slots, table, shared, stride, xb, logits):
    x = harness.bf16_tensor(xb, DEV)
    lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(DEV)
    ids = torch.empty(w.T, w.K, dtype=torch.int32, device=DEV)
    wts = torch.empty(w.T, w.K, dtype=torch.float32, device=DEV)
    y = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=DEV)
    nb = lib.moe_fmt_workspace_bytes(fmt, w.T, w.H, w.I, w.E, w.K, shared is not None)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    lib.moe_route(None, None, lg, w.T, w.H, w.E, w.K, 0, ids, wts)
    lib.moe_expert_ffn_fmt(fmt, x, ids, wts, w.T, w.H, w.I, w.E, w.K, table, slots, stride, shared, y, ws, nb, st)
    torch.cuda.synchronize()
    return ids, wts, y, st, (x, ws, nb)


@pytest.mark.parametrize(
    "fmt,w",
    [
        (gen.FMT_INT8_G32, gen.Workload("fmt8_t1_h512_e16_k4_i256_shared", 1, 512, 16, 4, 256, 1, 16, "normal", 71,
                                        shared=True)),
        (gen.FMT_INT8_G32, gen.Workload("fmt8_t7_h256_e8_k2_i96", 7, 256, 8, 2, 96, 1, 8, "normal", 72)),
        (gen.FMT_INT8_G32, gen.Workload("fmt8_t32_h1024_e32_k8_i512_shared", 32, 1024, 32, 8, 512, 1, 32, "zipf", 73,
                                        shared=True)),
        (gen.FMT_INT4_G128, gen.Workload("fmt4g128_t1_h512_e16_k4_i256_shared", 1, 512, 16, 4, 256, 1, 16, "normal",
                                         74, shared=True)),
        (gen.FMT_INT4_G128, gen.Workload("fmt4g128_t9_h1024_e8_k3_i384", 9, 1024, 8, 3, 384, 1, 8, "normal", 75)),
        (gen.FMT_INT4_G128, gen.Workload("fmt4g128_t32_h2048_e32_k8_i768", 32, 2048, 32, 8, 768, 1, 32, "zipf", 76)),
        (gen.FMT_INT4_G128, gen.Workload("fmt4g128_t77_h1024_e16_k4_i256_shared", 77, 1024, 16, 4, 256, 1, 16,
                                         "normal", 80, shared=True)),
        (gen.FMT_NVFP4, gen.Workload("nvfp4_t1_h512_e16_k4_i256_shared", 1, 512, 16, 4, 256, 1, 16, "normal", 81,
                                     shared=True)),
        (gen.FMT_NVFP4, gen.Workload("nvfp4_t7_h256_e8_k2_i96", 7, 256, 8, 2, 96, 1, 8, "normal", 82)),
        (gen.FMT_NVFP4, gen.Workload("nvfp4_t32_h2048_e32_k8_i768_shared", 32, 2048, 32, 8, 768, 1, 32, "zipf", 83,
                                     shared=True)),
        # more than 9 units per token, and h rows past 128 chunks: the per-pair down kernel and the
        # separate combine instead of the fused down
        (gen.FMT_INT8_G32, gen.Workload("fmt8_t3_h256_e16_k10_i128_shared", 3, 256, 16, 10, 128, 1, 16, "normal", 95,
                                        shared=True)),
        (gen.FMT_INT8_G32, gen.Workload("fmt8_t2_h256_e4_k2_i2560", 2, 256, 4, 2, 2560, 1, 4, "normal", 96)),
        (gen.FMT_NVFP4, gen.Workload("nvfp4_t2_h256_e16_k12_i256", 2, 256, 16, 12, 256, 1, 16, "normal", 97)),
        (gen.FMT_NVFP4, gen.Workload("nvfp4_t2_h256_e4_k2_i4608_shared", 2, 256, 4, 2, 4608, 1, 4, "normal", 98,
                                     shared=True)),
        # prompts (T > 32): the formats' grouped MFMA GEMMs
        (gen.FMT_INT8_G32, gen.Workload("fmt8_t40_h512_e16_k4_i256_shared", 40, 512, 16, 4, 256, 1, 16, "normal", 84,
                                        shared=True)),
        (gen.FMT_INT8_G32, gen.Workload("fmt8_t300_h256_e4_k2_i128", 300, 256, 4, 2, 128, 1, 4, "normal", 85)),
        (gen.FMT_NVFP4, gen.Workload("nvfp4_t77_h1024_e16_k4_i256_shared", 77, 1024, 16, 4, 256, 1, 16, "zipf", 86,
                                     shared=True)),
        (gen.FMT_NVFP4, gen.Workload("nvfp4_t300_h256_e4_k2_i192", 300, 256, 4, 2, 192, 1, 4, "normal", 89)),
    ],
    ids=lambda v: v.name if hasattr(v, "name") else f"fmt{v}",
)
def test_fmt_matches_oracle(fmt, w):
    """INT8 group-32, INT4 group-128 (on every path of moe_expert_ffn, 77 tokens on the
    grouped one) and NVFP4 experts (the fused down of up to 9 units and the per-pair down
    with its combine past that), one token to prompts of 300 (the formats' own grouped
    MFMA GEMMs above 32 tokens, experts over two 128-row tiles, a full and a half one; the
    seeds keep the oracle's bf16 rounding floor below the bar, so the plain bar holds): ids
    bit-exact, y within the oracle's bar, the same bits on a second run and under a
    permuted slot map."""
    say(f"format {fmt} {w.name}")
    xb = gen.activations_bf16(w.seed, 0, w.T, w.H)
    logits = {"normal": gen.normal_logits, "zipf": gen.zipf_logits}[w.router](w.seed, 0, w.T, w.E)
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = fmt_oracle_expert(fmt, w, 0, e)
        return cache[e]

    shared_ref = fmt_oracle_expert(fmt, w, 0, gen.SHARED_EXPERT) if w.shared else None
    y_ref, ids_ref, w_ref, _ = R.moe_layer(xb, expert, w.K, logits=logits, shared=shared_ref)
    outs = []
    for place in (None, 3):
        slots, table, shared, stride = fmt_layer(fmt, w, place_seed=place)
        ids, wts, y, st, _ = fmt_run(fmt, w, slots, table, shared, stride, xb, logits)
        assert int(st.item()) == 0
        assert np.array_equal(ids.cpu().numpy(), ids_ref)
        if place is None:
            check_close(y_f64(y), y_ref, f"  format {fmt} {w.name}")
        outs.append(y.view(torch.int16).clone())
        _, _, y2, _, _ = fmt_run(fmt, w, slots, table, shared, stride, xb, logits)
        assert torch.equal(y2.view(torch.int16), outs[-1])
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("fmt", [gen.FMT_INT8_G32, gen.FMT_INT4_G128, gen.FMT_NVFP4])
def test_fmt_decode_full_size(fmt):
    """One token, 256 experts, top-8, H 4096, I 1536 (the decode shape), the 8 routed experts
    in a 64-slot arena: against the oracle."""
    w = gen.Workload("fmt_decode_t1_h4096_e256_k8_i1536", 1, 4096, 256, 8, 1536, 1, 64, "normal", 77)
    xb = gen.activations_bf16(w.seed, 0, 1, w.H)
    logits = gen.normal_logits(w.seed, 0, 1, w.E)
    ids_ref, _ = R.route(logits, w.K)
    routed = sorted(set(ids_ref.ravel().tolist()))
    say(f"format {fmt} decode: packing {len(routed)} experts")
    slots, table, shared, stride = fmt_layer(fmt, w, place_seed=5, experts=routed, S=w.slots)
    y_ref, _, _, _ = R.moe_layer(xb, {e: fmt_oracle_expert(fmt, w, 0, e) for e in routed}, w.K, logits=logits)
    ids, wts, y, st, _ = fmt_run(fmt, w, slots, table, shared, stride, xb, logits)
    assert int(st.item()) == 0
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    check_close(y_f64(y), y_ref, f"  format {fmt} decode full size")


def test_nvfp4_every_e4m3_scale():
    """NVFP4 experts whose group scales run through all 254 finite E4M3 codes (zero, the
    subnormals, up to 448, both signs), with small global scales and activations so that h
    stays in fp16: one token through 8 experts against the oracle."""
    H, I, E, K = 64, 64, 8, 8
    say("nvfp4 with every finite E4M3 scale")
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)
    assert finite.size == 254
    rng = np.random.default_rng(41)
    stride = lib.moe_fmt_slot_stride(gen.FMT_NVFP4, H, I)
    slots = torch.zeros(E * stride, dtype=torch.uint8, device=DEV)
    experts = {}
    pos = 0
    for e in range(E):
        def scales(rows, cols):
            nonlocal pos
            n = rows * (cols // 16)
            out = finite[(pos + np.arange(n)) % finite.size].reshape(rows, cols // 16)
            pos += n
            return out
        t = {"qg": rng.integers(0, 256, size=(I, H // 2), dtype=np.uint8),
             "qu": rng.integers(0, 256, size=(I, H // 2), dtype=np.uint8),
             "qd": rng.integers(0, 256, size=(H, I // 2), dtype=np.uint8),
             "sg": scales(I, H), "su": scales(I, H), "sd": scales(H, I),
             "global": np.full(3, 2.0**-8, dtype=np.float32)}
        blob = np.zeros(stride, dtype=np.uint8)
        lib.moe_pack_expert_nvfp4(t["qg"], t["qu"], t["qd"], t["sg"], t["su"], t["sd"], t["global"], H, I, blob)
        slots[e * stride : (e + 1) * stride].copy_(torch.from_numpy(blob))
        experts[e] = R.Expert(t, H, I, g=16, bits=4)
    assert pos >= 3 * finite.size  # every code in several matrices
    table = torch.arange(E, dtype=torch.int32, device=DEV)
    xb = gen.bf16_bits_from_f32((rng.standard_normal((1, H)) * 0.125).astype(np.float32))
    logits = rng.standard_normal((1, E)).astype(np.float32)
    w = gen.Workload("nvfp4_all_e4m3_t1_h64_e8_k8_i64", 1, H, E, K, I, 1, E, "normal", 0)
    y_ref, ids_ref, _, _ = R.moe_layer(xb, experts.__getitem__, K, logits=logits)
    ids, _, y, st, _ = fmt_run(gen.FMT_NVFP4, w, slots, table, None, stride, xb, logits)
    assert int(st.item()) == 0
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    check_close(y_f64(y), y_ref, "  nvfp4 every E4M3 scale")


def test_fmt_status_and_argument_errors():
    fmt = gen.FMT_INT8_G32
    w = gen.Workload("fmt8_t3_h256_e8_k2_i96_err", 3, 256, 8, 2, 96, 1, 8, "normal", 78, shared=True)
    xb = gen.activations_bf16(w.seed, 0, w.T, w.H)
    logits = gen.normal_logits(w.seed, 0, w.T, w.E)
    slots, table, shared, stride = fmt_layer(fmt, w)
    ids, wts, y, st, (x, ws, nb) = fmt_run(fmt, w, slots, table, shared, stride, xb, logits)
    assert int(st.item()) == 0
    e0 = int(ids[0, 0].item())
    table[e0] = -1
    lib.moe_expert_ffn_fmt(fmt, x, ids, wts, w.T, w.H, w.I, w.E, w.K, table, slots, stride, shared, y, ws, nb, st)
    torch.cuda.synchronize()
    assert int(st.item()) == lib.MOE_ENOTRES
    st.zero_()
    table[e0] = 0
    ids[1, 1] = w.E
    lib.moe_expert_ffn_fmt(fmt, x, ids, wts, w.T, w.H, w.I, w.E, w.K, table, slots, stride, shared, y, ws, nb, st)
    torch.cuda.synchronize()
    assert int(st.item()) in (lib.MOE_EINVAL, lib.MOE_ENOTRES)
    args = (x, ids, wts, w.T, w.H, w.I, w.E, w.K, table, slots, stride, shared, y, ws, nb, st)
    for bad_fmt, code in ((7, lib.MOE_EINVAL),):
        with pytest.raises(lib.MoeError) as ex:
            lib.moe_expert_ffn_fmt(bad_fmt, *args)
        assert ex.value.status == code
    with pytest.raises(lib.MoeError) as ex:  # 33 tokens with I = 96: the prompt GEMM takes multiples of 64
        lib.moe_expert_ffn_fmt(fmt, x, ids, wts, 33, w.H, w.I, w.E, w.K, table, slots, stride, shared, y, ws, nb, st)
    assert ex.value.status == lib.MOE_EUNSUP
    assert lib.moe_fmt_workspace_bytes(fmt, 33, w.H, w.I, w.E, w.K, True) == 0
    with pytest.raises(lib.MoeError) as ex:
        lib.moe_expert_ffn_fmt(fmt, x, ids, wts, w.T, w.H, w.I, w.E, w.K, table, slots, stride, shared, y, ws, nb - 1, st)
    assert ex.value.status == lib.MOE_EWS
    with pytest.raises(lib.MoeError) as ex:
        lib.moe_expert_ffn_fmt(fmt, x, ids, wts, w.T, w.H, w.I, w.E, w.K, table, slots, 100, shared, y, ws, nb, st)
    assert ex.value.status == lib.MOE_EINVAL


def test_fmt_int4_g32_is_moe_expert_ffn():
    w = gen.Workload("fmt4g32_t5_h512_e16_k4_i256_shared", 5, 512, 16, 4, 256, 1, 16, "normal", 79, shared=True)
    L = harness.make_layer(w, 0, DEV, place_seed=1)
    run = harness.LayerRunner(w, DEV)
    run.route(L)
    run.ffn(L)
    torch.cuda.synchronize()
    y0 = run.y.view(torch.int16).clone()
    lib.moe_expert_ffn_fmt(gen.FMT_INT4_G32, L.x, run.ids, run.wts, w.T, w.H, w.I, w.E, w.K, L.table, L.slots,
                           L.stride, L.shared, run.y, run.ws, run.ws_bytes, run.status)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    assert torch.equal(run.y.view(torch.int16), y0)


# ------------------------------------------------------------------ read-ahead decode


@pytest.mark.parametrize(
    "predict,wrong,native,speculate,host_poll",
    [(0, False, False, False, False), (4, False, False, False, False), (0, False, True, True, True),
     (4, False, True, True, True), (8, False, True, True, True), (4, False, True, False, True),
     (4, True, True, True, True), (4, True, False, False, False), (4, False, True, True, False)],
    ids=["py_off", "py_p4", "native_spec_off", "native_spec_p4", "native_spec_p8", "native_p4",
         "native_spec_p4_wrong_predictor", "py_p4_wrong_predictor", "native_spec_p4_event"])
def test_readahead_paged_decode(predict, wrong, native, speculate, host_poll):
    """PagedDecode through 4 layers with 8-slot arenas, routed by per-layer router GEMVs on a
    residual stream, reading ahead the next layer's top-P (from its router or from an unrelated
    matrix), sequenced in Python or by moe_paged_layer (with or without the speculative FFN; the
    ids reach the host through the polled word, or through a copy and an event):
    every layer's output bitwise equal to the fully-resident run, ids equal to the oracle's
    selection on its own GEMV logits, the last token within the oracle's bar, and each arena's
    stats equal to the slot-policy model replayed on the logged calls."""
    from oracle.arena_ref import ArenaModel
    from quantized_routed_expert_moe_amd import paged

    w = gen.Workload("readahead_t1_h512_e32s1_k4_i256_x4", 1, 512, 32, 4, 256, 4, 8, "residual", 91, shared=True)
    steps = 10
    say(f"read-ahead decode predict={predict} wrong={wrong} native={native} speculate={speculate}")
    xs_bits = gen.residual_stream(w.seed, steps, w.layers, w.H, a=0.9, rho=0.2)
    stride, blob = lib.moe_slot_stride(w.H, w.I), lib.moe_blob_bytes(w.H, w.I)
    layers, routers, preds, shared, resident = [], [], [], [], []
    for l in range(w.layers):
        host = torch.empty(w.E * stride, dtype=torch.uint8, pin_memory=True)
        for e in range(w.E):
            host[e * stride : e * stride + blob].copy_(torch.from_numpy(harness.pack_expert(w.seed, l, e, w.H, w.I)))
        slots = torch.empty(w.slots * stride, dtype=torch.uint8, device=DEV)
        table = torch.full((w.E,), -1, dtype=torch.int32, device=DEV)
        layers.append((lib.Arena(w.E, w.slots, blob, stride, slots, table, host), slots, table))
        routers.append(torch.from_numpy(gen.router_weight(w.seed, l, w.E, w.H)).to(DEV))
        preds.append(torch.from_numpy(gen.router_weight(w.seed + 1000, l, w.E, w.H)).to(DEV) if wrong else routers[-1])
        shared.append(torch.from_numpy(harness.pack_expert(w.seed, l, gen.SHARED_EXPERT, w.H, w.I)).to(DEV))
        resident.append((host.to(DEV), torch.arange(w.E, dtype=torch.int32, device=DEV)))
    dec = paged.PagedDecode(layers, routers, stride, w.H, w.I, w.E, w.K, shared=shared, predict=predict,
                            device=DEV, predictors=preds, native=native, speculate=speculate, host_poll=host_poll)
    dec.log = []
    y = torch.empty(1, w.H, dtype=torch.bfloat16, device=DEV)
    y_res = torch.empty_like(y)
    ws2 = torch.empty_like(dec.ws)
    for t in range(steps):
        for l in range(w.layers):
            x = harness.bf16_tensor(xs_bits[t, l][None, :], DEV)
            dec.layer(l, x, y)
            ids_d, wts_d = dec.routed
            lib.moe_expert_ffn(x, ids_d, wts_d, 1, w.H, w.I, w.E, w.K, 32, resident[l][1], resident[l][0], stride,
                               shared[l], y_res, ws2, dec.ws_bytes, dec.status)
            torch.cuda.synchronize()
            assert int(dec.status.item()) == 0
            assert torch.equal(y.view(torch.int16), y_res.view(torch.int16)), (t, l)
            wr = gen.router_weight(w.seed, l, w.E, w.H)
            ids_ref, _ = R.route(R.router_logits(xs_bits[t, l][None, :], wr), w.K)
            assert np.array_equal(ids_d.cpu().numpy(), ids_ref), (t, l)
            if t == steps - 1:
                sh = R.Expert(gen.expert_tensors(w.seed, l, gen.SHARED_EXPERT, w.H, w.I), w.H, w.I)
                y_ref, _, _, _ = R.moe_layer(xs_bits[t, l][None, :], OracleExperts(w, l), w.K, w_router=wr, shared=sh)
                check_close(y_f64(y), y_ref, f"  read-ahead layer {l}")
    models = [ArenaModel(w.E, w.slots, blob) for _ in range(w.layers)]
    for op, l, ids in dec.log:
        if op == "map":
            assert models[l].map_slots(ids)[0] == 0
        else:
            assert models[l].prefetch(ids)[0] == 0
    for l in range(w.layers):
        st = layers[l][0].stats()
        assert st == models[l].stats, l
        say(f"  layer {l}: {st}")
    n_pre = sum(layers[l][0].stats()["prefetch_fills"] for l in range(w.layers))
    if predict:
        assert n_pre > 0 and sum(1 for op, _, _ in dec.log if op == "pre") == steps * (w.layers - 1)
    else:
        assert n_pre == 0
    if predict and not wrong:
        assert sum(layers[l][0].stats()["prefetch_hits"] for l in range(w.layers)) > 0


def test_paged_layer_argument_errors():
    """moe_paged_layer rejects a bookkeeping-only arena, the next layer's arena equal to its
    own, E other than the arena's, K above the slots, a short workspace and unknown flags,
    before launching anything."""
    H, I, E, K, S = 256, 128, 16, 4, 6
    stride, blob = lib.moe_slot_stride(H, I), lib.moe_blob_bytes(H, I)
    host = torch.zeros(E * stride, dtype=torch.uint8, pin_memory=True)

    def arena():
        sl = torch.zeros(S * stride, dtype=torch.uint8, device=DEV)
        tb = torch.full((E,), -1, dtype=torch.int32, device=DEV)
        return lib.Arena(E, S, blob, stride, sl, tb, host), sl, tb

    (a0, _, _), (a1, _, _) = arena(), arena()
    wr = torch.zeros(E, H, dtype=torch.float32, device=DEV)
    d0, d1 = lib.paged_layer_desc(a0, wr), lib.paged_layer_desc(a1, wr)
    x = torch.zeros(1, H, dtype=torch.bfloat16, device=DEV)
    y = torch.empty_like(x)
    logits = torch.empty(E, dtype=torch.float32, device=DEV)
    ids = torch.empty(2 * K, dtype=torch.int32, device=DEV)
    wts = torch.empty(2 * K, dtype=torch.float32, device=DEV)
    ids_h = torch.empty(2 * K, dtype=torch.int32, pin_memory=True)
    nb = lib.moe_paged_workspace_bytes(H, I, E, K, 0)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    side, ev = torch.cuda.Stream(), torch.cuda.Event()
    ev.record()
    torch.cuda.synchronize()

    def call(layer=d0, nxt=d1, P=K, E_=E, K_=K, nbytes=nb, flags=lib.MOE_PAGED_SPECULATE):
        with pytest.raises(lib.MoeError) as ex:
            lib.moe_paged_layer(layer, nxt, wr, P, x, H, I, E_, K_, 32, logits, ids, wts, ids_h, y, ws, nbytes, st,
                                flags, None, side, ev)
        return ex.value.status

    book = lib.Arena(E, S, blob, stride)  # no device buffers
    assert call(layer=lib.paged_layer_desc(book, wr)) == lib.MOE_EINVAL
    assert call(nxt=lib.paged_layer_desc(book, wr)) == lib.MOE_EINVAL
    assert call(nxt=d0) == lib.MOE_EINVAL
    assert call(E_=E + 1) == lib.MOE_EINVAL
    assert call(K_=S + 1) == lib.MOE_EINVAL
    assert call(P=S + 1) == lib.MOE_EINVAL
    assert call(nbytes=nb - 1) == lib.MOE_EWS
    assert call(flags=4) == lib.MOE_EINVAL
    torch.cuda.synchronize()
    assert a0.stats()["fills"] == 0 and a1.stats()["fills"] == 0 and int(st.item()) == 0


@pytest.mark.parametrize("speculate", [False, True], ids=["wait", "speculate"])
def test_paged_layer_logits_in_at_budget_top_k(speculate):
    """moe_paged_layer on supplied logits (no router) through arenas of S = K slots, every map
    a likely miss: each step bitwise equal to the fully-resident run, the stats equal to the
    slot-policy model on the same ids."""
    from oracle.arena_ref import ArenaModel
    from quantized_routed_expert_moe_amd import paged

    w = gen.Workload("paged_t1_h1024_e32s1_k4_i512_native", 1, 1024, 32, 4, 512, 2, 4, "locality", 42, shared=True)
    steps = 20
    say(f"paged layer, logits in, speculate={speculate}")
    lg = torch.from_numpy(gen.locality_logits(w.seed, w.layers, steps, w.E, w.K)).to(DEV)
    stride, blob = lib.moe_slot_stride(w.H, w.I), lib.moe_blob_bytes(w.H, w.I)
    layers, shared, resident, xs = [], [], [], []
    for l in range(w.layers):
        host = torch.empty(w.E * stride, dtype=torch.uint8, pin_memory=True)
        for e in range(w.E):
            host[e * stride : e * stride + blob].copy_(torch.from_numpy(harness.pack_expert(w.seed, l, e, w.H, w.I)))
        slots = torch.empty(w.slots * stride, dtype=torch.uint8, device=DEV)
        table = torch.full((w.E,), -1, dtype=torch.int32, device=DEV)
        layers.append((lib.Arena(w.E, w.slots, blob, stride, slots, table, host), slots, table))
        shared.append(torch.from_numpy(harness.pack_expert(w.seed, l, gen.SHARED_EXPERT, w.H, w.I)).to(DEV))
        resident.append((host.to(DEV), torch.arange(w.E, dtype=torch.int32, device=DEV)))
        xs.append(harness.bf16_tensor(gen.activations_bf16(w.seed, l, 1, w.H), DEV))
    dec = paged.PagedDecode(layers, [None] * w.layers, stride, w.H, w.I, w.E, w.K, shared=shared, device=DEV,
                            native=True, speculate=speculate)
    dec.log = []
    y = torch.empty(1, w.H, dtype=torch.bfloat16, device=DEV)
    y_res = torch.empty_like(y)
    ws2 = torch.empty_like(dec.ws)
    for s in range(steps):
        for l in range(w.layers):
            dec.layer(l, xs[l], y, lg[s, l])
            ids_d, wts_d = dec.routed
            lib.moe_expert_ffn(xs[l], ids_d, wts_d, 1, w.H, w.I, w.E, w.K, 32, resident[l][1], resident[l][0],
                               stride, shared[l], y_res, ws2, dec.ws_bytes, dec.status)
            torch.cuda.synchronize()
            assert int(dec.status.item()) == 0
            assert torch.equal(y.view(torch.int16), y_res.view(torch.int16)), (s, l)
            assert ids_d.cpu().numpy().tolist()[0] == R.route(lg[s, l][None, :].cpu().numpy(), w.K)[0][0].tolist()
    models = [ArenaModel(w.E, w.slots, blob) for _ in range(w.layers)]
    for op, l, ids in dec.log:
        assert op == "map" and models[l].map_slots(ids)[0] == 0
    for l in range(w.layers):
        assert layers[l][0].stats() == models[l].stats
        assert models[l].stats["misses"] > steps  # the arena really pages
