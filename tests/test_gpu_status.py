"""Exact or explicit failure on the GPU ("Strata" README, the execution rules: a run
completes the exact computation or reports a failure).

The single-token decode, batched, grouped (MFMA) and INT8 / NVFP4 paths stage x and
the intermediate h as fp16 operands; a value outside the fp16 range must set
MOE_EUNSUP in the device status word rather than be clamped. Each path is driven
with an activation past the range (one element of 2^17) and with activations whose h
overflows fp16 (x = +-1000, checked with the oracle first). The GEMV path keeps x in
bf16 and h in fp32, so the same activations compute there, against the oracle. A
speculative FFN whose result moe_paged_layer keeps reports its status too.
"""

import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from quantized_routed_expert_moe_amd import harness, lib
from synth import gen

from parity_util import DEV, check_close, oracle_layer, say, y_f64

pytestmark = pytest.mark.gpu

FP16_MAX = 65504.0


def big_x(kind, T, H, seed):
    """bf16 bits: "x" = N(0,1) with one element 2^17 (past fp16); "h" = +-1000 (fits fp16)."""
    rng = np.random.default_rng(seed)
    if kind == "x":
        x = rng.standard_normal((T, H)).astype(np.float32)
        x[0, 5] = 2.0**17
    else:
        x = np.where(rng.random((T, H)) < 0.5, -1000.0, 1000.0).astype(np.float32)
    return gen.bf16_bits_from_f32(x)


def max_h(expert, x_bits, ids):
    """Largest |h| = |silu(Wg x) * (Wu x)| over the routed pairs, from the oracle's matrices."""
    x = R.bf16_bits_to_f64(x_bits)
    m = 0.0
    for t in range(ids.shape[0]):
        for e in ids[t]:
            ex = expert(int(e))
            m = max(m, float(np.abs(R.silu(ex.Wg @ x[t]) * (ex.Wu @ x[t])).max()))
    return m


PATHS = {  # name: (T, flags); int4 group-32 experts, H 256, I 512, 8 experts, top-2, a shared expert
    "decode_t1": (1, 0),
    "batched_t5": (5, 0),
    "grouped_t40": (40, 0),
    "grouped_forced_t3": (3, lib.MOE_FORCE_GROUPED),
}


@pytest.mark.parametrize("kind", ["x", "h"])
@pytest.mark.parametrize("path", list(PATHS))
def test_int4_paths_report_fp16_overflow(path, kind):
    T, flags = PATHS[path]
    w = gen.Workload(f"status_{path}", T, 256, 8, 2, 512, 1, 8, "normal", 301, shared=True)
    xb = big_x(kind, T, w.H, 7)
    logits = gen.normal_logits(w.seed, 0, T, w.E)
    ids_ref, _ = R.route(logits, w.K)
    if kind == "h":
        from parity_util import OracleExperts

        assert max_h(OracleExperts(w, 0), xb, ids_ref) > FP16_MAX  # the premise: h leaves the fp16 range
    say(f"fp16 range {path} {kind}")
    L = harness.make_layer(w, 0, DEV, logits=logits, x_bits=xb)
    run = harness.LayerRunner(w, DEV, flags)
    run(L)
    torch.cuda.synchronize()
    assert np.array_equal(run.ids.cpu().numpy(), ids_ref)
    assert int(run.status.item()) == lib.MOE_EUNSUP


@pytest.mark.parametrize("kind", ["x", "h"])
def test_moe_layer_single_token_reports_fp16_overflow(kind):
    """moe_layer on one token (slots resolved in the routing kernel) with the router GEMV."""
    w = gen.Workload("status_layer_t1", 1, 256, 16, 4, 512, 1, 16, "gemv", 302)
    xb = big_x(kind, 1, w.H, 8)
    L = harness.make_layer(w, 0, DEV, x_bits=xb)
    run = harness.LayerRunner(w, DEV)
    run.layer(L)
    torch.cuda.synchronize()
    assert int(run.status.item()) == lib.MOE_EUNSUP


@pytest.mark.parametrize("fmt", [gen.FMT_INT8_G32, gen.FMT_NVFP4])
@pytest.mark.parametrize("kind", ["x", "h"])
@pytest.mark.parametrize("T", [1, 5])
def test_format_paths_report_fp16_overflow(fmt, kind, T):
    from test_gpu_parity import fmt_layer, fmt_oracle_expert, fmt_run

    w = gen.Workload(f"status_fmt{fmt}_t{T}", T, 256, 8, 2, 512, 1, 8, "normal", 303, shared=True)
    xb = big_x(kind, T, w.H, 9)
    logits = gen.normal_logits(w.seed, 0, T, w.E)
    if kind == "h":
        ids_ref, _ = R.route(logits, w.K)
        assert max_h(lambda e: fmt_oracle_expert(fmt, w, 0, e), xb, ids_ref) > FP16_MAX
    say(f"fp16 range format {fmt} T={T} {kind}")
    slots, table, shared, stride = fmt_layer(fmt, w)
    _, _, _, st, _ = fmt_run(fmt, w, slots, table, shared, stride, xb, logits)
    assert int(st.item()) == lib.MOE_EUNSUP


@pytest.mark.parametrize("T,H,I", [(1, 256, 96), (5, 96, 2080)])
def test_gemv_path_computes_large_activations(T, H, I):
    """The general GEMV kernels (bf16 x, fp32 h; the shapes the single-token and batched
    kernels do not take: I / 32 not a multiple of 16 for one token, I / 32 above 64 for
    several) compute activations whose h overflows fp16, against the oracle."""
    from parity_util import OracleExperts

    w = gen.Workload(f"large_x_gemv_t{T}_h{H}_i{I}", T, H, 8, 2, I, 1, 8, "normal", 304, shared=True)
    xb = big_x("h", T, w.H, 10)
    logits = gen.normal_logits(w.seed, 0, T, w.E)
    y_ref, ids_ref, _, _ = oracle_layer(w, 0, xb, logits=logits)
    assert max_h(OracleExperts(w, 0), xb, ids_ref) > FP16_MAX
    L = harness.make_layer(w, 0, DEV, logits=logits, x_bits=xb)
    run = harness.LayerRunner(w, DEV, lib.MOE_FORCE_GEMV)
    run(L)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    assert np.array_equal(run.ids.cpu().numpy(), ids_ref)
    check_close(y_f64(run.y), y_ref, f"  GEMV path, x = +-1000, T={T}")


def test_paged_layer_speculative_result_keeps_its_status():
    """moe_paged_layer with MOE_PAGED_SPECULATE: a layer whose experts are all resident
    keeps the speculative FFN's result, and with it that FFN's status word: an activation
    past the fp16 range must reach dev_status (and a normal one must leave it zero)."""
    from quantized_routed_expert_moe_amd import paged

    H, I, E, K, S = 512, 512, 16, 4, 8
    w = gen.Workload("status_paged_t1_h512_e16s1_k4_i512", 1, H, E, K, I, 1, S, "normal", 305, shared=True)
    stride, blob = lib.moe_slot_stride(H, I), lib.moe_blob_bytes(H, I)
    host = torch.empty(E * stride, dtype=torch.uint8, pin_memory=True)
    for e in range(E):
        host[e * stride : e * stride + blob].copy_(torch.from_numpy(harness.pack_expert(w.seed, 0, e, H, I)))
    slots = torch.empty(S * stride, dtype=torch.uint8, device=DEV)
    table = torch.full((E,), -1, dtype=torch.int32, device=DEV)
    arena = lib.Arena(E, S, blob, stride, slots, table, host)
    shared = torch.from_numpy(harness.pack_expert(w.seed, 0, gen.SHARED_EXPERT, H, I)).to(DEV)
    dec = paged.PagedDecode([(arena, slots, table)], [None], stride, H, I, E, K, shared=[shared], device=DEV,
                            native=True, speculate=True)
    logits = torch.from_numpy(gen.normal_logits(w.seed, 0, 1, E)[0]).to(DEV)
    y = torch.empty(1, H, dtype=torch.bfloat16, device=DEV)
    x_ok = harness.bf16_tensor(gen.activations_bf16(w.seed, 0, 1, H), DEV)
    x_bad = harness.bf16_tensor(big_x("x", 1, H, 11), DEV)
    for step, (x, want, misses) in enumerate([(x_ok, 0, True), (x_ok, 0, False), (x_bad, lib.MOE_EUNSUP, False),
                                              (x_ok, 0, False)]):
        st0 = arena.stats()
        dec.layer(0, x, y, logits)
        torch.cuda.synchronize()
        st1 = arena.stats()
        say(f"  step {step}: misses {st1['misses'] - st0['misses']}, status {int(dec.status.item())}")
        assert (st1["misses"] > st0["misses"]) == misses  # no miss: the speculative result is the one kept
        assert int(dec.status.item()) == want, step
        dec.status.zero_()


def test_batched_reports_scale_past_fp16_product_range():
    """The small-batch path forms fp16(q * s) as its MFMA operand; a group scale of
    magnitude >= 8192 could overflow that product and must set MOE_EUNSUP. One scale
    (gate, row 0, group 0) of a routed expert is set to 8192 in the arena."""
    T = 6
    w = gen.Workload("status_batched_scale", T, 256, 8, 2, 512, 1, 8, "normal", 302)
    logits = gen.normal_logits(w.seed, 0, T, w.E)
    ids_ref, _ = R.route(logits, w.K)
    L = harness.make_layer(w, 0, DEV, logits=logits)
    e = int(ids_ref[0, 0])
    slot = int(L.table[e].item())
    gate_scales = 3 * w.H * w.I // 2  # codes of gate, up and down come first in the blob
    off = slot * L.stride + gate_scales
    L.slots[off:off + 2] = torch.tensor([0x00, 0x70], dtype=torch.uint8, device=DEV)  # fp16 8192, little-endian
    say("batched scale 8192")
    run = harness.LayerRunner(w, DEV)
    run(L)
    torch.cuda.synchronize()
    assert np.array_equal(run.ids.cpu().numpy(), ids_ref)
    assert int(run.status.item()) == lib.MOE_EUNSUP


def test_grouped_reports_term_past_fp16_store():
    """The grouped path stores each routed term o in fp16; a term past the fp16 range
    must set MOE_EUNSUP. Every down scale of one routed expert is set to 8000 (below the
    operand guard of 8192): with I = 512 codes of magnitude up to 8 against h of order
    one, that expert's o is far past 65504."""
    T = 40
    w = gen.Workload("status_grouped_o", T, 256, 8, 2, 512, 1, 8, "normal", 305)
    logits = gen.normal_logits(w.seed, 0, T, w.E)
    ids_ref, _ = R.route(logits, w.K)
    L = harness.make_layer(w, 0, DEV, logits=logits)
    e = int(ids_ref[0, 0])
    slot = int(L.table[e].item())
    mat_scales = w.H * w.I // 32 * 2
    down_scales = 3 * w.H * w.I // 2 + 2 * mat_scales  # codes of the three matrices, then gate and up scales
    off = slot * L.stride + down_scales
    L.slots[off:off + mat_scales] = torch.tensor([0xD0, 0x6F], dtype=torch.uint8, device=DEV).repeat(mat_scales // 2)
    say("grouped o past fp16")
    run = harness.LayerRunner(w, DEV)
    run(L)
    torch.cuda.synchronize()
    assert np.array_equal(run.ids.cpu().numpy(), ids_ref)
    assert int(run.status.item()) == lib.MOE_EUNSUP


def test_int8_prompt_reports_scale_past_fp16_product_range():
    """The INT8 prompt GEMM forms fp16(q * s) as its MFMA operand (|q| <= 128); a group
    scale of magnitude >= 512 could overflow that product and must set MOE_EUNSUP. One
    gate scale of the expert every token picks first is set to 600 in the arena."""
    from test_gpu_parity import fmt_layer, fmt_run

    fmt = gen.FMT_INT8_G32
    w = gen.Workload("status_int8_prompt_scale", 48, 256, 8, 2, 128, 1, 8, "normal", 306)
    xb = gen.activations_bf16(w.seed, 0, w.T, w.H)
    logits = gen.normal_logits(w.seed, 0, w.T, w.E)
    ids_ref, _ = R.route(logits, w.K)
    slots, table, shared, stride = fmt_layer(fmt, w)
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731  (regions of the format blob start on 256 bytes)
    mat = w.I * w.H  # int8 codes of gate / up / down
    gate_scales = al(al(al(mat) + mat) + mat)
    off = int(table[int(ids_ref[0, 0])].item()) * stride + gate_scales
    slots[off:off + 2] = torch.tensor([0xB0, 0x60], dtype=torch.uint8, device=DEV)  # fp16 600, little-endian
    say("int8 prompt scale 600")
    ids, _, _, st, _ = fmt_run(fmt, w, slots, table, shared, stride, xb, logits)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert int(st.item()) == lib.MOE_EUNSUP
