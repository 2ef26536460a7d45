"""moe_layer_noalloc (the entry point that allocates nothing) against moe_layer with a
caller workspace, through the C ABI: two calls in a row, the second with a smaller input,
each bitwise equal to moe_layer (the same kernels) and within the oracle's bar; sizes past
the fixed workspace and the partial-pass flags are rejected before anything is enqueued."""

import numpy as np
import pytest
import torch

from quantized_routed_expert_moe_amd import harness, lib
from synth import gen

from parity_util import DEV, check_close, oracle_layer, say, y_f64

pytestmark = pytest.mark.gpu


def both_entry_points(w, layer=0):
    xb = gen.activations_bf16(w.seed, layer, w.T, w.H)
    L = harness.make_layer(w, layer, DEV, x_bits=xb, place_seed=5)
    run = harness.LayerRunner(w, DEV)
    run.layer(L)  # moe_layer with the caller's workspace
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    want = (L.logits.clone(), run.ids.clone(), run.wts.clone(), run.y.clone())
    logits = torch.full_like(L.logits, float("nan"))
    ids = torch.full_like(run.ids, -1)
    wts = torch.full_like(run.wts, float("nan"))
    y = torch.full_like(run.y, float("nan"))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    lib.moe_layer_noalloc(L.x, L.wr, logits, w.T, w.H, w.I, w.E, w.K, w.g, 0, ids, wts, L.table, L.slots, L.stride,
                          L.shared, y, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for a, b in zip((logits, ids, wts, y), want):
        assert torch.equal(a.view(torch.int32 if a.element_size() == 4 else torch.int16),
                           b.view(torch.int32 if b.element_size() == 4 else torch.int16))
    y_ref, ids_ref, _, _ = oracle_layer(w, layer, xb)
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    check_close(y_f64(y), y_ref, f"  moe_layer_noalloc {w.name}")


def test_noalloc_layer_equals_moe_layer_twice_then_smaller():
    say(f"scratch bytes per GPU: {lib.moe_noalloc_scratch_bytes()}")
    # first call: 40 tokens on the grouped (MFMA) path, a shared expert
    both_entry_points(gen.Workload("noalloc_t40_h512_e16_k4_i256_shared", 40, 512, 16, 4, 256, 1, 16, "gemv", 401,
                                   shared=True))
    # second call, smaller: one token on the single-token decode path
    both_entry_points(gen.Workload("noalloc_t1_h256_e8_k2_i512", 1, 256, 8, 2, 512, 1, 8, "gemv", 402))


def test_noalloc_rejections():
    w = gen.WORKLOADS["prefill_t9940_h4096_e256_k8_i1536"]
    need = lib.moe_ffn_workspace_bytes(w.T, w.H, w.I, w.E, w.K, 0, 0)
    assert need > lib.moe_noalloc_scratch_bytes()
    dummy = torch.zeros(16, dtype=torch.int32, device=DEV)
    with pytest.raises(lib.MoeError) as ex:  # past the fixed workspace: nothing is read or launched
        lib.moe_layer_noalloc(dummy, dummy, dummy, w.T, w.H, w.I, w.E, w.K, 32, 0, dummy, dummy, dummy, dummy,
                              lib.moe_slot_stride(w.H, w.I), None, dummy, dummy)
    assert ex.value.status == lib.MOE_EWS
    with pytest.raises(lib.MoeError) as ex:
        lib.moe_layer_noalloc(dummy, dummy, dummy, 4, 256, 512, 8, 2, 32, 0, dummy, dummy, dummy, dummy,
                              lib.moe_slot_stride(256, 512), None, dummy, dummy, lib.MOE_FFN_PARTIAL)
    assert ex.value.status == lib.MOE_EINVAL
    torch.cuda.synchronize()
    assert int(dummy.sum().item()) == 0  # untouched
