"""One-pass routing (the router GEMV and the softmax top-k in one dispatch) and
moe_layer's one-pass single-token path (routing fused with the gate/up dispatch),
through the C ABI: the same bits as the separate dispatches on every call of a
sequence on one workspace, ids equal to the oracle's, graph replays included, and
the rejections of what the one-pass path does not cover."""

import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from quantized_routed_expert_moe_amd import harness, lib
from synth import gen

from parity_util import DEV, check_close, oracle_layer, say, y_f64

pytestmark = pytest.mark.gpu


def as_bits(t):
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


@pytest.mark.parametrize("H,E,K,renorm", [(4096, 256, 8, False), (256, 8, 2, False), (512, 70, 9, True),
                                         (8192, 1024, 32, False), (2048, 128, 8, True), (96, 3, 3, False)])
def test_route_onepass_equals_moe_route(H, E, K, renorm):
    """Ten calls in a row on one zeroed workspace, each with new x and router: logits,
    ids and w bitwise equal to moe_route's, ids equal to the oracle's selection."""
    say(f"one-pass route H={H} E={E} K={K} renorm={renorm}")
    flags = lib.MOE_ROUTE_RENORM if renorm else 0
    nb = lib.moe_route_onepass_ws_bytes(E, K)
    ws = torch.zeros(nb, dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    for call in range(10):
        xb = gen.activations_bf16(500 + E, call, 1, H)
        wr_np = gen.router_weight(500 + E, call, E, H)
        x, wr = harness.bf16_tensor(xb, DEV), torch.from_numpy(wr_np).to(DEV)
        lg1, lg2 = torch.full((1, E), float("nan"), device=DEV), torch.full((1, E), float("nan"), device=DEV)
        ids1, ids2 = torch.full((1, K), -1, dtype=torch.int32, device=DEV), torch.full((1, K), -1, dtype=torch.int32,
                                                                                        device=DEV)
        w1, w2 = torch.full((1, K), float("nan"), device=DEV), torch.full((1, K), float("nan"), device=DEV)
        lib.moe_route(x, wr, lg1, 1, H, E, K, flags, ids1, w1)
        lib.moe_route_onepass(x, wr, lg2, H, E, K, flags, ids2, w2, ws, nb, st)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        for a, b in ((lg1, lg2), (ids1, ids2), (w1, w2)):
            assert torch.equal(as_bits(a), as_bits(b)), call
        if call in (0, 9):
            ids_ref, _ = R.route(R.router_logits(xb, wr_np), K, renorm)
            assert np.array_equal(ids2.cpu().numpy(), ids_ref)


def test_route_onepass_rejections():
    E, K, H = 64, 4, 256
    nb = lib.moe_route_onepass_ws_bytes(E, K)
    assert lib.moe_route_onepass_ws_bytes(E, 33) == 0 and lib.moe_route_onepass_ws_bytes(2048, 4) == 0
    t = torch.zeros(4096, dtype=torch.int32, device=DEV)
    for args, code in (((H, E, K, 0, nb - 8), lib.MOE_EWS), ((H, E, K, 4, nb), lib.MOE_EINVAL),
                       ((H, E, E + 1, 0, nb), lib.MOE_EINVAL), ((100, E, K, 0, nb), lib.MOE_EUNSUP)):
        Hh, Ee, Kk, fl, n = args
        with pytest.raises(lib.MoeError) as ex:
            lib.moe_route_onepass(t, t, t, Hh, Ee, Kk, fl, t, t, t, n, t)
        assert ex.value.status == code, args
    torch.cuda.synchronize()
    assert int(t.abs().sum().item()) == 0  # nothing ran


WLS = [
    gen.Workload("onepass_t1_h4096_e256_k8_i1536", 1, 4096, 256, 8, 1536, 3, 64, "gemv", 601),
    gen.Workload("onepass_t1_h512_e64_k4_i512_shared", 1, 512, 64, 4, 512, 3, 64, "gemv", 602, shared=True),
    gen.Workload("onepass_t1_h256_e8_k8_i512", 1, 256, 8, 8, 512, 3, 8, "gemv", 603),
    # 9 units of 48 groups: the two-kernel down splits a unit's columns between two waves
    gen.Workload("onepass_t1_h512_e64_k8_i1536_shared", 1, 512, 64, 8, 1536, 3, 64, "gemv", 605, shared=True),
    # the paged decode shape (6 routed + a shared expert, I 2048)
    gen.Workload("onepass_t1_h4096_e256_k6_i2048_shared", 1, 4096, 256, 6, 2048, 2, 64, "gemv", 606, shared=True),
]


@pytest.mark.parametrize("w", WLS, ids=lambda w: w.name)
@pytest.mark.parametrize("renorm", [False, True], ids=["softmax", "renorm"])
def test_layer_onepass_equals_layer(w, renorm):
    """A stack of layers run with and without MOE_ROUTE_ONEPASS: eager, then as a HIP graph
    replayed three times on poisoned outputs; every layer's logits, ids, w and y bitwise
    equal to the two-dispatch routing, and the last layer within the oracle's bar."""
    say(f"one-pass layer {w.name} renorm={renorm}")
    layers = harness.decode_stack(w, DEV)
    rf = lib.MOE_ROUTE_RENORM if renorm else 0
    base = harness.StackRunner(w, layers, DEV, route_flags=rf)
    fused = harness.StackRunner(w, layers, DEV, route_flags=rf | lib.MOE_ROUTE_ONEPASS)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        base.step(stream)
    stream.synchronize()
    want = base.outputs()
    logits_want = [L.logits.clone() for L in layers]
    fused.capture(stream)
    for rep in range(4):  # one eager step, then three replays
        fused.poison()
        torch.cuda.synchronize()
        if rep == 0:
            with torch.cuda.stream(stream):
                fused.step(stream)
        else:
            fused.replay(stream)
        stream.synchronize()
        assert int(fused.status.item()) == 0 and int(base.status.item()) == 0
        got = fused.outputs()
        for name, a, b in zip(("y", "ids", "w"), want, got):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (rep, name)
        for L, lw in zip(layers, logits_want):
            assert torch.equal(L.logits.view(torch.int32), lw.view(torch.int32)), rep
    l = w.layers - 1
    xb = gen.activations_bf16(w.seed, l, 1, w.H)
    y_ref, ids_ref, w_ref, _ = oracle_layer(w, l, xb, renorm=renorm)
    assert np.array_equal(got[1][l], ids_ref)
    assert np.abs(got[2][l] - w_ref).max() <= 1e-5
    check_close(R.bf16_bits_to_f64(got[0][l].astype(np.uint16)), y_ref, f"  one-pass {w.name} layer {l}")


def test_layer_onepass_not_resident_and_rejections():
    """A routed expert without a slot still reports MOE_ENOTRES through the hand-off; the
    one-pass flag with several tokens, without a router or on a short workspace is
    rejected before anything runs."""
    w = gen.Workload("onepass_status_t1_h256_e16_k4_i512", 1, 256, 16, 4, 512, 1, 16, "gemv", 604)
    L = harness.make_layer(w, 0, DEV, place_seed=2)
    run = harness.StackRunner(w, [L], DEV, route_flags=lib.MOE_ROUTE_ONEPASS)
    run.step()
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    e = int(run.ids[0, 0, 1].item())
    L.table[e] = -1
    run.step()
    torch.cuda.synchronize()
    assert int(run.status.item()) == lib.MOE_ENOTRES
    run.status.zero_()
    t = torch.zeros(1 << 16, dtype=torch.int32, device=DEV)
    args = dict(T=1, wr=L.wr, nb=run.ws_bytes)
    cases = [(dict(T=2), lib.MOE_EUNSUP), (dict(wr=None), lib.MOE_EUNSUP), (dict(nb=run.ws_bytes - 1), lib.MOE_EWS)]
    for over, code in cases:
        a = dict(args, **over)
        with pytest.raises(lib.MoeError) as ex:
            lib.moe_layer(L.x, a["wr"], t, a["T"], w.H, w.I, w.E, w.K, 32, lib.MOE_ROUTE_ONEPASS, t, t, L.table, L.slots,
                          L.stride, None, t, run.ws, a["nb"], t, 0)
        assert ex.value.status == code, over
    with pytest.raises(lib.MoeError) as ex:
        lib.moe_layer_noalloc(L.x, L.wr, t, 1, w.H, w.I, w.E, w.K, 32, lib.MOE_ROUTE_ONEPASS, t, t, L.table, L.slots,
                              L.stride, None, t, t)
    assert ex.value.status == lib.MOE_EINVAL
    torch.cuda.synchronize()
    assert int(t.abs().sum().item()) == 0
