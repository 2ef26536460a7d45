"""Parity at the full sizes of the workloads, against the CPU oracle (spread over worker
processes by oracle_pool), through the C ABI.

* single-token decode through all 48 layers (H 4096, 256 experts, top-8, I 1536, a
  64-slot arena per layer with a seeded random map), launched exactly as the benchmark
  times it: one moe_layer per layer, replayed as one HIP graph;
* the grouped (prefill) path with every expert spanning several 128-row M-tiles plus a
  partial tile (of at most 64 rows for some, more for others), every token compared;
* prefill of 9,940 tokens through one layer (256 experts, top-8), every token compared;
* paged decode at the paged shape (256 experts + a shared one, top-6, I 2048, 64-slot
  arenas filled from pinned host memory) over 20 tokens and 2 layers: every output bitwise
  equal to the fully-resident run ("How these numbers are measured", Fidelity).
"""

import concurrent.futures as cf

import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from quantized_routed_expert_moe_amd import harness, lib
from synth import gen

import oracle_pool as OP
from parity_util import DEV, check_close, say, y_f64

pytestmark = pytest.mark.gpu


def bf16_bits_f64(bits):
    return R.bf16_bits_to_f64(bits.astype(np.uint16))


def test_decode_48_layers_graph_replay_vs_oracle():
    w = gen.WORKLOADS["decode_t1_h4096_e256_k8_i1536_x48"]
    say(f"decode stack: building {w.layers} layers")
    with OP.pool() as ex:
        futs = [ex.submit(OP.layer_ref, w, l, gen.activations_bf16(w.seed, l, w.T, w.H)) for l in range(w.layers)]
        stack = harness.StackRunner(w, harness.decode_stack(w, DEV), DEV)
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            stack.step(stream)
        stream.synchronize()
        assert int(stack.status.item()) == 0
        eager = stack.outputs()
        stack.capture(stream)
        stack.poison()
        torch.cuda.synchronize()
        stack.replay(stream)
        stream.synchronize()
        assert int(stack.status.item()) == 0
        y_bits, ids, wts = stack.outputs()
        for e_, r_ in zip(eager, (y_bits, ids, wts)):
            assert np.array_equal(e_.view(np.uint8), r_.view(np.uint8))  # replay == eager, every layer
        say("  graph replay equals the eager step on all layers; comparing with the oracle")
        worst = 0.0
        for l, f in enumerate(futs):
            y_ref, ids_ref, w_ref, _ = f.result()
            assert np.array_equal(ids[l], ids_ref), l
            assert np.abs(wts[l] - w_ref).max() <= 1e-5, l
            y = bf16_bits_f64(y_bits[l])
            rms = np.sqrt(np.mean(y_ref**2))
            worst = max(worst, np.abs(y - y_ref).max() / rms)
            check_close(y, y_ref, f"  layer {l}")
        say(f"  worst layer: max|err| / rms = {worst:.3e}")


def test_grouped_every_expert_spans_several_m_tiles():
    """600 tokens, 8 experts, top-4, a shared expert: each expert holds 286-328 rows (two
    full 128-row tiles and a partial one of 30-72 rows), the shared unit 600 (four full
    tiles and 88 rows); every token against the oracle, and a rerun gives the same bits."""
    w = gen.Workload("grouped_t600_h512_e8_k4_i256_shared", 600, 512, 8, 4, 256, 1, 8, "normal", 56, shared=True)
    xb = gen.activations_bf16(w.seed, 0, w.T, w.H)
    logits = gen.normal_logits(w.seed, 0, w.T, w.E)
    ids_ref, _ = R.route(logits, w.K)
    counts = np.bincount(ids_ref.ravel(), minlength=w.E)
    say(f"grouped multi-tile: rows per expert {counts.tolist()}")
    assert counts.min() > 256 and (counts % 128).min() <= 64 < (counts % 128).max() and w.T % 128 > 64
    experts = {e: R.Expert(gen.expert_tensors(w.seed, 0, e, w.H, w.I), w.H, w.I) for e in range(w.E)}
    shared = R.Expert(gen.expert_tensors(w.seed, 0, gen.SHARED_EXPERT, w.H, w.I), w.H, w.I)
    y_ref, *_ = R.moe_layer(xb, experts, w.K, logits=logits, shared=shared)
    L = harness.make_layer(w, 0, DEV, logits=logits, x_bits=xb, place_seed=3)
    run = harness.LayerRunner(w, DEV)
    run(L)
    torch.cuda.synchronize()
    assert int(run.status.item()) == 0
    assert np.array_equal(run.ids.cpu().numpy(), ids_ref)
    check_close(y_f64(run.y), y_ref, "  grouped t600, every token")
    first = run.y.view(torch.int16).clone()
    run(L)
    torch.cuda.synchronize()
    assert torch.equal(run.y.view(torch.int16), first)


def test_prefill_9940_tokens_every_token_vs_oracle():
    """The prefill layer at full size: every one of the 9,940 tokens against the oracle
    (evaluated expert by expert over a worker pool). Over all 40.7M outputs max|y_ref| / rms
    is about 15, so rounding the exact result to bf16 alone costs about 5.2% of rms: no bf16
    output meets the plain 2e-2 bar here, and the bar applies beyond each output's own
    rounding (check_close asserts that this is so)."""
    w = gen.WORKLOADS["prefill_t9940_h4096_e256_k8_i1536"]
    logits = gen.normal_logits(w.seed, 0, w.T, w.E)
    xb = gen.activations_bf16(w.seed, 0, w.T, w.H)
    with OP.pool() as ex:
        ref = cf.ThreadPoolExecutor(1).submit(OP.expert_major_layer, ex, w, 0, xb, logits)
        say("prefill: packing 256 experts")
        L = harness.make_layer(w, 0, DEV, logits=logits, x_bits=xb, place_seed=4)
        run = harness.LayerRunner(w, DEV)
        run(L)
        torch.cuda.synchronize()
        assert int(run.status.item()) == 0
        y = y_f64(run.y)
        ids = run.ids.cpu().numpy()
        first = run.y.view(torch.int16).clone()
        run.ffn(L)
        torch.cuda.synchronize()
        assert torch.equal(run.y.view(torch.int16), first)
        say("  waiting for the oracle")
        y_ref, ids_ref, _ = ref.result()
    assert np.array_equal(ids, ids_ref)
    counts = np.bincount(ids_ref.ravel(), minlength=w.E)
    say(f"  rows per expert: min {counts.min()} max {counts.max()}")
    check_close(y, y_ref, "  prefill, all 9,940 tokens", beyond_half_ulp=True)
    d = np.abs(y - y_ref).max(axis=1) / np.sqrt(np.mean(y_ref**2))
    say(f"  per-token max|err| / rms: median {np.median(d):.3e}, max {d.max():.3e}")


def test_paged_shape_20_tokens_equals_resident():
    """Paged decode at the paged shape: 2 layers (each its own 256-expert weight set in
    pinned host memory, its own 64-slot arena), 20 tokens routed with 70% temporal
    locality, sequenced by moe_paged_layer with the speculative FFN: every output bitwise
    equal to the fully-resident FFN, the ids equal to the oracle's selection, the arenas
    paging (misses after the first token), and the last token against the oracle."""
    from concurrent.futures import ThreadPoolExecutor

    from quantized_routed_expert_moe_amd import paged

    base = gen.WORKLOADS["paged_t1_h4096_e256s1_k6_i2048_x43"]
    n_layers, steps = 2, 20
    w = gen.Workload("paged_t1_h4096_e256s1_k6_i2048_x2", 1, base.H, base.E, base.K, base.I, n_layers, base.slots,
                     base.router, base.seed, shared=True)
    stride, blob = lib.moe_slot_stride(w.H, w.I), lib.moe_blob_bytes(w.H, w.I)
    lg_np = gen.locality_logits(w.seed, n_layers, steps, w.E, w.K)
    layers, shared, resident, xs = [], [], [], []
    for l in range(n_layers):
        say(f"paged shape: packing layer {l}'s {w.E} experts into pinned host memory")
        host = torch.empty(w.E * stride, dtype=torch.uint8, pin_memory=True)
        hv = host.numpy()

        def put(e, l=l, hv=hv):
            hv[e * stride : (e + 1) * stride] = harness.pack_expert(w.seed, l, e, w.H, w.I)

        with ThreadPoolExecutor(8) as tp:
            list(tp.map(put, range(w.E)))
        slots = torch.empty(w.slots * stride, dtype=torch.uint8, device=DEV)
        table = torch.full((w.E,), -1, dtype=torch.int32, device=DEV)
        layers.append((lib.Arena(w.E, w.slots, blob, stride, slots, table, host), slots, table))
        shared.append(torch.from_numpy(harness.pack_expert(w.seed, l, gen.SHARED_EXPERT, w.H, w.I)).to(DEV))
        resident.append((host.to(DEV), torch.arange(w.E, dtype=torch.int32, device=DEV)))
        xs.append(harness.bf16_tensor(gen.activations_bf16(w.seed, l, 1, w.H), DEV))
    lg = torch.from_numpy(lg_np).to(DEV)
    dec = paged.PagedDecode(layers, [None] * n_layers, stride, w.H, w.I, w.E, w.K, shared=shared, device=DEV,
                            native=True, speculate=True)
    y = torch.empty(1, w.H, dtype=torch.bfloat16, device=DEV)
    y_res = torch.empty_like(y)
    ws2 = torch.empty_like(dec.ws)
    for s in range(steps):
        for l in range(n_layers):
            y.view(torch.int16).fill_(-1)
            dec.layer(l, xs[l], y, lg[s, l])
            ids_d, wts_d = dec.routed
            lib.moe_expert_ffn(xs[l], ids_d, wts_d, 1, w.H, w.I, w.E, w.K, 32, resident[l][1], resident[l][0], stride,
                               shared[l], y_res, ws2, dec.ws_bytes, dec.status)
            torch.cuda.synchronize()
            assert int(dec.status.item()) == 0
            assert torch.equal(y.view(torch.int16), y_res.view(torch.int16)), (s, l)
            assert ids_d.cpu().numpy()[0].tolist() == R.route(lg_np[s, l][None, :], w.K)[0][0].tolist(), (s, l)
    for l in range(n_layers):
        st = layers[l][0].stats()
        say(f"  layer {l}: {st}")
        assert st["misses"] > w.K and st["hits"] + st["misses"] == steps * w.K
        xb = gen.activations_bf16(w.seed, l, 1, w.H)
        y_ref, *_ = OP.layer_ref(w, l, xb, logits=lg_np[steps - 1, l][None, :])
        lib.moe_expert_ffn(xs[l], *dec_route(lg[steps - 1, l], w), 1, w.H, w.I, w.E, w.K, 32, resident[l][1],
                           resident[l][0], stride, shared[l], y_res, ws2, dec.ws_bytes, dec.status)
        torch.cuda.synchronize()
        check_close(y_f64(y_res), y_ref, f"  paged shape layer {l}, last token")


def dec_route(logits, w):
    ids = torch.empty(1, w.K, dtype=torch.int32, device=DEV)
    wts = torch.empty(1, w.K, dtype=torch.float32, device=DEV)
    lib.moe_route(None, None, logits.view(1, -1), 1, w.H, w.E, w.K, 0, ids, wts)
    return ids, wts
