"""Benchmark of the int4 routed-expert MoE layer on one MI355X.

Headline workload: single-token decode through 48 MoE layers (hidden 4096, 256
experts, top-8, intermediate 1536, int4 group-32 experts with fp16 scales, fp32
router, one 64-slot arena per layer with a seeded random expert-to-slot map and
every routed expert resident). One step = one token through all 48 layers:
per layer moe_route (router GEMV + softmax top-k) and moe_expert_ffn (int4
SwiGLU experts + combine), replayed as one HIP graph. Inputs are seeded
synthetic tensors already resident in HBM when the timed region starts.

Further workloads, reported in the same JSON line under "workloads":
prefill of 9,940 tokens through one layer (expert-grouped MFMA path) and
batched decode of 16 tokens with Zipf-skewed routing (rotating over distinct
layer weight sets so the 256 MB last-level cache cannot hold them).
Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=48)
    p.add_argument("--legs", default="decode,prefill,batched,paged,readahead,route_variants,chunked,formats",
                   help="comma list of decode,prefill,batched,paged,readahead,route_variants,chunked,formats")
    p.add_argument("--chunks", default="1024,2048,4096", help="prompt chunk sizes of the chunked paged prefill leg")
    p.add_argument("--paged-steps", type=int, default=64, help="measured tokens of the paged decode workload")
    p.add_argument("--readahead", default="2,3,4,6", help="experts read ahead per layer in the read-ahead leg")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-layers", type=int, default=3, help="decode layers in the oracle's timed sample")
    p.add_argument("--cpu-matrix", action="store_true",
                   help="also time the oracle on every workload at 1 thread and at all cores (about a minute)")
    p.add_argument("--graph", type=int, default=1, help="replay the decode layer stack as a HIP graph")
    p.add_argument("--onepass", type=int, default=1,
                   help="decode headline with one-pass routing fused into the gate/up dispatch (MOE_ROUTE_ONEPASS); "
                        "the other routing is timed beside it")
    p.add_argument("--copy-probe-mib", type=int, default=0,
                   help="first run one plain device-to-device copy of this many MiB (counter calibration for profiles)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ev():
    import torch

    return torch.cuda.Event(enable_timing=True)


def stage_times(calls, stream, reps=1):
    """Mean duration (us) of each named call over reps, from HIP events recorded on `stream`."""
    import torch

    acc = {}
    for _ in range(reps):
        marks = []
        with torch.cuda.stream(stream):
            for name, f in calls:
                e0, e1 = ev(), ev()
                e0.record(stream)
                f()
                e1.record(stream)
                marks.append((name, e0, e1))
        torch.cuda.synchronize()
        for name, e0, e1 in marks:
            acc.setdefault(name, []).append(e0.elapsed_time(e1) * 1e3)
    return {k: sum(v) / len(v) for k, v in acc.items()}


# HBM traffic per launch of the decode kernels, from the committed rocprofv3
# counter summary; reported only while the kernel sources still hash to the value
# recorded there (a changed kernel has not been measured).
TRAFFIC_SUMMARY = "profiles/decode_t1_h4096_e256_k8_i1536_x48_hbm_traffic.md"
DECODE_KERNEL_SOURCES = ("quantized_routed_expert_moe_amd/csrc/ffn_decode.hip",
                         "quantized_routed_expert_moe_amd/csrc/wave_ops.h",
                         "quantized_routed_expert_moe_amd/csrc/moe_internal.h")


def decode_traffic():
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    try:
        text = open(os.path.join(root, TRAFFIC_SUMMARY)).read()
    except OSError:
        return {}
    h = hashlib.sha256()
    for p in DECODE_KERNEL_SOURCES:
        h.update(open(os.path.join(root, p), "rb").read())
    rec = {}
    for line in text.splitlines():
        if line.startswith("traffic_bytes_per_launch "):
            k, v = line[len("traffic_bytes_per_launch "):].split(":")
            rec[k.strip()] = int(v)
        elif line.startswith("kernel_sources_sha256:"):
            rec["sha"] = line.split(":")[1].strip()
    if rec.get("sha") != h.hexdigest()[:16]:
        return {}
    return rec


# ------------------------------------------------------------------ decode (headline)


def decode_leg(a, dev):
    import numpy as np
    import torch

    from quantized_routed_expert_moe_amd import harness, lib
    from synth import gen

    base = gen.WORKLOADS["decode_t1_h4096_e256_k8_i1536_x48"]
    w = gen.Workload(base.name, base.T, base.H, base.E, base.K, base.I, a.layers, base.slots, base.router, base.seed)
    log(f"decode: building {w.layers} layers of {w.name}")
    stacks = harness.decode_stack(w, dev, log)
    # one moe_layer per layer, each layer with its own outputs; route_flags picks the routing
    stack = harness.StackRunner(w, stacks, dev, route_flags=lib.MOE_ROUTE_ONEPASS if a.onepass else 0)
    other = harness.StackRunner(w, stacks, dev, route_flags=0 if a.onepass else lib.MOE_ROUTE_ONEPASS)
    run = harness.LayerRunner(w, dev)  # per-stage timings below
    stream = torch.cuda.Stream()
    blob = lib.moe_blob_bytes(w.H, w.I)
    mat_bytes = w.H * w.I // 2 + w.H * w.I // 32 * 2  # codes + fp16 scales of one matrix
    bytes_router = w.E * w.H * 4 + w.T * w.H * 2 + w.T * w.E * 4 + w.T * w.K * 8
    bytes_gate_up = w.K * 2 * mat_bytes + w.T * w.H * 2 + w.T * w.K * w.I * 2  # experts + x + h (fp16)
    bytes_down = w.K * mat_bytes + w.T * w.K * w.I * 2 + w.T * w.H * 2  # experts + h (fp16) + y
    bytes_layer = bytes_router + w.K * blob + w.T * w.H * 2 * 2

    with torch.cuda.stream(stream):
        for _ in range(a.warmup):
            stack.step(stream)
    stream.synchronize()
    if int(stack.status.item()) != 0:
        raise RuntimeError(f"device status {int(stack.status.item())}")
    eager = stack.outputs()
    if a.graph:
        stack.capture(stream)
        # the captured step must recompute every layer: poison all outputs, replay once,
        # and compare every layer's y, ids and w with the eager step, bit for bit
        stack.poison()
        torch.cuda.synchronize()
        stack.replay(stream)
        stream.synchronize()
        replayed = stack.outputs()
        for name, e_, r_ in zip(("y", "ids", "w"), eager, replayed):
            if not np.array_equal(e_.view(np.uint8), r_.view(np.uint8)):
                raise RuntimeError(f"graph replay {name} differs from the eager step")
        log(f"  decode: graph replay equals the eager step bitwise on all {w.layers} layers")
        with torch.cuda.stream(stream):  # untimed warm replays of the graph itself
            for _ in range(a.warmup):
                stack.graph.replay()

    def step():
        stack.step(stream)

    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    t0 = time.perf_counter()
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(a.steps):
            if stack.graph is not None:
                stack.graph.replay()
            else:
                step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / a.steps
    after = stack.outputs()  # the timed steps left the same bits in every layer
    if not all(np.array_equal(e_.view(np.uint8), r_.view(np.uint8)) for e_, r_ in zip(eager, after)):
        raise RuntimeError("the timed decode steps left outputs that differ from the eager step")
    # the other routing on the same layers: the same bits, timed the same way
    with torch.cuda.stream(stream):
        for _ in range(a.warmup):
            other.step(stream)
    stream.synchronize()
    if not all(np.array_equal(e_.view(np.uint8), r_.view(np.uint8)) for e_, r_ in zip(eager, other.outputs())):
        raise RuntimeError("one-pass and two-dispatch routing give different outputs")
    if a.graph:
        other.capture(stream)
        with torch.cuda.stream(stream):
            for _ in range(a.warmup):
                other.graph.replay()
    o0, o1 = ev(), ev()
    o0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(a.steps):
            if other.graph is not None:
                other.graph.replay()
            else:
                other.step(stream)
    o1.record(stream)
    torch.cuda.synchronize()
    other_ms = o0.elapsed_time(o1) / a.steps
    if int(other.status.item()) != 0:
        raise RuntimeError(f"device status {int(other.status.item())}")

    # per-stage durations: each stage launched for every layer back to back on the
    # launch stream (each layer with its own routed experts), 3 passes, HIP events
    # around the batch -> mean per launch
    routed = []
    with torch.cuda.stream(stream):
        for L in stacks:
            run.route(L, stream)
            routed.append((run.ids.clone(), run.wts.clone()))
    stream.synchronize()
    calls = {
        "route": lambda i, L: run.route(L, stream),
        "gate_up": lambda i, L: run.ffn(L, stream, stage="gate_up", ids=routed[i][0], wts=routed[i][1]),
        "down": lambda i, L: run.ffn(L, stream, stage="down", ids=routed[i][0], wts=routed[i][1]),
    }
    us = {}
    for name, f in calls.items():
        b0, b1 = ev(), ev()
        with torch.cuda.stream(stream):
            for i, L in enumerate(stacks):  # warm
                f(i, L)
            b0.record(stream)
            for _ in range(3):
                for i, L in enumerate(stacks):
                    f(i, L)
            b1.record(stream)
        stream.synchronize()
        us[name] = b0.elapsed_time(b1) * 1e3 / (3 * len(stacks))
    if int(run.status.item()) != 0 or int(stack.status.item()) != 0:
        raise RuntimeError(f"device status {int(run.status.item())} / {int(stack.status.item())}")
    gu_gbs = bytes_gate_up / (us["gate_up"] * 1e-6) / 1e9
    dn_gbs = bytes_down / (us["down"] * 1e-6) / 1e9
    layer_gbs = bytes_layer * w.layers / (ms_step * 1e-3) / 1e9
    return w, {
        "tok_s": 1000.0 / ms_step,
        "ms_step": ms_step,
        "wall": wall,
        "graph": stack.graph is not None,
        "onepass": bool(a.onepass),
        "other_ms_step": other_ms,
        "layer_gbs": layer_gbs,
        "us": us,
        "bytes": {"router": bytes_router, "gate_up": bytes_gate_up, "down": bytes_down, "layer": bytes_layer},
        "gu_gbs": gu_gbs,
        "dn_gbs": dn_gbs,
    }


# ------------------------------------------------------------------ prefill


def prefill_leg(a, dev):
    import torch

    from quantized_routed_expert_moe_amd import harness
    from synth import gen

    w = gen.WORKLOADS["prefill_t9940_h4096_e256_k8_i1536"]
    log(f"prefill: packing {w.E} experts for {w.name}")
    t0 = time.time()
    L = harness.make_layer(w, 0, dev, place_seed=4)
    log(f"  prefill: packed ({time.time() - t0:.1f} s)")
    run = harness.LayerRunner(w, dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(2):
            run(L, stream)
    stream.synchronize()
    if int(run.status.item()) != 0:
        raise RuntimeError(f"device status {int(run.status.item())}")
    reps = 5
    e0, e1 = ev(), ev()
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            run(L, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    st = stage_times([("route", lambda: run.route(L, stream)),
                      ("gate_up", lambda: run.ffn(L, stream, stage="gate_up")),
                      ("down", lambda: run.ffn(L, stream, stage="down"))], stream, reps=3)
    P = w.T * w.K
    fl_gu = 2.0 * P * w.H * 2 * w.I
    fl_dn = 2.0 * P * w.I * w.H
    return w, {
        "tok_s": w.T / (ms * 1e-3),
        "ms_layer": ms,
        "us": st,
        "tflops_layer": (fl_gu + fl_dn) / (ms * 1e-3) / 1e12,
        "tflops_gate_up": fl_gu / (st["gate_up"] * 1e-6) / 1e12,
        "tflops_down": fl_dn / (st["down"] * 1e-6) / 1e12,
        "flops": fl_gu + fl_dn,
    }


# ------------------------------------------------------------------ batched decode


def batched_leg(a, dev, n_sets=16):
    import numpy as np
    import torch

    from quantized_routed_expert_moe_amd import harness
    from synth import gen

    w = gen.WORKLOADS["batched_t16_h2048_e128_k8_i768_zipf"]
    log(f"batched: packing {n_sets} distinct layer weight sets of {w.name}")
    t0 = time.time()
    sets = []
    for layer in range(n_sets):
        lg = gen.zipf_logits(w.seed, layer, w.T, w.E)
        top = np.argsort(-lg, axis=1, kind="stable")[:, : w.K]  # set-up only: which experts to pack
        experts = sorted(set(top.ravel().tolist()))
        sets.append(harness.make_layer(w, layer, dev, experts=experts, place_seed=layer, logits=lg))
    log(f"  batched: packed ({time.time() - t0:.1f} s)")
    run = harness.LayerRunner(w, dev)
    stream = torch.cuda.Stream()
    # each layer is one moe_layer call (route and expert FFN; on this path the plan
    # kernel does the top-k selection itself)
    with torch.cuda.stream(stream):
        for L in sets:
            run.layer(L, stream)
    stream.synchronize()
    if int(run.status.item()) != 0:
        raise RuntimeError(f"device status {int(run.status.item())}")
    distinct = []
    for L in sets:
        run.route(L, stream)
        stream.synchronize()
        distinct.append(len(set(run.ids.cpu().numpy().ravel().tolist())))
    reps = 10
    e0, e1 = ev(), ev()
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(reps):
            for L in sets:
                run.layer(L, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us_layer = e0.elapsed_time(e1) * 1e3 / (reps * len(sets))
    blob = harness.lib.moe_blob_bytes(w.H, w.I)
    bytes_layer = float(np.mean(distinct)) * blob + w.T * w.E * 4 + 2 * w.T * w.H * 2
    return w, {
        "tok_s": w.T / (us_layer * 1e-6),
        "us_layer": us_layer,
        "distinct_experts": float(np.mean(distinct)),
        "hbm_gbs": bytes_layer / (us_layer * 1e-6) / 1e9,
        "bytes_layer": bytes_layer,
    }


# ------------------------------------------------------------------ router variants


def route_variants_leg(dev, reps=48):
    """moe_route / moe_route_scored from logits (E = 256, K = 8): the time per call of each
    scoring function (and of the bitonic selection), for one decode token and for the
    9,940-token prompt."""
    import numpy as np
    import torch

    from quantized_routed_expert_moe_amd import lib
    from synth import gen

    E, K = 256, 8
    stream = torch.cuda.Stream()
    bias = torch.from_numpy((0.05 * np.random.default_rng(7).standard_normal(E)).astype(np.float32)).to(dev)
    out = {}
    for T in (1, 9940):
        logits = [torch.from_numpy(gen.normal_logits(31, i, T, E)).to(dev) for i in range(4)]
        ids = torch.empty(T, K, dtype=torch.int32, device=dev)
        wts = torch.empty(T, K, dtype=torch.float32, device=dev)
        variants = {
            "softmax": lambda l: lib.moe_route(None, None, l, T, 0, E, K, 0, ids, wts, stream),
            "softmax_bitonic_select": lambda l: lib.moe_route(None, None, l, T, 0, E, K, lib.MOE_ROUTE_BITONIC, ids,
                                                              wts, stream),
            "sigmoid_bias_renorm_scale2.5": lambda l: lib.moe_route_scored(
                None, None, l, T, 0, E, K, lib.MOE_SCORE_SIGMOID, bias, 2.5, lib.MOE_ROUTE_RENORM, ids, wts, stream),
            "sqrtsoftplus_bias_renorm": lambda l: lib.moe_route_scored(
                None, None, l, T, 0, E, K, lib.MOE_SCORE_SQRTSOFTPLUS, bias, 1.0, lib.MOE_ROUTE_RENORM, ids, wts,
                stream),
        }
        for name, call in variants.items():
            for i in range(4):
                call(logits[i])
            stream.synchronize()
            e0, e1 = ev(), ev()
            e0.record(stream)
            for r in range(reps):
                call(logits[r % 4])
            e1.record(stream)
            torch.cuda.synchronize()
            out[f"t{T}_{name}_us"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    log(f"  route variants: {out}")
    return out


# ------------------------------------------------------------------ paged decode


def paged_leg(a, dev):
    """Paged single-token decode through 43 layers with 64-slot arenas filled from pinned host memory.

    Every layer's arena draws its misses from one pinned, expert-major host copy
    of 256 experts (one weight set shared by the layers, so the host copy fits in
    3.6 GB; arena keys stay per layer, so every miss is a real 14 MB copy). Per
    layer and token: moe_route on logits with temporal locality, the ids come
    back to the host (the hand-shake), arena_map_slots, arena_fill_async on a
    side stream, the compute stream waits on its event, then moe_expert_ffn
    (six routed experts plus the shared expert). Timed twice from empty arenas on
    the same tokens: sequenced from Python (paged.PagedDecode(native=False)) and
    by moe_paged_layer with the speculative FFN (the reported rate).
    """
    from concurrent.futures import ThreadPoolExecutor

    import torch

    from quantized_routed_expert_moe_amd import harness, lib, paged
    from synth import gen

    w = gen.WORKLOADS["paged_t1_h4096_e256s1_k6_i2048_x43"]
    warm = 16
    steps = warm + a.paged_steps
    stride = lib.moe_slot_stride(w.H, w.I)
    blob = lib.moe_blob_bytes(w.H, w.I)
    log(f"paged: packing {w.E} experts into pinned host memory ({w.E * stride / 2**30:.1f} GiB)")
    t0 = time.time()
    host = torch.empty(w.E * stride, dtype=torch.uint8, pin_memory=True)
    hv = host.numpy()

    def put(e):
        hv[e * stride : (e + 1) * stride] = harness.pack_expert(w.seed, 0, e, w.H, w.I)

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(put, range(w.E)))
    shared = torch.from_numpy(harness.pack_expert(w.seed, 0, gen.SHARED_EXPERT, w.H, w.I)).to(dev)
    resident = host.to(dev)  # all 256 experts, identity slot map: the fully-resident comparison
    resident_table = torch.arange(w.E, dtype=torch.int32, device=dev)
    log(f"  paged: packed ({time.time() - t0:.1f} s)")
    lg = torch.from_numpy(gen.locality_logits(w.seed, w.layers, steps, w.E, w.K)).to(dev)  # [steps, layers, E]
    xs = [harness.bf16_tensor(gen.activations_bf16(w.seed, l, 1, w.H), dev) for l in range(w.layers)]
    layers = []
    for l in range(w.layers):
        sl = torch.empty(w.slots * stride, dtype=torch.uint8, device=dev)
        tb = torch.full((w.E,), -1, dtype=torch.int32, device=dev)
        layers.append((lib.Arena(w.E, w.slots, blob, stride, sl, tb, host), sl, tb))
    ys = [torch.empty(1, w.H, dtype=torch.bfloat16, device=dev) for _ in range(w.layers)]
    y_res = torch.empty(1, w.H, dtype=torch.bfloat16, device=dev)
    res = {}
    # native: ids to the host through the polled word; native_event: through a copy and an event
    for mode, native, poll in (("python", False, False), ("native_event", True, False), ("native", True, True)):
        for ar, _, tb in layers:
            ar.reset()
            tb.fill_(-1)
        dec = paged.PagedDecode(layers, [None] * w.layers, stride, w.H, w.I, w.E, w.K, shared=[shared] * w.layers,
                                device=dev, native=native, speculate=native, host_poll=poll)
        lgs = [[lg[s, l] for l in range(w.layers)] for s in range(steps)]
        for s in range(warm):
            dec.token(xs, ys, lgs[s])
        torch.cuda.synchronize()
        st0 = [ar.stats() for ar, _, _ in layers]
        t0 = time.perf_counter()
        for s in range(warm, steps):
            dec.token(xs, ys, lgs[s])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        st1 = [ar.stats() for ar, _, _ in layers]
        if int(dec.status.item()) != 0:
            raise RuntimeError(f"device status {int(dec.status.item())}")
        d = {k: sum(b[k] - a_[k] for a_, b in zip(st0, st1)) for k in st0[0]}
        identical = True  # one more token, every layer's paged output against the fully-resident one
        for l in range(w.layers):
            dec.layer(l, xs[l], ys[l], lg[steps - 1, l])
            ids_d, wts_d = dec.routed
            lib.moe_expert_ffn(xs[l], ids_d, wts_d, 1, w.H, w.I, w.E, w.K, 32, resident_table, resident, stride,
                               shared, y_res, dec.ws, dec.ws_bytes, dec.status)
            torch.cuda.synchronize()
            identical = identical and torch.equal(ys[l].view(torch.int16), y_res.view(torch.int16))
        res[mode] = (dt, d, identical)
        log(f"  paged {mode}: {(steps - warm) / dt:.2f} tok/s")
    # the same tokens with every expert resident (identity slot map, no hand-shake): the
    # rate of the layer stack when the arena holds everything. One token's 43 moe_layer
    # calls are replayed as a HIP graph (checked bitwise against eager), its logits
    # copied into the graph's input before each replay.
    ids_r = torch.empty(1, w.K, dtype=torch.int32, device=dev)
    wts_r = torch.empty(1, w.K, dtype=torch.float32, device=dev)
    ws_r = torch.empty(max(lib.moe_ffn_workspace_bytes(1, w.H, w.I, w.E, w.K, True), 256), dtype=torch.uint8,
                       device=dev)
    st_r = torch.zeros(1, dtype=torch.int32, device=dev)
    lg_cur = torch.empty(w.layers, w.E, dtype=torch.float32, device=dev)
    rs = torch.cuda.Stream()

    def resident_token():
        for l in range(w.layers):
            lib.moe_layer(xs[l], None, lg_cur[l], 1, w.H, w.I, w.E, w.K, 32, 0, ids_r, wts_r, resident_table, resident,
                          stride, shared, ys[l], ws_r, ws_r.numel(), st_r, 0, rs)

    with torch.cuda.stream(rs):
        lg_cur.copy_(lg[steps - 1])
        resident_token()
        y_eager = torch.stack([y.clone() for y in ys])
    rs.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=rs):
        resident_token()
    for y in ys:  # poisoned: a replay that computed nothing cannot pass
        y.view(torch.int16).fill_(-1)
    torch.cuda.synchronize()
    with torch.cuda.stream(rs):
        graph.replay()
    rs.synchronize()
    if not torch.equal(torch.stack(ys).view(torch.int16), y_eager.view(torch.int16)):
        raise RuntimeError("resident graph replay differs from the eager run")
    e0, e1 = ev(), ev()
    with torch.cuda.stream(rs):
        for s in range(warm):
            lg_cur.copy_(lg[s])
            graph.replay()
        e0.record(rs)
        for s in range(warm, steps):
            lg_cur.copy_(lg[s])
            graph.replay()
        e1.record(rs)
    torch.cuda.synchronize()
    if int(st_r.item()) != 0:
        raise RuntimeError(f"device status {int(st_r.item())}")
    res_ms = e0.elapsed_time(e1) / (steps - warm)
    res_bytes = w.layers * ((w.K + 1) * blob + w.E * 4 + 2 * w.H * 2)  # 6 routed + shared blobs, logits, x, y
    # pinned host -> device copy rate for context
    probe_dev = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    probe_host = torch.empty(1 << 30, dtype=torch.uint8, pin_memory=True)
    e0, e1 = ev(), ev()
    e0.record()
    for _ in range(3):
        probe_dev.copy_(probe_host, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d_peak = 3 * (1 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    n_tok = steps - warm
    dt, d, identical = res["native"]
    return w, {
        "tok_s": n_tok / dt,
        "ms_per_token": dt * 1e3 / n_tok,
        "hit_rate": d["hits"] / max(1, d["hits"] + d["misses"]),
        "misses_per_layer_step": d["misses"] / (n_tok * w.layers),
        "h2d_gbs": d["h2d_bytes"] / dt / 1e9,
        "h2d_peak_gbs": h2d_peak,
        "identical": identical and res["python"][2] and res["native_event"][2],
        "python_tok_s": n_tok / res["python"][0],
        "event_handshake_tok_s": n_tok / res["native_event"][0],
        "event_handshake_h2d_gbs": res["native_event"][1]["h2d_bytes"] / res["native_event"][0] / 1e9,
        "resident_tok_s": 1e3 / res_ms,
        "resident_hbm_gbs": res_bytes / (res_ms * 1e-3) / 1e9,
    }


def readahead_leg(a, dev):
    """Paged single-token decode through 43 layers routed by per-layer router GEMVs on a
    residual stream, without and with next-layer read-ahead (paged.PagedDecode).

    The paged shape (256 experts + a shared one, top-6, I 2048, 64 slots per layer);
    the layers draw misses from one pinned host copy of one 256-expert weight set (arena
    keys stay per layer, so every miss is a real 14 MB copy); each layer has its own
    router. The layer inputs follow gen.residual_stream (a 0.99 between tokens, rho 0.15
    between layers). Read-ahead predicts layer l + 1's top-6 with its router on layer
    l's input. Modes: "python_off" sequences each layer from Python (route, hand-shake,
    map, fill, FFN); "off" and "next_layer_topP" are one moe_paged_layer call per layer
    (native sequencing, speculative FFN), without and with read-ahead of P experts. Every
    mode runs the same tokens from empty arenas; 16 warm-up tokens.
    """
    from concurrent.futures import ThreadPoolExecutor

    import torch

    from quantized_routed_expert_moe_amd import harness, lib, paged
    from synth import gen

    w = gen.WORKLOADS["readahead_t1_h4096_e256s1_k6_i2048_x43"]
    warm = 16
    steps = warm + a.paged_steps
    stride = lib.moe_slot_stride(w.H, w.I)
    blob = lib.moe_blob_bytes(w.H, w.I)
    log(f"read-ahead: packing {w.E} experts into pinned host memory ({w.E * stride / 2**30:.1f} GiB)")
    host = torch.empty(w.E * stride, dtype=torch.uint8, pin_memory=True)
    hv = host.numpy()

    def put(e):
        hv[e * stride : (e + 1) * stride] = harness.pack_expert(w.seed, 0, e, w.H, w.I)

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(put, range(w.E)))
    shared = torch.from_numpy(harness.pack_expert(w.seed, 0, gen.SHARED_EXPERT, w.H, w.I)).to(dev)
    resident = host.to(dev)
    resident_table = torch.arange(w.E, dtype=torch.int32, device=dev)
    routers = [torch.from_numpy(gen.router_weight(w.seed, l, w.E, w.H)).to(dev) for l in range(w.layers)]
    xs_all = torch.from_numpy(gen.residual_stream(w.seed, steps + 1, w.layers, w.H).view("int16")).to(dev)
    xs_all = xs_all.view(torch.bfloat16)  # [steps + 1, layers, H]
    layers = []
    for l in range(w.layers):
        sl = torch.empty(w.slots * stride, dtype=torch.uint8, device=dev)
        tb = torch.full((w.E,), -1, dtype=torch.int32, device=dev)
        layers.append((lib.Arena(w.E, w.slots, blob, stride, sl, tb, host), sl, tb))
    ys = [torch.empty(1, w.H, dtype=torch.bfloat16, device=dev) for _ in range(w.layers)]
    y_res = torch.empty(1, w.H, dtype=torch.bfloat16, device=dev)
    out = {}
    modes = [("python_off", 0, False), ("off", 0, True)]
    modes += [(f"next_layer_top{P}", P, True) for P in (int(v) for v in a.readahead.split(",") if v)]
    for mode, P, native in modes:
        for ar, _, tb in layers:
            ar.reset()
            tb.fill_(-1)
        dec = paged.PagedDecode(layers, routers, stride, w.H, w.I, w.E, w.K, shared=[shared] * w.layers,
                                predict=P, device=dev, native=native, speculate=native)
        for t in range(warm):
            dec.token([xs_all[t, l][None, :] for l in range(w.layers)], ys)
        torch.cuda.synchronize()
        st0 = [ar.stats() for ar, _, _ in layers]
        t0 = time.perf_counter()
        for t in range(warm, steps):
            dec.token([xs_all[t, l][None, :] for l in range(w.layers)], ys)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        st1 = [ar.stats() for ar, _, _ in layers]
        if int(dec.status.item()) != 0:
            raise RuntimeError(f"device status {int(dec.status.item())}")
        d = {k: sum(b[k] - a_[k] for a_, b in zip(st0, st1)) for k in st0[0]}
        identical = True  # one more token, each layer against the fully-resident run
        for l in range(w.layers):
            x = xs_all[steps, l][None, :]
            dec.layer(l, x, ys[l])
            ids_d, wts_d = dec.routed
            lib.moe_expert_ffn(x, ids_d, wts_d, 1, w.H, w.I, w.E, w.K, 32, resident_table, resident, stride,
                               shared, y_res, dec.ws, dec.ws_bytes, dec.status)
            torch.cuda.synchronize()
            identical = identical and torch.equal(ys[l].view(torch.int16), y_res.view(torch.int16))
        n_tok, n_lay = steps - warm, (steps - warm) * w.layers
        out[mode] = {
            "tokens_per_s": round(n_tok / dt, 2),
            "ms_per_token": round(dt * 1e3 / n_tok, 3),
            "hit_rate": round(d["hits"] / max(1, d["hits"] + d["misses"]), 4),
            "demand_misses_per_layer_step": round(d["misses"] / n_lay, 3),
            "prefetch_fills_per_layer_step": round(d["prefetch_fills"] / n_lay, 3),
            "prefetch_precision": round(d["prefetch_hits"] / d["prefetch_fills"], 4) if d["prefetch_fills"] else None,
            "copies_per_layer_step": round(d["fills"] / n_lay, 3),
            "h2d_gbs": round(d["h2d_bytes"] / dt / 1e9, 2),
            "bit_identical_to_resident": identical,
        }
        log(f"  read-ahead {mode}: {out[mode]}")
    out["speedup_vs_off"] = {m: round(v["tokens_per_s"] / out["off"]["tokens_per_s"], 4) for m, v in out.items()
                             if m != "off"}
    return w, out


def pinned_expert_copy(w, layer):
    """All E experts of a layer packed into one pinned, expert-major host buffer."""
    from concurrent.futures import ThreadPoolExecutor

    import torch

    from quantized_routed_expert_moe_amd import harness, lib

    stride = lib.moe_slot_stride(w.H, w.I)
    host = torch.empty(w.E * stride, dtype=torch.uint8, pin_memory=True)
    hv = host.numpy()

    def put(e):
        hv[e * stride : (e + 1) * stride] = harness.pack_expert(w.seed, layer, e, w.H, w.I)

    with ThreadPoolExecutor(8) as ex:
        list(ex.map(put, range(w.E)))
    return host, stride


def chunked_leg(a, dev):
    """Chunked paged prefill: a 4,096-token prompt through one layer (256 experts, top-6, shared
    expert, I = 2048) with a 64-slot arena fed from pinned host memory, per chunk size.

    Each chunk routes, hands its ids to the host, runs passes of at most 32 experts (half
    the arena, so the next pass's fills overlap the current pass's compute) and combines.
    Per chunk size the prompt runs once untimed (the arena reaches its steady state) and
    once timed; the fully-resident grouped run of the same chunks is timed beside it, and
    the last chunk's output is compared bitwise with it.
    """
    import numpy as np
    import torch

    from quantized_routed_expert_moe_amd import harness, lib
    from quantized_routed_expert_moe_amd.paged import ChunkedPrefill
    from synth import gen

    w = gen.WORKLOADS["chunked_t4096_h4096_e256s1_k6_i2048"]
    log(f"chunked: packing {w.E} experts into pinned host memory")
    t0 = time.time()
    host, stride = pinned_expert_copy(w, 0)
    blob = lib.moe_blob_bytes(w.H, w.I)
    resident = host.to(dev)
    table_res = torch.arange(w.E, dtype=torch.int32, device=dev)
    shared = torch.from_numpy(harness.pack_expert(w.seed, 0, gen.SHARED_EXPERT, w.H, w.I)).to(dev)
    x = harness.bf16_tensor(gen.activations_bf16(w.seed, 0, w.T, w.H), dev)
    logits = torch.from_numpy(gen.normal_logits(w.seed, 0, w.T, w.E)).to(dev)
    y = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
    y_res = torch.empty_like(y)
    log(f"  chunked: packed ({time.time() - t0:.1f} s)")
    cap = w.slots // 2
    out = {}
    for chunk in [int(c) for c in a.chunks.split(",")]:
        slots = torch.empty(w.slots * stride, dtype=torch.uint8, device=dev)
        table = torch.full((w.E,), -1, dtype=torch.int32, device=dev)
        arena = lib.Arena(w.E, w.slots, blob, stride, slots, table, host)
        cp = ChunkedPrefill(arena, slots, stride, w.H, w.I, w.E, w.K, chunk, cap, shared=shared, device=dev)
        ids = torch.empty(chunk, w.K, dtype=torch.int32, device=dev)
        wts = torch.empty(chunk, w.K, dtype=torch.float32, device=dev)
        nb = lib.moe_ffn_workspace_bytes(chunk, w.H, w.I, w.E, w.K, 1, lib.MOE_FORCE_GROUPED)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)

        def resident_prompt():
            for c0 in range(0, w.T, chunk):
                T = min(chunk, w.T - c0)
                lib.moe_route(None, None, logits[c0 : c0 + T], T, w.H, w.E, w.K, 0, ids[:T], wts[:T])
                lib.moe_expert_ffn(x[c0 : c0 + T], ids[:T], wts[:T], T, w.H, w.I, w.E, w.K, 32, table_res, resident,
                                   stride, shared, y_res[c0 : c0 + T], ws, nb, status, lib.MOE_FORCE_GROUPED)

        cp.run_prompt(x, logits, y, chunk)  # untimed: the arena's steady state
        torch.cuda.synchronize()
        st0 = arena.stats()
        passes = 0
        t0 = time.perf_counter()
        for c0 in range(0, w.T, chunk):
            cp.run_chunk(x[c0 : c0 + chunk], logits[c0 : c0 + chunk], y[c0 : c0 + chunk])
            passes += len(cp.last_passes)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        st1 = arena.stats()
        resident_prompt()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        resident_prompt()
        torch.cuda.synchronize()
        dt_res = time.perf_counter() - t1
        if int(cp.status.item()) != 0 or int(status.item()) != 0:
            raise RuntimeError(f"device status {int(cp.status.item())} / {int(status.item())}")
        identical = torch.equal(y.view(torch.int16), y_res.view(torch.int16))
        n_chunks = (w.T + chunk - 1) // chunk
        fills = st1["fills"] - st0["fills"]
        out[str(chunk)] = {
            "tokens_per_s": round(w.T / dt, 1),
            "ms_per_prompt": round(dt * 1e3, 2),
            "passes_per_chunk": round(passes / n_chunks, 2),
            "expert_reads_per_chunk": round(fills / n_chunks, 1),
            "h2d_gb_per_prompt": round((st1["h2d_bytes"] - st0["h2d_bytes"]) / 1e9, 3),
            "h2d_gbs": round((st1["h2d_bytes"] - st0["h2d_bytes"]) / dt / 1e9, 2),
            "resident_tokens_per_s": round(w.T / dt_res, 1),
            "bit_identical_to_resident": identical,
        }
        log(f"  chunk {chunk}: {out[str(chunk)]}")
        del cp, arena, slots, table, ws
        torch.cuda.empty_cache()
    return w, out


def formats_leg(dev, steps=192, n_blobs=64):
    """Expert FFN of one token (H 4096, I 1536, 256 experts, top-8) per weight format:
    int4 group 32 and int4 group 128 (the single-token path of moe_expert_ffn), int8
    group 32 and NVFP4 (moe_expert_ffn_fmt). 64 distinct experts are packed per format (the
    table maps expert e to blob e % 64, more bytes than the 256 MB last-level cache);
    every timed call routes to 8 other experts (seeded draws without replacement). Also a
    prompt of 2,048 tokens over the 64 packed experts (top-8 of seeded N(0,1) logits): the
    int4 grouped GEMM and the int8 / NVFP4 prompt GEMMs, ms per layer and useful TFLOP/s."""
    import numpy as np
    import torch

    from quantized_routed_expert_moe_amd import harness, lib
    from synth import gen

    H, I, E, K, seed = 4096, 1536, 256, 8, 7
    rng = np.random.default_rng(seed)
    ids_all = np.stack([rng.choice(E, size=K, replace=False) for _ in range(steps + 8)]).astype(np.int32)
    ids_d = torch.from_numpy(ids_all).to(dev)
    wts = torch.full((K,), 1.0 / K, dtype=torch.float32, device=dev)
    x = harness.bf16_tensor(gen.activations_bf16(seed, 0, 1, H), dev)
    y = torch.empty(1, H, dtype=torch.bfloat16, device=dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    table = torch.from_numpy((np.arange(E) % n_blobs).astype(np.int32)).to(dev)
    out = {}
    for name, fmt in (("int4_g32", gen.FMT_INT4_G32), ("int4_g128", gen.FMT_INT4_G128), ("int8_g32", gen.FMT_INT8_G32),
                      ("nvfp4", gen.FMT_NVFP4)):
        stride = lib.moe_fmt_slot_stride(fmt, H, I)
        blob = lib.moe_fmt_blob_bytes(fmt, H, I)
        slots = torch.empty(n_blobs * stride, dtype=torch.uint8, device=dev)
        for b in range(n_blobs):
            slots[b * stride : (b + 1) * stride].copy_(torch.from_numpy(harness.pack_expert_fmt(seed, 0, b, H, I, fmt)))
        nb = lib.moe_fmt_workspace_bytes(fmt, 1, H, I, E, K, 0)
        ws = torch.empty(nb, dtype=torch.uint8, device=dev)

        def call(i):
            lib.moe_expert_ffn_fmt(fmt, x, ids_d[i], wts, 1, H, I, E, K, table, slots, stride, None, y, ws, nb, status)

        for i in range(8):
            call(steps + i)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for i in range(steps):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        if int(status.item()) != 0:
            raise RuntimeError(f"device status {int(status.item())}")
        us = e0.elapsed_time(e1) * 1e3 / steps
        out[name] = {"us_per_layer": round(us, 2), "blob_bytes": blob,
                     "hbm_gbs": round(K * blob / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(K * blob / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
        if name != "int4_g128":  # a prompt: 2,048 tokens routed over the 64 packed experts
            Tp, Ep = 2048, n_blobs
            lg = torch.from_numpy(gen.normal_logits(seed, 1, Tp, Ep)).to(dev)
            ids_p = torch.empty(Tp, K, dtype=torch.int32, device=dev)
            wts_p = torch.empty(Tp, K, dtype=torch.float32, device=dev)
            lib.moe_route(None, None, lg, Tp, H, Ep, K, 0, ids_p, wts_p)
            xp = harness.bf16_tensor(gen.activations_bf16(seed, 1, Tp, H), dev)
            yp = torch.empty(Tp, H, dtype=torch.bfloat16, device=dev)
            tbl_p = torch.arange(Ep, dtype=torch.int32, device=dev)
            nbp = lib.moe_fmt_workspace_bytes(fmt, Tp, H, I, Ep, K, 0)
            wsp = torch.empty(nbp, dtype=torch.uint8, device=dev)

            def prompt():
                lib.moe_expert_ffn_fmt(fmt, xp, ids_p, wts_p, Tp, H, I, Ep, K, tbl_p, slots, stride, None, yp, wsp,
                                       nbp, status)

            prompt()
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record()
            for _ in range(5):
                prompt()
            e1.record()
            torch.cuda.synchronize()
            if int(status.item()) != 0:
                raise RuntimeError(f"device status {int(status.item())}")
            ms = e0.elapsed_time(e1) / 5
            flops = 2.0 * Tp * K * 3 * H * I
            out[name]["prompt_t2048_e64_ms"] = round(ms, 3)
            out[name]["prompt_t2048_e64_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
            del wsp, yp, xp
        log(f"  formats {name}: {out[name]}")
        del slots, ws
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------ CPU oracle baseline


def cpu_baseline(w, n_layers):
    """The oracle, as it stands, on the first n_layers decode layers of the headline workload."""
    from oracle import moe_ref as R
    from synth import gen

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = 1
    t_total = 0.0
    for layer in range(n_layers):
        xb = gen.activations_bf16(w.seed, layer, w.T, w.H)
        wr = gen.router_weight(w.seed, layer, w.E, w.H)
        tensors = {}
        ids = R.select_topk(R.router_logits(xb, wr), w.K)
        for e in set(ids.ravel().tolist()):  # input generation stays outside the timed region
            tensors[e] = gen.expert_tensors(w.seed, layer, e, w.H, w.I)

        def experts(e, layer=layer, tensors=tensors):
            return R.Expert(tensors[e], w.H, w.I)

        t = time.perf_counter()
        R.moe_layer(xb, experts, w.K, w_router=wr)
        t_total += time.perf_counter() - t
    per_layer = t_total / n_layers
    return {
        "value": round(1.0 / (per_layer * w.layers), 5),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n_layers} of the {w.layers} decode layers (1 token each, fp64 NumPy oracle incl. "
        f"dequantisation); {per_layer:.2f} s per layer, scaled to one {w.layers}-layer token",
    }


def cpu_matrix():
    """The oracle on a bounded sample of each workload, at one thread and at all cores
    (NumPy's BLAS pool; the oracle's own loops are single-threaded Python). Expert
    tensors are generated outside the timed region; each used expert is dequantised
    (fp64) once inside it, on first use. Rates are scaled from the sample to the
    workload's unit: tokens/s of the layer stack (decode, paged) or of one layer."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import moe_ref as R
    from synth import gen

    all_cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])

    def time_layer(w, layer, tokens, logits=None, with_router=False):
        xb = gen.activations_bf16(w.seed, layer, w.T, w.H)[:tokens]
        wr = gen.router_weight(w.seed, layer, w.E, w.H) if with_router else None
        lg = None if logits is None else logits[:tokens]
        ids = R.select_topk(R.router_logits(xb, wr) if with_router else lg, w.K)
        tensors = {e: gen.expert_tensors(w.seed, layer, e, w.H, w.I) for e in set(ids.ravel().tolist())}
        sh_t = gen.expert_tensors(w.seed, layer, gen.SHARED_EXPERT, w.H, w.I) if w.shared else None
        t = time.perf_counter()
        built = {}

        def experts(e):
            if e not in built:
                built[e] = R.Expert(tensors[e], w.H, w.I)
            return built[e]

        shared = R.Expert(sh_t, w.H, w.I) if sh_t is not None else None
        R.moe_layer(xb, experts, w.K, logits=lg, w_router=wr, shared=shared)
        return time.perf_counter() - t

    W = gen.WORKLOADS
    cases = [  # (workload, sample, tokens per sample, scale: seconds of the sample -> tokens/s)
        (W["tiny_t4_h256_e8_k2"], "the whole layer (4 tokens)", lambda w: time_layer(w, 0, 4, with_router=True),
         lambda w, t: 4 / t),
        (W["decode_t1_h4096_e256_k8_i1536_x48"], "1 of 48 layers (1 token), scaled to 48 layers",
         lambda w: time_layer(w, 0, 1, with_router=True), lambda w, t: 1 / (t * w.layers)),
        (W["batched_t16_h2048_e128_k8_i768_zipf"], "the whole layer (16 tokens)",
         lambda w: time_layer(w, 0, 16, logits=gen.zipf_logits(w.seed, 0, w.T, w.E)), lambda w, t: 16 / t),
        (W["prefill_t9940_h4096_e256_k8_i1536"], "4 of the 9,940 tokens, scaled to tokens/s",
         lambda w: time_layer(w, 0, 4, logits=gen.normal_logits(w.seed, 0, 4, w.E)), lambda w, t: 4 / t),
        (W["paged_t1_h4096_e256s1_k6_i2048_x43"], "1 of 43 layers (1 token, 6 routed + 1 shared), scaled to 43 layers",
         lambda w: time_layer(w, 0, 1, logits=gen.locality_logits(w.seed, 1, 1, w.E, w.K)[0]),
         lambda w, t: 1 / (t * w.layers)),
    ]
    out = []
    for w, sample, run, scale in cases:
        row = {"workload": w.name, "unit": "tokens/s", "sample": sample}
        for label, n in (("1_thread", 1), ("all_cores", all_cores)):
            with threadpool_limits(n):
                row[label] = round(scale(w, run(w)), 6)
        row["all_cores_threads"] = all_cores
        log(f"  oracle {w.name}: {row['1_thread']} / {row['all_cores']} tokens/s")
        out.append(row)
    return out


def hbm_read_probe(dev, gib=2, reps=5):
    """GB/s of a plain streaming read: torch's sum over a 2 GiB int64 tensor (best of 5; the
    integer sum keeps up with HBM where torch's fp32 reductions do not)."""
    import torch

    t = torch.ones(gib << 27, dtype=torch.int64, device=dev)
    t.sum()
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        e0, e1 = ev(), ev()
        e0.record()
        t.sum()
        e1.record()
        torch.cuda.synchronize()
        best = max(best, (gib << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del t
    torch.cuda.empty_cache()
    return best


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {a.gpus} is not supported: the layer has no multi-GPU path "
              "(expert-parallel sharding over xGMI is designed, not built)", file=sys.stderr)
        sys.exit(2)
    import torch

    from quantized_routed_expert_moe_amd import lib

    lib.load()
    dev = "cuda:0"
    # The cyclic garbage collector runs only between legs (gc.collect() before
    # each): a full pass over a process holding torch takes tens of milliseconds,
    # and one that started inside a timed region would stall the host while the
    # GPU drains its queue.
    gc.collect()
    gc.disable()
    legs = set(a.legs.split(","))
    if a.copy_probe_mib:
        src = torch.empty(a.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {a.copy_probe_mib} MiB read + {a.copy_probe_mib} MiB written")
        del src, dst
    gc.collect()
    w, d = decode_leg(a, dev)
    traffic = decode_traffic()
    probe_gbs = hbm_read_probe(dev)
    out = {
        "metric": "MoE-layer decode tokens/s (one token through 48 layers) + achieved HBM GB/s",
        "value": round(d["tok_s"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(d["ms_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights (fp16 group scales); bf16 x and y, x and h fed to the dot products as fp16; fp32 accumulate",
        "data": "synthetic (seeded)",
        "config": {
            "workload": w.name,
            "tokens": w.T,
            "layers": w.layers,
            "hidden": w.H,
            "experts": w.E,
            "top_k": w.K,
            "intermediate": w.I,
            "group": w.g,
            "arena_slots": w.slots,
            "hip_graph": d["graph"],
            "routing": "one-pass (router GEMV + top-k + gate/up in one dispatch)" if d["onepass"]
            else "two dispatches (router GEMV, then top-k) before the gate/up dispatch",
        },
        # the same layers and tokens with the other routing (same bits, checked)
        "other_routing_tokens_per_s": round(1000.0 / d["other_ms_step"], 2),
        "hbm_gbs": round(d["layer_gbs"], 1),
        "hbm_frac": round(d["layer_gbs"] / HBM_PEAK_GBS, 4),
        "per_layer_us": {k: round(v, 2) for k, v in d["us"].items()} | {"step_avg": round(d["ms_step"] * 1e3 / w.layers, 2)},
        "roofline": {
            "kernel": "dec_gateup_kernel (moe_ffn_gate_up, single-token path)",
            "bound": "hbm",
            "achieved": round(d["gu_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(d["gu_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic.get("dec_gateup_kernel"),
            "bytes_per_launch": d["bytes"]["gate_up"],
        },
        "roofline_down": {
            "kernel": "dec_down_kernel (moe_ffn_down, single-token path)",
            "bound": "hbm",
            "achieved": round(d["dn_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(d["dn_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": traffic.get("dec_down_kernel"),
            "bytes_per_launch": d["bytes"]["down"],
        },
        "wall_s_timed": round(d["wall"], 4),
        # context: a plain streaming read (torch's int64 sum over 2 GiB) on the same GPU
        "hbm_read_probe_gbs": round(probe_gbs, 1),
        "frac_of_read_probe": {"gate_up": round(d["gu_gbs"] / probe_gbs, 4), "down": round(d["dn_gbs"] / probe_gbs, 4)},
        "workloads": {},
    }
    torch.cuda.empty_cache()
    if "prefill" in legs:
        gc.collect()
        wp, p = prefill_leg(a, dev)
        out["workloads"]["prefill"] = {
            "workload": wp.name,
            "tokens_per_s": round(p["tok_s"], 1),
            "ms_per_layer": round(p["ms_layer"], 3),
            "stage_us": {k: round(v, 1) for k, v in p["us"].items()},
            "tflops": round(p["tflops_layer"], 1),
            "mfma_frac_layer": round(p["tflops_layer"] / BF16_PEAK_TFLOPS, 4),
            "roofline_gate_up": {"bound": "mfma", "achieved": round(p["tflops_gate_up"], 1), "peak": BF16_PEAK_TFLOPS,
                                 "unit": "TFLOP/s", "frac": round(p["tflops_gate_up"] / BF16_PEAK_TFLOPS, 4)},
            "roofline_down": {"bound": "mfma", "achieved": round(p["tflops_down"], 1), "peak": BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(p["tflops_down"] / BF16_PEAK_TFLOPS, 4)},
            "useful_flops_per_layer": p["flops"],
        }
        torch.cuda.empty_cache()
    if "batched" in legs:
        gc.collect()
        wb, b = batched_leg(a, dev)
        out["workloads"]["batched"] = {
            "workload": wb.name,
            "tokens_per_s_per_layer": round(b["tok_s"], 1),
            "us_per_layer": round(b["us_layer"], 2),
            "distinct_experts_per_layer": round(b["distinct_experts"], 2),
            "hbm_gbs": round(b["hbm_gbs"], 1),
            "hbm_frac": round(b["hbm_gbs"] / HBM_PEAK_GBS, 4),
        }
    if "route_variants" in legs:
        gc.collect()
        out["workloads"]["route_variants"] = {"experts": 256, "top_k": 8, "from": "logits"} | route_variants_leg(dev)
    if "paged" in legs:
        torch.cuda.empty_cache()
        gc.collect()
        wq, q = paged_leg(a, dev)
        out["workloads"]["paged"] = {
            "workload": wq.name,
            "tokens_per_s": round(q["tok_s"], 2),
            "ms_per_token": round(q["ms_per_token"], 3),
            "hit_rate": round(q["hit_rate"], 4),
            "misses_per_layer_step": round(q["misses_per_layer_step"], 3),
            "h2d_gbs": round(q["h2d_gbs"], 2),
            "h2d_pinned_copy_gbs": round(q["h2d_peak_gbs"], 2),
            "bit_identical_to_resident": q["identical"],
            "host_weight_sets": 1,
            "sequencing": "moe_paged_layer (native, speculative FFN, ids to the host through a polled word)",
            "event_handshake_tokens_per_s": round(q["event_handshake_tok_s"], 2),
            "event_handshake_h2d_gbs": round(q["event_handshake_h2d_gbs"], 2),
            "python_sequenced_tokens_per_s": round(q["python_tok_s"], 2),
            "resident_tokens_per_s": round(q["resident_tok_s"], 1),
            "resident_hbm_gbs": round(q["resident_hbm_gbs"], 1),
            "resident_hbm_frac": round(q["resident_hbm_gbs"] / HBM_PEAK_GBS, 4),
        }
    if "readahead" in legs:
        torch.cuda.empty_cache()
        gc.collect()
        wr, r = readahead_leg(a, dev)
        out["workloads"]["readahead_paged"] = {"workload": wr.name, "predictor": "next layer's router on this "
                                               "layer's input, top-P", "residual_stream": {"a": 0.99, "rho": 0.15}} | r
    if "formats" in legs:
        gc.collect()
        out["workloads"]["formats"] = {"workload": "decode_t1_h4096_e256_k8_i1536 expert FFN per weight format",
                                       "by_format": formats_leg(dev)}
    if "chunked" in legs:
        torch.cuda.empty_cache()
        gc.collect()
        wc, c = chunked_leg(a, dev)
        out["workloads"]["chunked_paged_prefill"] = {"workload": wc.name, "arena_slots": wc.slots,
                                                     "experts_per_pass": wc.slots // 2, "by_chunk": c}
    if not a.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(w, min(a.cpu_layers, w.layers))
        if a.cpu_matrix:
            out["cpu_baseline"]["by_workload"] = cpu_matrix()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
