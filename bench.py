"""Benchmark of the int4 routed-expert MoE layer on one MI355X.

Default workload: single-token decode through 48 MoE layers (hidden 4096, 256
experts, top-8, intermediate 1536, int4 group-32 experts with fp16 scales, fp32
router, a 64-slot arena per layer with a seeded random expert-to-slot map and
every routed expert resident). One step = one token through all 48 layers:
per layer moe_route (router GEMV + softmax top-k) and moe_expert_ffn (int4
SwiGLU experts + combine). Inputs are seeded synthetic tensors already resident
in HBM. Prints one JSON line.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=48)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-layers", type=int, default=3, help="layers in the oracle's timed sample")
    p.add_argument("--graph", type=int, default=1, help="replay the layer stack as a HIP graph (1) or eagerly (0)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_decode_stack(w, layers, dev):
    import numpy as np
    import torch

    from quantized_routed_expert_moe_amd import harness, lib
    from synth import gen

    stacks = []
    run = harness.LayerRunner(w, dev)
    t0 = time.time()
    lg = torch.empty(w.T, w.E, dtype=torch.float32, device=dev)
    for layer in range(layers):
        xb = gen.activations_bf16(w.seed, layer, w.T, w.H)
        # routing first (set-up only): the routed experts are the ones placed in the arena
        x = harness.bf16_tensor(xb, dev)
        wr = torch.from_numpy(gen.router_weight(w.seed, layer, w.E, w.H)).to(dev)
        lib.moe_route(x, wr, lg, w.T, w.H, w.E, w.K, 0, run.ids, run.wts)
        routed = sorted(set(run.ids.cpu().numpy().ravel().tolist()))
        L = harness.make_layer(w, layer, dev, slots=w.slots, experts=routed, place_seed=1000 + layer, x_bits=xb)
        stacks.append(L)
        if layer % 8 == 7:
            log(f"  packed layers 0..{layer} ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize()
    return stacks


def cpu_baseline(w, n_layers):
    """The oracle, as it stands, on the first n_layers layers of the same workload."""
    import numpy as np

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

        def experts(e, layer=layer, tensors=tensors):
            return R.Expert(tensors.setdefault(e, gen.expert_tensors(w.seed, layer, e, w.H, w.I)), w.H, w.I)

        # input generation is outside the timed region: draw the routed experts first
        ids = R.select_topk(R.router_logits(xb, wr), w.K)
        for e in set(ids.ravel().tolist()):
            tensors[e] = gen.expert_tensors(w.seed, layer, e, w.H, w.I)
        t = time.perf_counter()
        R.moe_layer(xb, experts, w.K, w_router=wr)
        t_total += time.perf_counter() - t
    per_layer = t_total / n_layers
    return {
        "value": 1.0 / (per_layer * w.layers),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{n_layers} of {w.layers} layers (1 token each), fp64 NumPy oracle; "
        f"{per_layer:.2f} s per layer, scaled to a {w.layers}-layer token",
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported (this build has no multi-GPU path)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from quantized_routed_expert_moe_amd import harness, lib
    from synth import gen

    lib.load()
    dev = "cuda:0"
    base = gen.WORKLOADS["decode_t1_h4096_e256_k8_i1536_x48"]
    w = gen.Workload(base.name, base.T, base.H, base.E, base.K, base.I, a.layers, base.slots, base.router, base.seed)
    log(f"building {w.layers} layers of {w.name}")
    stacks = build_decode_stack(w, w.layers, dev)
    run = harness.LayerRunner(w, dev)
    stream = torch.cuda.Stream()
    blob = lib.moe_blob_bytes(w.H, w.I)
    bytes_router = w.E * w.H * 4 + w.T * w.H * 2 + w.T * w.E * 4
    bytes_ffn = w.K * blob + w.T * w.H * 2 * 2  # routed experts + x read + y write
    bytes_layer = bytes_router + bytes_ffn

    def step():
        for L in stacks:
            run.route(L, stream)
            run.ffn(L, stream)

    with torch.cuda.stream(stream):
        for _ in range(a.warmup):
            step()
    stream.synchronize()
    if int(run.status.item()) != 0:
        raise RuntimeError(f"device status {int(run.status.item())}")
    graph = None
    if a.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        stream.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(a.steps):
            if graph is not None:
                graph.replay()
            else:
                step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / a.steps
    tok_s = 1000.0 / ms_step

    # per-call durations with HIP events on the launch stream (diagnostics and roofline)
    n_probe = min(len(stacks), 48)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
            torch.cuda.Event(enable_timing=True)) for _ in range(n_probe)]
    with torch.cuda.stream(stream):
        for L, (e0, e1, e2) in zip(stacks[:n_probe], evs):
            e0.record(stream)
            run.route(L, stream)
            e1.record(stream)
            run.ffn(L, stream)
            e2.record(stream)
    torch.cuda.synchronize()
    t_route = float(np.mean([e0.elapsed_time(e1) for e0, e1, _ in evs])) * 1e3
    t_ffn = float(np.mean([e1.elapsed_time(e2) for _, e1, e2 in evs])) * 1e3
    achieved = bytes_ffn / (t_ffn * 1e-6) / 1e9

    out = {
        "metric": "MoE-layer decode tokens/s (48 layers per token) + achieved HBM GB/s",
        "value": round(tok_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4 weights (fp16 group scales), bf16 activations, fp32 accumulate",
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
            "hip_graph": bool(graph is not None),
        },
        "hbm_gbs_layer": round(bytes_layer * w.layers / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac_layer": round(bytes_layer * w.layers / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "per_layer_us": {"route": round(t_route, 2), "expert_ffn": round(t_ffn, 2), "step_avg": round(ms_step * 1e3 / w.layers, 2)},
        "roofline": {
            "kernel": "moe_expert_ffn (gate/up + down/combine)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
        },
        "wall_s_timed": round(wall, 4),
    }
    if not a.no_cpu_baseline:
        log("timing the CPU oracle")
        out["cpu_baseline"] = cpu_baseline(w, min(a.cpu_layers, w.layers))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
