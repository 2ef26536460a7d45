"""Per-workgroup timeline of one MoE layer, from the instrumented library.

Loads ``libmoe_timeline.so`` (the same kernels as ``libmoe.so`` plus per-workgroup
stamps, include/moe_timeline.h) in place of the product library, runs a workload
the way ``bench.py`` does, and prints a Markdown summary of the last layer's
dispatches: when each kernel's workgroups started, passed their named points and
finished (µs from the layer's first workgroup), how they spread over the XCDs and
compute units, and which workgroup ended last.

    python -m quantized_routed_expert_moe_amd.timeline decode [--routing onepass|separate]
    python -m quantized_routed_expert_moe_amd.timeline batched

Needs a GPU and the instrumented build (``python -m quantized_routed_expert_moe_amd.build
--timeline``; ``__graft_entry__.build()`` makes both libraries).
"""

from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

from . import build as _build
from . import lib

TICK_US = 0.01  # s_memrealtime runs at 100 MHz
MAX_BLOCKS, MARKS, WORDS = 8192, 5, 8
KERNELS = {
    "router_gemv1_kernel": 0,
    "route_select_kernel": 1,
    "dec_route_gateup_kernel": 2,
    "dec_gateup_kernel": 3,
    "dec_down_kernel": 4,
    "bat_plan_kernel": 5,
    "bmx_gateup_kernel": 6,
    "bmx_down_kernel": 7,
    "bat_combine_kernel": 8,
}
MARK_NAMES = {
    "dec_route_gateup_kernel": {0: "logit published", 1: "all logits seen (selector)", 2: "slots published (selector)",
                                3: "slot known", 4: "weight loads issued"},
    "dec_gateup_kernel": {3: "slot known", 4: "weight loads issued"},
    "dec_down_kernel": {0: "weight loads issued", 1: "h staged", 2: "sums done"},
    "bmx_gateup_kernel": {0: "unit record loaded", 1: "A rows in LDS", 2: "MFMAs done"},
    "bmx_down_kernel": {0: "unit record loaded", 1: "A rows in LDS", 2: "MFMAs done"},
}


def load():
    """The instrumented library, loaded as the binding's library (before any other use)."""
    if lib._lib is not None and getattr(lib._lib, "_name", "") != _build.TIMELINE_LIB:
        raise RuntimeError("the product library is already loaded in this process")
    L = lib.load(_build.TIMELINE_LIB)
    L.moe_timeline_read.restype = ctypes.c_int
    L.moe_timeline_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int]
    L.moe_timeline_clear.restype = ctypes.c_int
    L.moe_timeline_clear.argtypes = []
    return L


def clear(L):
    st = L.moe_timeline_clear()
    if st != 0:
        raise lib.MoeError(st, "moe_timeline_clear")


def read(L, kernel: str, blocks: int = MAX_BLOCKS) -> np.ndarray:
    """Rows [blocks][8] (uint64) of the kernel's last dispatch; rows with no start dropped."""
    buf = np.zeros((blocks, WORDS), dtype=np.uint64)
    st = L.moe_timeline_read(KERNELS[kernel], buf.ctypes.data, blocks)
    if st != 0:
        raise lib.MoeError(st, "moe_timeline_read")
    idx = np.nonzero(buf[:, 1])[0]
    out = buf[idx].astype(np.int64)
    # a mark outside its row's [start, end] was left by an earlier dispatch
    marks = out[:, 2:2 + MARKS]
    marks[(marks < out[:, 1:2]) | (marks > out[:, 7:8])] = 0
    return np.concatenate([idx[:, None], out], axis=1)  # [block, hw, start, m0..m4, end]


def cu_key(hw_word: np.ndarray) -> np.ndarray:
    """(XCD, shader engine, shader array, compute unit) packed into one integer."""
    xcc = hw_word >> 32
    hw = hw_word & 0xFFFFFFFF
    return (xcc << 16) | (((hw >> 13) & 7) << 8) | (((hw >> 12) & 1) << 4) | ((hw >> 8) & 15)


def max_resident(rows: np.ndarray) -> int:
    """Most workgroups of this dispatch seen on one compute unit at the same time."""
    best = 0
    keys = cu_key(rows[:, 1])
    for k in np.unique(keys):
        r = rows[keys == k]
        ev = sorted([(s, 1) for s in r[:, 2]] + [(e, -1) for e in r[:, 8]], key=lambda t: (t[0], t[1]))
        cur = 0
        for _, d in ev:
            cur += d
            best = max(best, cur)
    return best


def q(v, p):
    return float(np.percentile(v, p)) if len(v) else float("nan")


def summarize(name: str, rows: np.ndarray, t0: int) -> list[str]:
    us = lambda v: (np.asarray(v, dtype=np.float64) - t0) * TICK_US  # noqa: E731
    start, end = rows[:, 2], rows[:, 8]
    dur = (end - start) * TICK_US
    xcc = rows[:, 1] >> 32
    out = [f"### `{name}`: {len(rows)} workgroups", ""]
    out.append("| point | first | median | 90th pct | last |")
    out.append("|---|---|---|---|---|")
    out.append(f"| start | {us(start).min():.2f} | {q(us(start), 50):.2f} | {q(us(start), 90):.2f} | {us(start).max():.2f} |")
    for m, label in MARK_NAMES.get(name, {}).items():
        col = rows[:, 3 + m]
        col = col[col != 0]
        if len(col):
            out.append(f"| {label} ({len(col)} wg) | {us(col).min():.2f} | {q(us(col), 50):.2f} | "
                       f"{q(us(col), 90):.2f} | {us(col).max():.2f} |")
    out.append(f"| end | {us(end).min():.2f} | {q(us(end), 50):.2f} | {q(us(end), 90):.2f} | {us(end).max():.2f} |")
    out.append("")
    out.append(f"Workgroup duration: median {np.median(dur):.2f} µs, 90th percentile {q(dur, 90):.2f}, "
               f"max {dur.max():.2f}. Most resident on one compute unit at once: {max_resident(rows)}.")
    per = []
    for x in range(8):
        sel = xcc == x
        if sel.any():
            per.append(f"XCD {x}: {int(sel.sum())} wg, last end {us(end[sel]).max():.2f}")
    out.append("Per XCD: " + "; ".join(per) + ".")
    last = rows[np.argmax(end)]
    marks = ", ".join(f"{MARK_NAMES.get(name, {}).get(m, m)} {us(last[3 + m]):.2f}"
                      for m in range(MARKS) if last[3 + m] != 0)
    out.append(f"Last to end: workgroup {int(last[0])} on XCD {int(last[1] >> 32)}, started {us(last[2]):.2f}"
               + (f", {marks}" if marks else "") + f", ended {us(last[8]):.2f}.")
    out.append("")
    return out


def layer_report(L, kernels: list[str], title: str) -> str:
    data = {k: read(L, k) for k in kernels}
    data = {k: v for k, v in data.items() if len(v)}
    t0 = min(int(v[:, 2].min()) for v in data.values())
    order = sorted(data, key=lambda k: int(data[k][:, 2].min()))
    lines = [f"## {title}", "", "| kernel | workgroups | first start | last start | last end | span |",
             "|---|---|---|---|---|---|"]
    for k in order:
        r = data[k]
        lines.append(f"| `{k}` | {len(r)} | {(r[:, 2].min() - t0) * TICK_US:.2f} | {(r[:, 2].max() - t0) * TICK_US:.2f} | "
                     f"{(r[:, 8].max() - t0) * TICK_US:.2f} | {(r[:, 8].max() - r[:, 2].min()) * TICK_US:.2f} |")
    lines.append("")
    for k in order:
        lines += summarize(k, data[k], t0)
    return "\n".join(lines)


def decode(routing: str, layers: int) -> str:
    import torch

    from synth import gen

    from . import harness

    L = load()
    dev = "cuda:0"
    base = gen.WORKLOADS["decode_t1_h4096_e256_k8_i1536_x48"]
    w = gen.Workload(base.name, base.T, base.H, base.E, base.K, base.I, layers, base.slots, base.router, base.seed)
    print(f"decode: building {w.layers} layers", file=sys.stderr, flush=True)
    stacks = harness.decode_stack(w, dev)
    flags = lib.MOE_ROUTE_ONEPASS if routing == "onepass" else 0
    run = harness.StackRunner(w, stacks, dev, route_flags=flags)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        run.step(stream)
    stream.synchronize()
    run.capture(stream)
    for _ in range(5):
        run.replay(stream)
    stream.synchronize()
    clear(L)
    run.replay(stream)
    stream.synchronize()
    if int(run.status.item()) != 0:
        raise RuntimeError(f"device status {int(run.status.item())}")
    kernels = (["dec_route_gateup_kernel", "dec_down_kernel"] if routing == "onepass" else
               ["router_gemv1_kernel", "route_select_kernel", "dec_gateup_kernel", "dec_down_kernel"])
    title = (f"{w.name}, layer {w.layers - 1} of a {w.layers}-layer HIP graph replay, "
             f"{'one-pass' if routing == 'onepass' else 'separate'} routing")
    return layer_report(L, kernels, title)


def batched(n_sets: int) -> str:
    import torch

    from synth import gen

    from . import harness

    L = load()
    dev = "cuda:0"
    w = gen.WORKLOADS["batched_t16_h2048_e128_k8_i768_zipf"]
    print(f"batched: packing {n_sets} layer weight sets", file=sys.stderr, flush=True)
    sets = []
    for layer in range(n_sets):
        lg = gen.zipf_logits(w.seed, layer, w.T, w.E)
        top = np.argsort(-lg, axis=1, kind="stable")[:, : w.K]  # set-up only: which experts to pack
        sets.append(harness.make_layer(w, layer, dev, experts=sorted(set(top.ravel().tolist())), place_seed=layer,
                                       logits=lg))
    run = harness.LayerRunner(w, dev)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for _ in range(3):
            for Ly in sets:
                run.layer(Ly, stream)
    stream.synchronize()
    clear(L)
    with torch.cuda.stream(stream):
        for Ly in sets:
            run.layer(Ly, stream)
    stream.synchronize()
    if int(run.status.item()) != 0:
        raise RuntimeError(f"device status {int(run.status.item())}")
    units = len(set(run.ids.cpu().numpy().ravel().tolist()))
    title = (f"{w.name}, layer set {n_sets - 1} of {n_sets} ({units} distinct experts), after the other sets; "
             "one moe_layer call per set")
    return layer_report(L, ["route_select_kernel", "bat_plan_kernel", "bmx_gateup_kernel", "bmx_down_kernel",
                            "bat_combine_kernel"], title)


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("workload", choices=["decode", "batched"])
    p.add_argument("--routing", choices=["onepass", "separate"], default="onepass")
    p.add_argument("--layers", type=int, default=48)
    p.add_argument("--sets", type=int, default=16)
    a = p.parse_args(argv)
    if not os.path.exists(_build.TIMELINE_LIB):
        raise ImportError(f"{_build.TIMELINE_LIB} is missing: build it with "
                          "`python -m quantized_routed_expert_moe_amd.build --timeline`")
    print(decode(a.routing, a.layers) if a.workload == "decode" else batched(a.sets), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
