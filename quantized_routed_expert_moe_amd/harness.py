"""Device-side set-up for the layer: pack seeded experts into arenas and run a layer.

Harness code only: input generation comes from ``synth``, packing from the C
library (``moe_pack_expert``), and torch is used for device memory, copies and
streams. Nothing here computes any part of the layer.
"""

from __future__ import annotations

import dataclasses

import numpy as np
import torch

from synth import gen

from . import lib


def pack_expert(seed: int, layer: int, expert: int, H: int, I: int, g: int = 32) -> np.ndarray:
    """Seeded expert -> host blob (uint8, one slot stride long, zero padded)."""
    t = gen.expert_tensors(seed, layer, expert, H, I, g)
    out = np.zeros(lib.moe_slot_stride(H, I, g), dtype=np.uint8)
    lib.moe_pack_expert(
        t["qg"], t["qu"], t["qd"], t["sg"].view(np.uint16), t["su"].view(np.uint16), t["sd"].view(np.uint16),
        H, I, g, out,
    )
    return out


def pack_expert_fmt(seed: int, layer: int, expert: int, H: int, I: int, fmt: int) -> np.ndarray:
    """Seeded expert in format ``fmt`` -> host blob (uint8, one slot stride long)."""
    t = gen.expert_tensors_fmt(seed, layer, expert, H, I, fmt)
    out = np.zeros(lib.moe_fmt_slot_stride(fmt, H, I), dtype=np.uint8)
    if fmt == gen.FMT_NVFP4:
        lib.moe_pack_expert_nvfp4(t["qg"], t["qu"], t["qd"], t["sg"], t["su"], t["sd"], t["global"], H, I, out)
        return out
    lib.moe_pack_expert_fmt(
        fmt, t["qg"], t["qu"], t["qd"], t["sg"].view(np.uint16), t["su"].view(np.uint16), t["sd"].view(np.uint16),
        H, I, out,
    )
    return out


def bf16_tensor(bits: np.ndarray, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def placeholder_blob_fill(slots: torch.Tensor) -> None:
    """Fill unused slots with a valid all-zero-code expert (nibbles 0x8 = q 0)."""
    slots.fill_(0x88)


@dataclasses.dataclass
class DeviceLayer:
    w: gen.Workload
    layer: int
    x: torch.Tensor  # bf16 [T, H]
    wr: torch.Tensor | None  # fp32 [E, H] or None (logits supplied)
    logits: torch.Tensor  # fp32 [T, E]
    slots: torch.Tensor  # uint8 [S * stride]
    table: torch.Tensor  # int32 [E]
    shared: torch.Tensor | None  # uint8 [stride]
    arena: lib.Arena
    stride: int


def make_layer(w: gen.Workload, layer: int, device, slots: int | None = None, experts=None, place_seed=None,
               logits: np.ndarray | None = None, x_bits: np.ndarray | None = None, fill_unused=True) -> DeviceLayer:
    """Build one layer on ``device``.

    ``experts``: the expert ids to pack and place (default: all E). They go to
    slots given by a seeded random permutation when ``place_seed`` is set, else
    to slots 0, 1, ... in order. Other slots hold the zero-code placeholder.
    """
    T, H, E, I = w.T, w.H, w.E, w.I
    S = slots if slots is not None else E
    stride = lib.moe_slot_stride(H, I, w.g)
    xb = x_bits if x_bits is not None else gen.activations_bf16(w.seed, layer, T, H)
    x = bf16_tensor(xb, device)
    if w.router == "gemv":
        wr = torch.from_numpy(gen.router_weight(w.seed, layer, E, H)).to(device)
        lg = torch.empty(T, E, dtype=torch.float32, device=device)
    else:
        wr = None
        if logits is None:
            logits = {"normal": gen.normal_logits, "zipf": gen.zipf_logits}[w.router](w.seed, layer, T, E)
        lg = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(device)
    sl = torch.empty(S * stride, dtype=torch.uint8, device=device)
    if fill_unused:
        placeholder_blob_fill(sl)
    table = torch.full((E,), -1, dtype=torch.int32, device=device)
    arena = lib.Arena(E, S, lib.moe_blob_bytes(H, I, w.g), stride, sl, table, None)
    ex = list(range(E)) if experts is None else list(experts)
    if len(ex) > S:
        raise ValueError("more experts than slots")
    if place_seed is not None:
        order = np.random.default_rng(place_seed).permutation(S)[: len(ex)]
    else:
        order = np.arange(len(ex))
    host_table = np.full(E, -1, dtype=np.int32)
    for e, s in zip(ex, order):
        blob = pack_expert(w.seed, layer, int(e), H, I, w.g)
        sl[int(s) * stride : (int(s) + 1) * stride].copy_(torch.from_numpy(blob), non_blocking=False)
        arena.place(int(e), int(s))
        host_table[int(e)] = int(s)
    table.copy_(torch.from_numpy(host_table))
    shared = None
    if w.shared:
        shared = torch.from_numpy(pack_expert(w.seed, layer, gen.SHARED_EXPERT, H, I, w.g)).to(device)
    return DeviceLayer(w, layer, x, wr, lg, sl, table, shared, arena, stride)


class LayerRunner:
    """Route + expert FFN of one layer with preallocated outputs and workspace."""

    def __init__(self, w: gen.Workload, device, flags: int = 0):
        self.w, self.flags = w, flags
        T, H, E, K, I = w.T, w.H, w.E, w.K, w.I
        self.ids = torch.empty(T, K, dtype=torch.int32, device=device)
        self.wts = torch.empty(T, K, dtype=torch.float32, device=device)
        self.y = torch.empty(T, H, dtype=torch.bfloat16, device=device)
        self.ws_bytes = lib.moe_ffn_workspace_bytes(T, H, I, E, K, w.shared, flags)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)

    def route(self, L: DeviceLayer, stream=None, renorm=False):
        w = self.w
        lib.moe_route(L.x, L.wr, L.logits, w.T, w.H, w.E, w.K, lib.MOE_ROUTE_RENORM if renorm else 0, self.ids,
                      self.wts, stream)

    def ffn(self, L: DeviceLayer, stream=None, y=None, stage="both", ids=None, wts=None):
        """Expert FFN of the layer: stage "both", "gate_up" or "down" (ids / wts default to the last route)."""
        w = self.w
        fn = {"both": lib.moe_expert_ffn, "gate_up": lib.moe_ffn_gate_up, "down": lib.moe_ffn_down}[stage]
        fn(L.x, self.ids if ids is None else ids, self.wts if wts is None else wts, w.T, w.H, w.I, w.E, w.K, w.g,
           L.table, L.slots, L.stride, L.shared, self.y if y is None else y, self.ws, self.ws_bytes, self.status,
           self.flags, stream)

    def layer(self, L: DeviceLayer, stream=None, renorm=False):
        """The whole layer in one call (moe_layer): same results as route() then ffn()."""
        w = self.w
        lib.moe_layer(L.x, L.wr, L.logits, w.T, w.H, w.I, w.E, w.K, w.g, lib.MOE_ROUTE_RENORM if renorm else 0,
                      self.ids, self.wts, L.table, L.slots, L.stride, L.shared, self.y, self.ws, self.ws_bytes,
                      self.status, self.flags, stream)

    def __call__(self, L: DeviceLayer, stream=None):
        self.route(L, stream)
        self.ffn(L, stream)
        return self.y


def decode_stack(w: gen.Workload, device, log=None) -> list[DeviceLayer]:
    """The layers of single-token decode: per layer a fresh seeded x and router, and an
    arena of ``w.slots`` slots holding the layer's routed experts in seeded random slots
    (set-up only: the layer is routed once to know which experts to place)."""
    import time

    stacks = []
    ids = torch.empty(w.T, w.K, dtype=torch.int32, device=device)
    wts = torch.empty(w.T, w.K, dtype=torch.float32, device=device)
    lg = torch.empty(w.T, w.E, dtype=torch.float32, device=device)
    t0 = time.time()
    for layer in range(w.layers):
        xb = gen.activations_bf16(w.seed, layer, w.T, w.H)
        x = bf16_tensor(xb, device)
        wr = torch.from_numpy(gen.router_weight(w.seed, layer, w.E, w.H)).to(device)
        lib.moe_route(x, wr, lg, w.T, w.H, w.E, w.K, 0, ids, wts)
        routed = sorted(set(ids.cpu().numpy().ravel().tolist()))
        stacks.append(make_layer(w, layer, device, slots=w.slots, experts=routed, place_seed=1000 + layer, x_bits=xb))
        if log is not None and layer % 16 == 15:
            log(f"  decode: packed layers 0..{layer} ({time.time() - t0:.1f} s)")
    torch.cuda.synchronize(device)
    return stacks


class StackRunner:
    """One token through a stack of layers: one ``moe_layer`` call per layer, in order on
    one stream, each layer with its own logits, ids, w and y (the workspace is shared:
    the layers run one after another)."""

    def __init__(self, w: gen.Workload, layers: list[DeviceLayer], device, route_flags: int = 0):
        n = len(layers)
        self.w, self.layers, self.route_flags = w, layers, route_flags
        self.ids = torch.empty(n, w.T, w.K, dtype=torch.int32, device=device)
        self.wts = torch.empty(n, w.T, w.K, dtype=torch.float32, device=device)
        self.y = torch.empty(n, w.T, w.H, dtype=torch.bfloat16, device=device)
        self.ws_bytes = lib.moe_ffn_workspace_bytes(w.T, w.H, w.I, w.E, w.K, w.shared, 0)
        # zeroed: with MOE_ROUTE_ONEPASS the workspace holds hand-off words that start at zero
        self.ws = torch.zeros(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.graph = None

    def step(self, stream=None) -> None:
        w = self.w
        for i, L in enumerate(self.layers):
            lib.moe_layer(L.x, L.wr, L.logits, w.T, w.H, w.I, w.E, w.K, w.g, self.route_flags, self.ids[i],
                          self.wts[i], L.table, L.slots, L.stride, L.shared, self.y[i], self.ws, self.ws_bytes,
                          self.status, 0, stream)

    def poison(self) -> None:
        """Overwrite every output (y with bf16 NaN bits, ids with -1, w with NaN) and the
        logits the router writes, so that a run which does nothing cannot pass a check."""
        self.y.view(torch.int16).fill_(-1)
        self.ids.fill_(-1)
        self.wts.fill_(float("nan"))
        for L in self.layers:
            if L.wr is not None:
                L.logits.fill_(float("nan"))

    def capture(self, stream) -> None:
        """Record one step as a HIP graph on ``stream`` (the capture does not execute it)."""
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=stream):
            self.step(stream)

    def replay(self, stream) -> None:
        with torch.cuda.stream(stream):
            self.graph.replay()

    def outputs(self):
        """Host copies: (y bit patterns int16 [n, T, H], ids, w)."""
        return (self.y.view(torch.int16).cpu().numpy().copy(), self.ids.cpu().numpy().copy(),
                self.wts.cpu().numpy().copy())
