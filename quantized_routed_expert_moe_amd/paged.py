"""Paged runs whose experts do not all fit in device memory: chunked prefill and read-ahead decode.

ChunkedPrefill: one MoE layer over a prompt whose chunks use more experts than the arena holds.

"Strata on a Mac", Measured (the UD-Q4/Q5/Q6_K_XL part): prompts stream in
chunks, and each chunk makes one pass over the experts it uses that are not in
the arena, so a longer chunk reads those experts fewer times. Per chunk, on one
compute stream and one side stream:

1. ``moe_route`` on the chunk, then the chosen ids to the host (the one
   hand-shake per chunk);
2. ``arena_chunk_passes``: the chunk's distinct experts, resident ones first,
   cut into passes of at most ``cap`` experts;
3. per pass: ``arena_map_slots`` on its experts, a pass slot table that maps
   exactly those experts (copied from pinned host memory), ``arena_fill_async``
   of the misses on the side stream, and one ``moe_expert_ffn`` pass with
   ``MOE_FFN_PARTIAL`` (the first pass, flagged ``MOE_FFN_PARTIAL_FIRST``, also
   computes the shared expert);
4. ``moe_ffn_combine`` writes the chunk's y, and flags in the status word any
   pair whose expert no pass computed.

With ``cap <= S / 2`` the fills of pass p + 1 evict nothing pass p reads, so
they wait only for pass p - 1 and overlap pass p's compute; with a larger cap
they wait for pass p. The outputs are bit-identical to the fully-resident
grouped run of the same chunk.

PagedDecode: single-token decode through a stack of layers, each with its own
arena, with read-ahead ("Strata on a Mac", What you need: the experts the next
layer will probably use are read ahead). Per layer l:

1. ``moe_route`` of x_l with layer l's router; with read-ahead, also the top-P
   of layer l + 1's router on the same x_l (the prediction: a residual stream
   changes little from one layer to the next);
2. the ids (and the prediction) to the host, the one hand-shake per layer;
3. ``arena_map_slots`` and ``arena_fill_async`` of the misses on the side
   stream, recording this layer's event;
4. ``arena_prefetch`` of the prediction into layer l + 1's arena and its fills
   on the side stream, after this layer's (so they never delay them);
5. the compute stream waits on the event, then ``moe_expert_ffn``.

The hand-shake has drained every earlier compute launch, so no GPU work still
reads a slot that the map or the prefetch may evict. Layer l + 1's event is
recorded after its prefetched copies on the same side stream, so its FFN never
reads a slot before its bytes have landed. A prediction only moves copies
earlier: every output equals the run without read-ahead, bit for bit ("Strata"
README: a predictor never changes what is computed).

With ``native=True`` (the default) each layer is one ``moe_paged_layer`` call,
which runs the same steps in the library's C++ and, with ``speculate``, starts
the FFN before the hand-shake and runs it again only when the layer missed.
This module only sequences library calls.
"""

from __future__ import annotations

import torch

from . import lib


class ChunkedPrefill:
    """Runs chunks of up to ``max_T`` tokens of one layer through a paged arena.

    ``arena``: a ``lib.Arena`` with device slots, its device slot table and the
    pinned expert-major host copy. ``slots``: the arena's device slot buffer.
    ``shared``: device blob of the shared expert, or None.
    """

    def __init__(self, arena: lib.Arena, slots: torch.Tensor, stride: int, H: int, I: int, E: int, K: int,
                 max_T: int, cap: int, shared: torch.Tensor | None = None, g: int = 32, device="cuda"):
        if not 1 <= cap <= arena.S:
            raise ValueError("cap must be in [1, S]")
        self.arena, self.slots, self.stride = arena, slots, stride
        self.H, self.I, self.E, self.K, self.g = H, I, E, K, g
        self.max_T, self.cap, self.shared = max_T, cap, shared
        self.ids = torch.empty(max_T, K, dtype=torch.int32, device=device)
        self.wts = torch.empty(max_T, K, dtype=torch.float32, device=device)
        self.ids_h = torch.empty(max_T * K, dtype=torch.int32, pin_memory=True)
        self.ws_bytes = lib.moe_ffn_workspace_bytes(max_T, H, I, E, K, shared is not None, lib.MOE_FFN_PARTIAL)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.max_passes = (E + cap - 1) // cap
        self.table_h = torch.full((self.max_passes, E), -1, dtype=torch.int32, pin_memory=True)
        self.table_d = torch.full((self.max_passes, E), -1, dtype=torch.int32, device=device)
        self.side = torch.cuda.Stream(device=device)
        self.filled = [torch.cuda.Event() for _ in range(self.max_passes)]
        self.computed = [torch.cuda.Event() for _ in range(self.max_passes)]
        for e in self.filled + self.computed:
            e.record(self.side)  # creates the HIP events
        torch.cuda.synchronize(device)
        self.last_passes: list[list[int]] = []

    def run_chunk(self, x: torch.Tensor, logits: torch.Tensor, y: torch.Tensor, w_router=None) -> None:
        """x bf16 [T, H], logits fp32 [T, E] (written when ``w_router`` is given), y bf16 [T, H] out."""
        T = x.shape[0]
        if T > self.max_T:
            raise ValueError("chunk longer than max_T")
        if T == 0:
            return
        H, I, E, K, g = self.H, self.I, self.E, self.K, self.g
        comp = torch.cuda.current_stream()
        ids, wts = self.ids[:T], self.wts[:T]
        lib.moe_route(x if w_router is not None else None, w_router, logits, T, H, E, K, 0, ids, wts, comp)
        self.ids_h[: T * K].copy_(ids.view(-1), non_blocking=True)
        comp.synchronize()  # the hand-shake; also: no earlier work still reads the slots or the tables
        passes = self.arena.chunk_passes(self.ids_h[: T * K].tolist(), self.cap)
        self.last_passes = passes
        overlap = 2 * self.cap <= self.arena.S
        for p, experts in enumerate(passes):
            slots_of, _ = self.arena.map_slots(experts)
            row = self.table_h[p]
            row.fill_(-1)
            row[torch.tensor(experts, dtype=torch.long)] = torch.tensor(slots_of, dtype=torch.int32)
            self.table_d[p].copy_(row, non_blocking=True)  # on comp, before this pass's FFN
            wait = p - 2 if overlap else p - 1
            if wait >= 0:
                self.side.wait_event(self.computed[wait])
            self.arena.fill_async(self.side, self.filled[p])
            comp.wait_event(self.filled[p])
            flags = lib.MOE_FFN_PARTIAL | (lib.MOE_FFN_PARTIAL_FIRST if p == 0 else 0)
            flags |= lib.MOE_FFN_PARTIAL_SHARED if p == 0 and self.shared is not None else 0
            lib.moe_expert_ffn(x, ids, wts, T, H, I, E, K, g, self.table_d[p], self.slots, self.stride, self.shared,
                               y, self.ws, self.ws_bytes, self.status, flags, comp)
            self.computed[p].record(comp)
        lib.moe_ffn_combine(ids, wts, T, H, I, E, K, self.shared is not None, y, self.ws, self.ws_bytes, self.status,
                            comp)

    def run_prompt(self, x: torch.Tensor, logits: torch.Tensor, y: torch.Tensor, chunk: int, w_router=None) -> None:
        """The whole prompt in chunks of ``chunk`` tokens (the last one ragged)."""
        if not 1 <= chunk <= self.max_T:
            raise ValueError("chunk must be in [1, max_T]")
        for t0 in range(0, x.shape[0], chunk):
            t1 = min(t0 + chunk, x.shape[0])
            self.run_chunk(x[t0:t1], logits[t0:t1], y[t0:t1], w_router)


class PagedDecode:
    """Single-token decode through per-layer arenas, optionally reading the next layer ahead.

    ``layers``: per layer ``(arena, slots, table)`` (a ``lib.Arena``, its device
    slot buffer and device slot table). ``routers``: per layer, device fp32
    ``[E, H]``, or None when the caller passes the layer's logits to ``layer``.
    ``shared``: per layer a device blob of the shared expert, or None.
    ``predict``: experts read ahead per layer (0: none). ``predictors``: per layer,
    the device fp32 ``[E, H]`` matrix applied to the previous layer's input to
    predict this layer's experts (default: the layer's own router). ``native``:
    one ``moe_paged_layer`` call per layer (else the same steps from Python);
    ``speculate``: with ``native``, the FFN starts before the hand-shake;
    ``host_poll``: with ``native``, the ids reach the host through a polled word in
    pinned memory rather than a copy and an event.
    """

    def __init__(self, layers, routers, stride: int, H: int, I: int, E: int, K: int, shared=None,
                 predict: int = 0, g: int = 32, device="cuda", predictors=None, native: bool = True,
                 speculate: bool = True, host_poll: bool = True):
        if len(routers) != len(layers) or (predictors is not None and len(predictors) != len(layers)):
            raise ValueError("one router (and one predictor) per layer")
        if not 0 <= predict <= min([E] + [a.S for a, _, _ in layers]):
            raise ValueError("predict must be in [0, min(E, S)]")
        self.layers, self.routers, self.stride = layers, routers, stride
        self.predictors = predictors if predictors is not None else routers
        if predict and any(p is None for p in self.predictors[1:]):
            raise ValueError("read-ahead needs a predictor for every layer after the first")
        self.H, self.I, self.E, self.K, self.g, self.predict = H, I, E, K, g, predict
        self.shared = shared if shared is not None else [None] * len(layers)
        self.logits = torch.empty(1, E, dtype=torch.float32, device=device)
        self.ids = torch.empty(1, K, dtype=torch.int32, device=device)
        self.wts = torch.empty(1, K, dtype=torch.float32, device=device)
        P = max(predict, 1)
        self.p_logits = torch.empty(1, E, dtype=torch.float32, device=device)
        self.p_ids = torch.empty(1, P, dtype=torch.int32, device=device)
        self.p_wts = torch.empty(1, P, dtype=torch.float32, device=device)
        self.ids_h = torch.zeros(K + P + 1, dtype=torch.int32, pin_memory=True)  # + the polled word
        has_shared = any(b is not None for b in self.shared)
        self.ws_bytes = lib.moe_ffn_workspace_bytes(1, H, I, E, K, has_shared)
        self.native, self.speculate, self.host_poll = native, speculate, host_poll
        if native:
            self.ws_bytes = lib.moe_paged_workspace_bytes(H, I, E, K, has_shared)
            self.nat_ids = torch.empty(K + P, dtype=torch.int32, device=device)
            self.nat_w = torch.empty(K + P, dtype=torch.float32, device=device)
            self.descs = [lib.paged_layer_desc(a, r, b) for (a, _, _), r, b in zip(layers, routers, self.shared)]
            self.ids_ready = torch.cuda.Event()
            self.ids_ready.record()  # creates the HIP event
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.side = torch.cuda.Stream(device=device)
        self.done = torch.cuda.Event()
        self.done.record(self.side)  # creates the HIP event
        torch.cuda.synchronize(device)
        self.log: list | None = None  # (op, layer, ids) of every arena call when a list

    def layer(self, l: int, x: torch.Tensor, y: torch.Tensor, logits: torch.Tensor | None = None) -> None:
        """x bf16 [1, H]: layer l's input; y bf16 [1, H] out; logits fp32 [E]: layer l's
        logits when it has no router (the native path with read-ahead then reuses that
        buffer for the prediction's logits)."""
        if (logits is None) != (self.routers[l] is not None):
            raise ValueError("pass logits exactly when the layer has no router")
        lg = self.logits if logits is None else logits.view(1, -1)
        if self.native:
            self._layer_native(l, x, y, lg)
            return
        H, E, K, P = self.H, self.E, self.K, self.predict
        comp = torch.cuda.current_stream()
        arena, slots, table = self.layers[l]
        router = self.routers[l]
        lib.moe_route(x if router is not None else None, router, lg, 1, H, E, K, 0, self.ids, self.wts, comp)
        self.ids_h[:K].copy_(self.ids.view(-1), non_blocking=True)
        ahead = P > 0 and l + 1 < len(self.layers)
        if ahead:
            lib.moe_route(x, self.predictors[l + 1], self.p_logits, 1, H, E, P, 0, self.p_ids, self.p_wts, comp)
            self.ids_h[K : K + P].copy_(self.p_ids.view(-1), non_blocking=True)
        comp.synchronize()  # the hand-shake; no earlier launch still reads any arena
        ids = self.ids_h[:K].tolist()
        arena.map_slots(ids)
        arena.fill_async(self.side, self.done)
        if self.log is not None:
            self.log.append(("map", l, ids))
        if ahead:
            pred = self.ids_h[K : K + P].tolist()
            self.layers[l + 1][0].prefetch(pred)
            self.layers[l + 1][0].fill_async(self.side, None)
            if self.log is not None:
                self.log.append(("pre", l + 1, pred))
        comp.wait_event(self.done)
        lib.moe_expert_ffn(x, self.ids, self.wts, 1, H, self.I, E, K, self.g, table, slots, self.stride,
                           self.shared[l], y, self.ws, self.ws_bytes, self.status, 0, comp)

    def _layer_native(self, l: int, x: torch.Tensor, y: torch.Tensor, lg: torch.Tensor) -> None:
        K, P = self.K, self.predict
        ahead = P > 0 and l + 1 < len(self.layers)
        lib.moe_paged_layer(self.descs[l], self.descs[l + 1] if ahead else None,
                            self.predictors[l + 1] if ahead else None, P if ahead else 0, x, self.H, self.I, self.E,
                            K, self.g, lg, self.nat_ids, self.nat_w, self.ids_h, y, self.ws, self.ws_bytes,
                            self.status, (lib.MOE_PAGED_SPECULATE if self.speculate else 0)
                            | (lib.MOE_PAGED_HOST_POLL if self.host_poll else 0),
                            torch.cuda.current_stream(), self.side, self.ids_ready)
        if self.log is not None:
            self.log.append(("map", l, self.ids_h[:K].tolist()))
            if ahead:
                self.log.append(("pre", l + 1, self.ids_h[K : K + P].tolist()))

    @property
    def routed(self):
        """The last layer's ids and weights on the device ([1, K] each)."""
        if self.native:
            return self.nat_ids[: self.K].view(1, -1), self.nat_w[: self.K].view(1, -1)
        return self.ids, self.wts

    def token(self, xs, ys, logits=None) -> None:
        """One token through every layer: xs[l] the inputs, ys[l] the outputs (logits[l]
        the logits of the layers without a router)."""
        for l in range(len(self.layers)):
            self.layer(l, xs[l], ys[l], None if logits is None else logits[l])

