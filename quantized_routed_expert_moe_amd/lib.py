"""ctypes binding of ``libmoe.so`` (include/moe.h): argument marshalling only.

Every function keeps the C name and argument order. Device buffers may be
passed as torch tensors (their ``data_ptr()`` is used) or as integer addresses;
streams and events as ``torch.cuda.Stream`` / ``torch.cuda.Event`` or raw
handles. Each call raises ``MoeError`` on a negative status. Nothing here
computes any part of the layer, and a missing library is an error, never a
reason to compute elsewhere.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOSLOT, MOE_ENOTRES, MOE_EHIP, MOE_EUNSUP, MOE_EWS = 0, -1, -2, -3, -4, -5, -6
MOE_ROUTE_RENORM = 1 << 0
MOE_ROUTE_ONEPASS = 1 << 1
MOE_ROUTE_BITONIC = 4
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID, MOE_SCORE_SQRTSOFTPLUS = 0, 1, 2
MOE_FORCE_GEMV = 1 << 8
MOE_FORCE_GROUPED = 1 << 9
MOE_FMT_INT4_G32, MOE_FMT_INT4_G128, MOE_FMT_INT8_G32, MOE_FMT_NVFP4 = 0, 1, 2, 3
MOE_FFN_PARTIAL = 1 << 10
MOE_FFN_PARTIAL_SHARED = 1 << 11
MOE_FFN_PARTIAL_FIRST = 1 << 12

# every symbol include/moe.h declares
EXPORTS = (
    "moe_strerror",
    "moe_version",
    "moe_blob_bytes",
    "moe_slot_stride",
    "moe_pack_expert",
    "moe_route",
    "moe_route_scored",
    "moe_route_onepass_ws_bytes",
    "moe_route_onepass",
    "moe_ffn_workspace_bytes",
    "moe_expert_ffn",
    "moe_ffn_gate_up",
    "moe_ffn_down",
    "moe_layer",
    "moe_noalloc_scratch_bytes",
    "moe_layer_noalloc",
    "moe_ffn_combine",
    "moe_fmt_blob_bytes",
    "moe_fmt_slot_stride",
    "moe_pack_expert_fmt",
    "moe_pack_expert_nvfp4",
    "moe_fmt_workspace_bytes",
    "moe_expert_ffn_fmt",
    "arena_create",
    "arena_map_slots",
    "arena_fill_async",
    "arena_place",
    "arena_slot_table",
    "arena_reset",
    "arena_stats",
    "arena_destroy",
    "arena_chunk_passes",
    "arena_prefetch",
    "moe_paged_workspace_bytes",
    "moe_paged_layer",
)


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_strerror(status)} ({status})")


class moe_fill(ctypes.Structure):
    _fields_ = [("expert", ctypes.c_int32), ("slot", ctypes.c_int32)]


class moe_paged_layer_t(ctypes.Structure):
    _fields_ = [("arena", ctypes.c_void_p), ("w_router", ctypes.c_void_p), ("shared_blob", ctypes.c_void_p)]


MOE_PAGED_SPECULATE = 1
MOE_PAGED_HOST_POLL = 2


class moe_arena_stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64)
                for n in ("hits", "misses", "evictions", "fills", "h2d_bytes", "prefetch_fills", "prefetch_hits")]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t


def load(path: str | None = None):
    """Load libmoe.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(p)
    sig = {
        "moe_strerror": (ctypes.c_char_p, [_I]),
        "moe_version": (_I, []),
        "moe_blob_bytes": (_SZ, [_I, _I, _I]),
        "moe_slot_stride": (_SZ, [_I, _I, _I]),
        "moe_pack_expert": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P]),
        "moe_route": (_I, [_P, _P, _P, _I, _I, _I, _I, ctypes.c_uint, _P, _P, _P]),
        "moe_route_scored": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P, ctypes.c_float, ctypes.c_uint, _P, _P, _P]),
        "moe_route_onepass_ws_bytes": (_SZ, [_I, _I]),
        "moe_route_onepass": (_I, [_P, _P, _P, _I, _I, _I, ctypes.c_uint, _P, _P, _P, _SZ, _P, _P]),
        "moe_ffn_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, ctypes.c_uint]),
        "moe_expert_ffn": (
            _I,
            [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _SZ, _P, _P, _P, _SZ, _P, ctypes.c_uint, _P],
        ),
        "moe_ffn_gate_up": (
            _I,
            [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _SZ, _P, _P, _P, _SZ, _P, ctypes.c_uint, _P],
        ),
        "moe_ffn_down": (
            _I,
            [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _SZ, _P, _P, _P, _SZ, _P, ctypes.c_uint, _P],
        ),
        "moe_layer": (
            _I,
            [_P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_uint, _P, _P, _P, _P, _SZ, _P, _P, _P, _SZ, _P,
             ctypes.c_uint, _P],
        ),
        "moe_noalloc_scratch_bytes": (_SZ, []),
        "moe_layer_noalloc": (
            _I,
            [_P, _P, _P, _I, _I, _I, _I, _I, _I, ctypes.c_uint, _P, _P, _P, _P, _SZ, _P, _P, _P, ctypes.c_uint, _P],
        ),
        "moe_ffn_combine": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _SZ, _P, _P]),
        "moe_fmt_blob_bytes": (_SZ, [_I, _I, _I]),
        "moe_fmt_slot_stride": (_SZ, [_I, _I, _I]),
        "moe_pack_expert_fmt": (_I, [_I, _P, _P, _P, _P, _P, _P, _I, _I, _P]),
        "moe_pack_expert_nvfp4": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _P]),
        "moe_fmt_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
        "moe_expert_ffn_fmt": (
            _I,
            [_I, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _SZ, _P, _P, _P, _SZ, _P, _P],
        ),
        "arena_create": (_I, [_I, _I, _SZ, _SZ, _P, _P, _P, ctypes.POINTER(_P)]),
        "arena_map_slots": (_I, [_P, _P, _I, _P, _P, ctypes.POINTER(_I)]),
        "arena_fill_async": (_I, [_P, _P, _I, _P, _P]),
        "arena_place": (_I, [_P, _I, _I]),
        "arena_slot_table": (_I, [_P, _P]),
        "arena_reset": (_I, [_P]),
        "arena_stats": (_I, [_P, ctypes.POINTER(moe_arena_stats)]),
        "arena_destroy": (None, [_P]),
        "arena_chunk_passes": (_I, [_P, _P, _I, _I, _P, _P, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
        "arena_prefetch": (_I, [_P, _P, _I, _P, ctypes.POINTER(_I)]),
        "moe_paged_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
        "moe_paged_layer": (_I, [ctypes.POINTER(moe_paged_layer_t), ctypes.POINTER(moe_paged_layer_t), _P, _I, _P, _I,
                                 _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P, ctypes.c_uint, _P, _P, _P,
                                 ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _strerror(status: int) -> str:
    return load().moe_strerror(status).decode()


def _ptr(x) -> int | None:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if hasattr(x, "ctypes"):  # numpy array
        return x.ctypes.data
    return int(x)


def _stream(s) -> int | None:
    if s is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    return int(s)


def _event(e) -> int | None:
    if e is None:
        return None
    if hasattr(e, "cuda_event"):
        if not e.cuda_event:  # torch creates the HIP event on its first record
            raise ValueError("the event has no HIP event yet: record it once before passing it")
        return e.cuda_event
    return int(e)


def _check(status: int, what: str) -> int:
    if status < 0:
        raise MoeError(status, what)
    return status


def moe_version() -> int:
    return load().moe_version()


def moe_blob_bytes(H: int, I: int, g: int = 32) -> int:
    return load().moe_blob_bytes(H, I, g)


def moe_slot_stride(H: int, I: int, g: int = 32) -> int:
    return load().moe_slot_stride(H, I, g)


def moe_pack_expert(qg, qu, qd, sg, su, sd, H, I, g, blob_out) -> None:
    """Host arrays in the plain interchange format -> host blob (numpy uint8)."""
    _check(
        load().moe_pack_expert(_ptr(qg), _ptr(qu), _ptr(qd), _ptr(sg), _ptr(su), _ptr(sd), H, I, g, _ptr(blob_out)),
        "moe_pack_expert",
    )


def moe_pack_expert_fmt(fmt, qg, qu, qd, sg, su, sd, H, I, blob_out) -> None:
    """moe_pack_expert for format ``fmt`` (host numpy arrays)."""
    _check(
        load().moe_pack_expert_fmt(fmt, _ptr(qg), _ptr(qu), _ptr(qd), _ptr(sg), _ptr(su), _ptr(sd), H, I,
                                   _ptr(blob_out)),
        "moe_pack_expert_fmt",
    )


def moe_pack_expert_nvfp4(qg, qu, qd, sg, su, sd, global3, H, I, blob_out) -> None:
    _check(
        load().moe_pack_expert_nvfp4(_ptr(qg), _ptr(qu), _ptr(qd), _ptr(sg), _ptr(su), _ptr(sd), _ptr(global3), H, I,
                                     _ptr(blob_out)),
        "moe_pack_expert_nvfp4",
    )


def moe_route(x, w_router, logits, T, H, E, K, flags, ids, w, stream=None) -> None:
    _check(
        load().moe_route(_ptr(x), _ptr(w_router), _ptr(logits), T, H, E, K, flags, _ptr(ids), _ptr(w), _stream(stream)),
        "moe_route",
    )


def moe_route_scored(x, w_router, logits, T, H, E, K, score, bias, routed_scale, flags, ids, w, stream=None) -> None:
    _check(
        load().moe_route_scored(_ptr(x), _ptr(w_router), _ptr(logits), T, H, E, K, score, _ptr(bias),
                                float(routed_scale), flags, _ptr(ids), _ptr(w), _stream(stream)),
        "moe_route_scored",
    )


def moe_route_onepass_ws_bytes(E, K) -> int:
    return load().moe_route_onepass_ws_bytes(E, K)


def moe_route_onepass(x, w_router, logits, H, E, K, flags, ids, w, ws, ws_bytes, dev_status, stream=None) -> None:
    _check(
        load().moe_route_onepass(_ptr(x), _ptr(w_router), _ptr(logits), H, E, K, flags, _ptr(ids), _ptr(w), _ptr(ws),
                                 ws_bytes, _ptr(dev_status), _stream(stream)),
        "moe_route_onepass",
    )


def moe_ffn_workspace_bytes(T, H, I, E, K, has_shared, flags=0) -> int:
    return load().moe_ffn_workspace_bytes(T, H, I, E, K, int(bool(has_shared)), flags)


def _ffn_call(name, x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
              dev_status, flags, stream):
    _check(
        getattr(load(), name)(
            _ptr(x), _ptr(ids), _ptr(w), T, H, I, E, K, g, _ptr(slot_table), _ptr(slots), stride,
            _ptr(shared_blob), _ptr(y), _ptr(ws), ws_bytes, _ptr(dev_status), flags, _stream(stream),
        ),
        name,
    )


def moe_expert_ffn(x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
                   dev_status, flags=0, stream=None) -> None:
    _ffn_call("moe_expert_ffn", x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws,
              ws_bytes, dev_status, flags, stream)


def moe_ffn_gate_up(x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
                    dev_status, flags=0, stream=None) -> None:
    _ffn_call("moe_ffn_gate_up", x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws,
              ws_bytes, dev_status, flags, stream)


def moe_ffn_down(x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
                 dev_status, flags=0, stream=None) -> None:
    _ffn_call("moe_ffn_down", x, ids, w, T, H, I, E, K, g, slot_table, slots, stride, shared_blob, y, ws,
              ws_bytes, dev_status, flags, stream)


def moe_layer(x, w_router, logits, T, H, I, E, K, g, route_flags, ids, w, slot_table, slots, stride, shared_blob,
              y, ws, ws_bytes, dev_status, ffn_flags=0, stream=None) -> None:
    _check(
        load().moe_layer(
            _ptr(x), _ptr(w_router), _ptr(logits), T, H, I, E, K, g, route_flags, _ptr(ids), _ptr(w),
            _ptr(slot_table), _ptr(slots), stride, _ptr(shared_blob), _ptr(y), _ptr(ws), ws_bytes,
            _ptr(dev_status), ffn_flags, _stream(stream),
        ),
        "moe_layer",
    )


def moe_noalloc_scratch_bytes() -> int:
    return load().moe_noalloc_scratch_bytes()


def moe_layer_noalloc(x, w_router, logits, T, H, I, E, K, g, route_flags, ids, w, slot_table, slots, stride,
                      shared_blob, y, dev_status, ffn_flags=0, stream=None) -> None:
    _check(
        load().moe_layer_noalloc(
            _ptr(x), _ptr(w_router), _ptr(logits), T, H, I, E, K, g, route_flags, _ptr(ids), _ptr(w),
            _ptr(slot_table), _ptr(slots), stride, _ptr(shared_blob), _ptr(y), _ptr(dev_status), ffn_flags,
            _stream(stream),
        ),
        "moe_layer_noalloc",
    )


def moe_ffn_combine(ids, w, T, H, I, E, K, has_shared, y, ws, ws_bytes, dev_status, stream=None) -> None:
    _check(
        load().moe_ffn_combine(_ptr(ids), _ptr(w), T, H, I, E, K, int(bool(has_shared)), _ptr(y), _ptr(ws), ws_bytes,
                               _ptr(dev_status), _stream(stream)),
        "moe_ffn_combine",
    )


def moe_fmt_blob_bytes(fmt, H, I) -> int:
    return load().moe_fmt_blob_bytes(fmt, H, I)


def moe_fmt_slot_stride(fmt, H, I) -> int:
    return load().moe_fmt_slot_stride(fmt, H, I)


def moe_fmt_workspace_bytes(fmt, T, H, I, E, K, has_shared) -> int:
    return load().moe_fmt_workspace_bytes(fmt, T, H, I, E, K, int(bool(has_shared)))


def moe_expert_ffn_fmt(fmt, x, ids, w, T, H, I, E, K, slot_table, slots, stride, shared_blob, y, ws, ws_bytes,
                       dev_status, stream=None) -> None:
    _check(
        load().moe_expert_ffn_fmt(
            fmt, _ptr(x), _ptr(ids), _ptr(w), T, H, I, E, K, _ptr(slot_table), _ptr(slots), stride,
            _ptr(shared_blob), _ptr(y), _ptr(ws), ws_bytes, _ptr(dev_status), _stream(stream),
        ),
        "moe_expert_ffn_fmt",
    )


def moe_paged_workspace_bytes(H, I, E, K, has_shared) -> int:
    return load().moe_paged_workspace_bytes(H, I, E, K, int(bool(has_shared)))


def paged_layer_desc(arena, w_router, shared_blob=None) -> moe_paged_layer_t:
    return moe_paged_layer_t(arena.handle, _ptr(w_router), _ptr(shared_blob))


def moe_paged_layer(layer, next_layer, w_predict, P, x, H, I, E, K, g, logits, ids, w, ids_host, y, ws, ws_bytes,
                    dev_status, flags, stream, side, ids_ready):
    """layer, next_layer: moe_paged_layer_t (next_layer may be None). Returns (misses, prefetched)."""
    nm, npf = _I(0), _I(0)
    _check(
        load().moe_paged_layer(ctypes.byref(layer), ctypes.byref(next_layer) if next_layer is not None else None,
                               _ptr(w_predict), P, _ptr(x), H, I, E, K, g, _ptr(logits), _ptr(ids), _ptr(w),
                               _ptr(ids_host), _ptr(y), _ptr(ws), ws_bytes, _ptr(dev_status), flags, _stream(stream),
                               _stream(side), _event(ids_ready), ctypes.byref(nm), ctypes.byref(npf)),
        "moe_paged_layer",
    )
    return nm.value, npf.value


class Arena:
    """Owner of one ``moe_arena`` handle (the C object holds host metadata only)."""

    def __init__(self, E, S, blob_bytes, stride, slots_dev=None, slot_table_dev=None, host_src=None):
        h = _P()
        _check(
            load().arena_create(E, S, blob_bytes, stride, _ptr(slots_dev), _ptr(slot_table_dev), _ptr(host_src),
                                ctypes.byref(h)),
            "arena_create",
        )
        self.handle = h.value
        self.E, self.S = E, S
        # keep borrowed buffers alive as long as the arena
        self._keep = (slots_dev, slot_table_dev, host_src)

    def map_slots(self, ids):
        """ids: host int sequence -> (slots list, fills list of (expert, slot)); raises on MOE_ENOSLOT."""
        n = len(ids)
        arr = (ctypes.c_int32 * max(n, 1))(*[int(i) for i in ids])
        slots = (ctypes.c_int32 * max(n, 1))()
        fills = (moe_fill * max(n, 1))()
        nf = _I(0)
        _check(load().arena_map_slots(self.handle, arr, n, slots, fills, ctypes.byref(nf)), "arena_map_slots")
        self._last_fills = fills
        self._last_nf = nf.value
        return list(slots[:n]), [(fills[i].expert, fills[i].slot) for i in range(nf.value)]

    def map_slots_status(self, ids) -> int:
        """Like map_slots but returns the raw status instead of raising."""
        n = len(ids)
        arr = (ctypes.c_int32 * max(n, 1))(*[int(i) for i in ids])
        slots = (ctypes.c_int32 * max(n, 1))()
        fills = (moe_fill * max(n, 1))()
        nf = _I(0)
        return load().arena_map_slots(self.handle, arr, n, slots, fills, ctypes.byref(nf))

    def prefetch(self, ids):
        """Read-ahead of predicted ids (host int sequence) -> fills list of (expert, slot)."""
        n = len(ids)
        arr = (ctypes.c_int32 * max(n, 1))(*[int(i) for i in ids])
        fills = (moe_fill * max(n, 1))()
        nf = _I(0)
        _check(load().arena_prefetch(self.handle, arr, n, fills, ctypes.byref(nf)), "arena_prefetch")
        self._last_fills = fills
        self._last_nf = nf.value
        return [(fills[i].expert, fills[i].slot) for i in range(nf.value)]

    def prefetch_status(self, ids) -> int:
        """Like prefetch but returns the raw status instead of raising."""
        n = len(ids)
        arr = (ctypes.c_int32 * max(n, 1))(*[int(i) for i in ids])
        fills = (moe_fill * max(n, 1))()
        nf = _I(0)
        return load().arena_prefetch(self.handle, arr, n, fills, ctypes.byref(nf))

    def fill_async(self, side=None, done=None) -> None:
        """Enqueue the fills of the last map_slots or prefetch call on ``side``; record ``done``."""
        _check(
            load().arena_fill_async(self.handle, self._last_fills, self._last_nf, _stream(side), _event(done)),
            "arena_fill_async",
        )

    def chunk_passes(self, ids, max_per_pass):
        """ids: host int sequence -> list of passes, each a list of expert ids (arena_chunk_passes)."""
        n = len(ids)
        arr = (ctypes.c_int32 * max(n, 1))(*[int(i) for i in ids])
        experts = (ctypes.c_int32 * max(n, 1))()
        ends = (ctypes.c_int32 * max(n, 1))()
        nd, npass = _I(0), _I(0)
        _check(
            load().arena_chunk_passes(self.handle, arr, n, max_per_pass, experts, ends, ctypes.byref(nd),
                                      ctypes.byref(npass)),
            "arena_chunk_passes",
        )
        out, b = [], 0
        for p in range(npass.value):
            out.append(list(experts[b : ends[p]]))
            b = ends[p]
        return out

    def place(self, expert: int, slot: int) -> None:
        _check(load().arena_place(self.handle, expert, slot), "arena_place")

    def slot_table(self):
        out = (ctypes.c_int32 * self.E)()
        _check(load().arena_slot_table(self.handle, out), "arena_slot_table")
        return list(out)

    def reset(self) -> None:
        _check(load().arena_reset(self.handle), "arena_reset")

    def stats(self) -> dict:
        st = moe_arena_stats()
        _check(load().arena_stats(self.handle, ctypes.byref(st)), "arena_stats")
        return {n: getattr(st, n) for n, _ in moe_arena_stats._fields_}

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.arena_destroy(self.handle)
            self.handle = None
