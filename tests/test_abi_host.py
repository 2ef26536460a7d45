"""Host-side checks of the C-ABI library (CPU only, no GPU compute calls).

* libmoe.so loads and exports every function include/moe.h declares, and its
  instrumented twin libmoe_timeline.so also those of include/moe_timeline.h;
* moe_pack_expert writes the documented blob layout (decoded here by an
  independent reader of that layout and compared with the interchange input);
* the arena's slot policy in C++ replays the reference model's slot, fill,
  eviction and statistics sequences exactly, including failure cases.
"""

import os
import re

import numpy as np
import pytest

from oracle.arena_ref import ArenaModel
from quantized_routed_expert_moe_amd import lib
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b((?:moe|arena)_\w+)\s*\(", src))


def test_library_exports_every_declared_function():
    L = lib.load()
    names = header_functions()
    assert names == set(lib.EXPORTS), names ^ set(lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_timeline_build_exports_its_functions_and_the_product_does_not():
    """libmoe_timeline.so (the instrumented twin) exports what include/moe.h and
    include/moe_timeline.h declare; libmoe.so exports nothing of the timeline."""
    import ctypes

    from quantized_routed_expert_moe_amd import build

    src = open(os.path.join(ROOT, "include", "moe_timeline.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    tl_names = set(re.findall(r"\b(moe_timeline_\w+)\s*\(", src))
    assert tl_names == {"moe_timeline_read", "moe_timeline_clear"}
    T = ctypes.CDLL(build.TIMELINE_LIB)
    for n in tl_names | header_functions():
        assert hasattr(T, n), n
    P = lib.load()
    for n in tl_names:
        assert not hasattr(P, n), n


def test_strerror_and_sizes():
    assert lib.load().moe_strerror(lib.MOE_ENOSLOT).decode().startswith("no free slot")
    assert lib.moe_version() >= 100
    # 3 matrices of H*I int4 codes (1/2 byte) + one fp16 scale per 32 codes
    for H, I, want in ((256, 512, 221184), (4096, 1536, 10616832), (2048, 768, 2654208), (4096, 2048, 14155776)):
        assert lib.moe_blob_bytes(H, I, 32) == want
        assert lib.moe_slot_stride(H, I, 32) % 4096 == 0 and lib.moe_slot_stride(H, I, 32) >= want
    assert lib.moe_blob_bytes(4096, 1536, 64) == 0  # only g = 32
    assert lib.moe_blob_bytes(4000 + 16, 1536, 32) == 0  # H not a multiple of 32


def decode_blob_matrix(blob, off_codes, off_scales, N, C, R):
    """Independent reader of the documented blob layout (blocks of R rows) ->
    (codes int [N][C], scales f16 [N][C/32])."""
    G = C // 32
    # [N/R][G][R rows][4 dwords] -> [G][N][4]
    codes = np.frombuffer(blob, dtype=np.uint32, count=G * N * 4, offset=off_codes).reshape(N // R, G, R, 4)
    codes = codes.transpose(1, 0, 2, 3).reshape(G, N, 4)
    q = np.empty((N, C), dtype=np.int64)
    for d in range(4):
        w = codes[:, :, d]  # [G][N]
        for i in range(8):
            col = 8 * d + (2 * i if i < 4 else 2 * (i - 4) + 1)
            u = (w >> (4 * i)) & 0xF
            q[:, col::32] = (u.astype(np.int64) - 8).T
    sc = np.frombuffer(blob, dtype=np.float16, count=N * G, offset=off_scales).reshape(N // R, G, R)
    s = sc.transpose(0, 2, 1).reshape(N, G)
    return q, s


def unpack_plain(packed, C):
    lo = (packed & 0xF).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    out = np.empty(packed.shape[:-1] + (C,), dtype=np.int64)
    out[..., 0::2] = np.where(lo >= 8, lo - 16, lo)
    out[..., 1::2] = np.where(hi >= 8, hi - 16, hi)
    return out


@pytest.mark.parametrize("H,I", [(256, 512), (2048, 768)])
def test_pack_layout_roundtrip(H, I):
    t = gen.expert_tensors(9, 0, 3, H, I)
    blob = np.zeros(lib.moe_slot_stride(H, I), dtype=np.uint8)
    lib.moe_pack_expert(t["qg"], t["qu"], t["qd"], t["sg"].view(np.uint16), t["su"].view(np.uint16),
                        t["sd"].view(np.uint16), H, I, 32, blob)
    mc, ms = H * I // 2, H * I // 16
    # gate and up in blocks of 8 rows, down in blocks of 4
    offs = [(0, 3 * mc, I, H, 8, "qg", "sg"), (mc, 3 * mc + ms, I, H, 8, "qu", "su"),
            (2 * mc, 3 * mc + 2 * ms, H, I, 4, "qd", "sd")]
    for oc, os_, N, C, R, qk, sk in offs:
        q, s = decode_blob_matrix(blob.tobytes(), oc, os_, N, C, R)
        assert np.array_equal(q, unpack_plain(t[qk], C))
        assert np.array_equal(s.view(np.uint16), t[sk].view(np.uint16))
    assert not blob[3 * mc + 3 * ms :].any()  # padding stays zero


def test_pack_rejects_bad_args():
    z = np.zeros(16, np.uint8)
    with pytest.raises(lib.MoeError):
        lib.moe_pack_expert(z, z, z, z, z, z, 4096, 1536, 64, z)


def run_both(E, S, stream, blob=100):
    a = lib.Arena(E, S, blob, 4096)  # bookkeeping only: no device buffers
    m = ArenaModel(E, S, blob)
    for ids in stream:
        st_m, slots_m, fills_m = m.map_slots(ids)
        st_c = a.map_slots_status(ids) if st_m != 0 else 0
        if st_m != 0:
            assert st_c == st_m, ids
            continue
        slots_c, fills_c = a.map_slots(ids)
        assert slots_c == slots_m, ids
        assert fills_c == fills_m, ids
        assert a.slot_table() == m.slot_of
    assert a.stats() == m.stats
    return a, m


def test_arena_cpp_matches_model_random_streams():
    rng = np.random.default_rng(1)
    for E, S, n in ((16, 4, 4), (256, 64, 8), (8, 8, 8), (40, 6, 7)):
        stream = [rng.integers(0, E, size=int(rng.integers(1, n + 1))).tolist() for _ in range(400)]
        stream += [[E], [-1, 0]]  # invalid ids
        run_both(E, S, stream)


def test_arena_cpp_locality_stream():
    # single-token decode with temporal locality, one arena per layer, budget = top-k
    lg = gen.locality_logits(5, 2, 64, 256, 6)
    for S in (6, 64):
        for layer in range(2):
            stream = [np.argsort(-lg[s, layer], kind="stable")[:6].tolist() for s in range(64)]
            run_both(256, S, stream)


def test_arena_cpp_prefetch_matches_model():
    """arena_prefetch interleaved with arena_map_slots: the same fills, slots, statuses and
    stats as the model, on random streams and on a next-layer prediction stream."""
    rng = np.random.default_rng(6)
    for E, S, n in ((16, 4, 4), (256, 64, 8), (8, 8, 8), (40, 6, 7)):
        a = lib.Arena(E, S, 100, 4096)
        m = ArenaModel(E, S, 100)
        for i in range(500):
            ids = rng.integers(0, E, size=int(rng.integers(1, n + 1))).tolist()
            if i % 97 == 5:
                ids = ids + [E if i % 2 else -1]  # invalid id
            if rng.random() < 0.5:
                st_m, fills_m = m.prefetch(ids)
                if st_m != 0:
                    assert a.prefetch_status(ids) == st_m, ids
                    continue
                assert a.prefetch(ids) == fills_m, ids
            else:
                st_m, slots_m, fills_m = m.map_slots(ids)
                if st_m != 0:
                    assert a.map_slots_status(ids) == st_m, ids
                    continue
                assert a.map_slots(ids) == (slots_m, fills_m), ids
            assert a.slot_table() == m.slot_of
        assert a.stats() == m.stats
    # the read-ahead decode pattern: demand at one layer, prediction for the next
    lg = gen.locality_logits(5, 3, 48, 256, 6)
    arenas = [(lib.Arena(256, 64, 100, 4096), ArenaModel(256, 64, 100)) for _ in range(3)]
    for s in range(48):
        for layer in range(3):
            ids = np.argsort(-lg[s, layer], kind="stable")[:6].tolist()
            a, m = arenas[layer]
            assert a.map_slots(ids) == m.map_slots(ids)[1:]
            if layer + 1 < 3 and s + 1 < 48:
                pred = np.argsort(-lg[s + 1, layer + 1], kind="stable")[:6].tolist()
                a, m = arenas[layer + 1]
                assert a.prefetch(pred) == m.prefetch(pred)[1]
    for a, m in arenas:
        assert a.stats() == m.stats and a.slot_table() == m.slot_of


def test_arena_place_reset_and_errors():
    a = lib.Arena(10, 4, 100, 4096)
    a.place(7, 2)
    assert a.map_slots([3, 7, 5]) == ([0, 2, 1], [(3, 0), (5, 1)])
    a.place(3, 3)
    assert a.slot_table()[3] == 3 and a.slot_table()[7] == 2
    assert a.map_slots_status([0, 1, 2, 3, 4]) == lib.MOE_ENOSLOT
    with pytest.raises(lib.MoeError):
        a.place(10, 0)
    with pytest.raises(lib.MoeError):
        a.fill_async(side=0)  # bookkeeping-only arena cannot fill
    a.reset()
    assert a.slot_table() == [-1] * 10 and a.stats()["hits"] == 0


def test_arena_cpp_chunk_passes_matches_model():
    rng = np.random.default_rng(4)
    for E, S, T, K in ((64, 16, 40, 4), (256, 64, 200, 6), (32, 6, 9, 3)):
        a = lib.Arena(E, S, 100, 4096)
        m = ArenaModel(E, S, 100)
        for chunk in range(5):
            ids = rng.integers(0, E, size=T * K).tolist()
            for cap in (1, S // 2, S):
                st, passes = m.chunk_passes(ids, cap)
                assert st == 0
                assert a.chunk_passes(ids, cap) == passes
            for p in m.chunk_passes(ids, S // 2)[1]:
                assert a.map_slots(p) == m.map_slots(p)[1:]
        with pytest.raises(lib.MoeError):
            a.chunk_passes([0, E], 2)
        with pytest.raises(lib.MoeError):
            a.chunk_passes([0], S + 1)
        assert a.chunk_passes([], 1) == []


def al256(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("H,I", [(512, 256), (4096, 1536)])
def test_fmt_int4_g128_is_the_g32_blob_with_repeated_scales(H, I):
    t = gen.expert_tensors_fmt(9, 0, 3, H, I, gen.FMT_INT4_G128)
    assert lib.moe_fmt_blob_bytes(gen.FMT_INT4_G128, H, I) == lib.moe_blob_bytes(H, I, 32)
    blob = np.zeros(lib.moe_fmt_slot_stride(gen.FMT_INT4_G128, H, I), dtype=np.uint8)
    lib.moe_pack_expert_fmt(gen.FMT_INT4_G128, t["qg"], t["qu"], t["qd"], t["sg"].view(np.uint16),
                            t["su"].view(np.uint16), t["sd"].view(np.uint16), H, I, blob)
    mc, ms = H * I // 2, H * I // 16
    offs = [(0, 3 * mc, I, H, 8, "qg", "sg"), (mc, 3 * mc + ms, I, H, 8, "qu", "su"),
            (2 * mc, 3 * mc + 2 * ms, H, I, 4, "qd", "sd")]
    for oc, os_, N, C, R, qk, sk in offs:
        q, s = decode_blob_matrix(blob.tobytes(), oc, os_, N, C, R)
        assert np.array_equal(q, unpack_plain(t[qk], C))
        assert np.array_equal(s.view(np.uint16), np.repeat(t[sk].view(np.uint16), 4, axis=1))


@pytest.mark.parametrize("fmt,H,I", [(gen.FMT_INT8_G32, 256, 96), (gen.FMT_INT8_G32, 4096, 1536)])
def test_fmt_pack_layout_roundtrip(fmt, H, I):
    """The int8 blobs decode back to the interchange codes and scales (an independent
    reader of the documented row-major layout)."""
    bits, g = gen.FMT_BITS_G[fmt]
    t = gen.expert_tensors_fmt(9, 0, 3, H, I, fmt)
    nb = lib.moe_fmt_blob_bytes(fmt, H, I)
    cb_gu, cb_dn = I * H * bits // 8, H * I * bits // 8
    sb_gu, sb_dn = I * (H // g) * 2, H * (I // g) * 2
    offs = [0]
    for size in (cb_gu, cb_gu, cb_dn, sb_gu, sb_gu, sb_dn):
        offs.append(al256(offs[-1] + size))
    assert nb == offs[-1]
    assert lib.moe_fmt_slot_stride(fmt, H, I) == (nb + 4095) // 4096 * 4096
    blob = np.zeros(lib.moe_fmt_slot_stride(fmt, H, I), dtype=np.uint8)
    lib.moe_pack_expert_fmt(fmt, t["qg"], t["qu"], t["qd"], t["sg"].view(np.uint16), t["su"].view(np.uint16),
                            t["sd"].view(np.uint16), H, I, blob)
    mats = [("qg", "sg", I, H, offs[0], offs[3]), ("qu", "su", I, H, offs[1], offs[4]),
            ("qd", "sd", H, I, offs[2], offs[5])]
    for qk, sk, N, C, oc, os_ in mats:
        u = blob[oc : oc + N * C].reshape(N, C).astype(np.int64)
        assert np.array_equal(u - 128, t[qk].view(np.int8).astype(np.int64))
        s = np.frombuffer(blob.tobytes(), dtype=np.uint16, count=N * (C // g), offset=os_).reshape(N, C // g)
        assert np.array_equal(s, t[sk].view(np.uint16))


def test_fmt_sizes_and_rejections():
    assert lib.moe_fmt_blob_bytes(gen.FMT_INT4_G32, 4096, 1536) == lib.moe_blob_bytes(4096, 1536, 32)
    assert lib.moe_fmt_slot_stride(gen.FMT_INT4_G32, 4096, 1536) == lib.moe_slot_stride(4096, 1536, 32)
    assert lib.moe_fmt_blob_bytes(gen.FMT_INT4_G128, 4096, 1600) == 0  # I not a multiple of 128
    assert lib.moe_fmt_blob_bytes(gen.FMT_INT8_G32, 8192, 1536) == 0  # int8 rows past 4096 columns
    assert lib.moe_fmt_blob_bytes(7, 4096, 1536) == 0
    # T > 32: the grouped (prompt) workspace, for H and I multiples of 64 only
    assert lib.moe_fmt_workspace_bytes(gen.FMT_INT8_G32, 33, 4096, 1536, 256, 8, 1) == lib.moe_ffn_workspace_bytes(
        33, 4096, 1536, 256, 8, 1, lib.MOE_FORCE_GROUPED)
    assert lib.moe_fmt_workspace_bytes(gen.FMT_NVFP4, 33, 4096, 1504, 256, 8, 1) == 0
    z = np.zeros(16, np.uint8)
    with pytest.raises(lib.MoeError):
        lib.moe_pack_expert_fmt(7, z, z, z, z, z, z, 256, 96, z)
    with pytest.raises(lib.MoeError):
        lib.moe_pack_expert_fmt(gen.FMT_INT4_G128, z, z, z, z, z, z, 256, 96, z)


@pytest.mark.parametrize("H,I", [(256, 96), (4096, 1536)])
def test_nvfp4_pack_layout_roundtrip(H, I):
    t = gen.expert_tensors_fmt(9, 0, 3, H, I, gen.FMT_NVFP4)
    nb = lib.moe_fmt_blob_bytes(gen.FMT_NVFP4, H, I)
    offs = [0]
    for size in (I * H // 2, I * H // 2, H * I // 2, I * H // 16, I * H // 16, H * I // 16, 12):
        offs.append(al256(offs[-1] + size))
    assert nb == offs[-1]
    blob = np.zeros(lib.moe_fmt_slot_stride(gen.FMT_NVFP4, H, I), dtype=np.uint8)
    lib.moe_pack_expert_nvfp4(t["qg"], t["qu"], t["qd"], t["sg"], t["su"], t["sd"], t["global"], H, I, blob)
    for i, (k, n) in enumerate((("qg", I * H // 2), ("qu", I * H // 2), ("qd", H * I // 2), ("sg", I * H // 16),
                                ("su", I * H // 16), ("sd", H * I // 16))):
        assert np.array_equal(blob[offs[i] : offs[i] + n], t[k].ravel())
    assert np.array_equal(blob[offs[6] : offs[6] + 12].view(np.float32), t["global"])


def test_nvfp4_pack_rejections():
    H, I = 256, 96
    t = gen.expert_tensors_fmt(9, 0, 3, H, I, gen.FMT_NVFP4)
    blob = np.zeros(lib.moe_fmt_slot_stride(gen.FMT_NVFP4, H, I), dtype=np.uint8)
    bad = t["sd"].copy()
    bad[3, 2] = 0xFF  # the E4M3 NaN
    with pytest.raises(lib.MoeError):
        lib.moe_pack_expert_nvfp4(t["qg"], t["qu"], t["qd"], t["sg"], t["su"], bad, t["global"], H, I, blob)
    g = t["global"].copy()
    g[1] = np.inf
    with pytest.raises(lib.MoeError):
        lib.moe_pack_expert_nvfp4(t["qg"], t["qu"], t["qd"], t["sg"], t["su"], t["sd"], g, H, I, blob)
    with pytest.raises(lib.MoeError):  # H not a multiple of 32
        lib.moe_pack_expert_nvfp4(t["qg"], t["qu"], t["qd"], t["sg"], t["su"], t["sd"], t["global"], 240, I, blob)
    assert lib.moe_fmt_blob_bytes(gen.FMT_NVFP4, 16384, 1536) == 0


def test_missing_library_is_an_error():
    """Without the built library nothing computes: loading fails with ImportError (checked in a
    fresh process, since this one has the library loaded)."""
    import subprocess
    import sys

    code = ("import quantized_routed_expert_moe_amd.lib as L\n"
            "L.LIB_PATH = '/nonexistent/libmoe.so'\n"
            "try:\n    L.load()\nexcept ImportError as e:\n    print('ImportError', e)\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                         cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert out.returncode == 0 and out.stdout.startswith("ImportError"), (out.stdout, out.stderr)
