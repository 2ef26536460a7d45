"""Build the HIP library ``libmoe.so`` in-tree with hipcc for gfx950, and its
instrumented twin ``libmoe_timeline.so`` (the same sources with MOE_TIMELINE:
per-workgroup stamps, include/moe_timeline.h)."""

from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe.so")
TIMELINE_LIB = os.path.join(PKG, "libmoe_timeline.so")

SOURCES = ["api.cpp", "pack.cpp", "arena.cpp", "paged.cpp", "route.hip", "ffn_gemv.hip", "ffn_batched.hip", "ffn_decode.hip",
           "ffn_grouped.hip", "ffn_formats.hip", "scratch.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    f"--offload-arch={ARCH}",
    # keep hipcc from forming packed-fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, jobs: int = 8, timeline: bool = False) -> str:
    """Compile every source to an object (in parallel) and link libmoe.so (timeline:
    libmoe_timeline.so); returns its path."""
    objdir = os.path.join(PKG, "_build_timeline" if timeline else "_build")
    lib = TIMELINE_LIB if timeline else LIB
    os.makedirs(objdir, exist_ok=True)
    cc = hipcc()
    procs, objs = [], []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        objs.append(obj)
        cmd = [cc, *HIPCC_FLAGS, *(["-DMOE_TIMELINE"] if timeline else []), "-I", INCLUDE, "-I", CSRC]
        cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        if len([p for p in procs if p[1].poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if out.strip() and (verbose or p.returncode):
            print(out, file=sys.stderr)
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, timeline="--timeline" in sys.argv))
