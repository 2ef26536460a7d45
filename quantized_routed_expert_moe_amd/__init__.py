"""int4 routed-expert MoE layer for MI355X (gfx950): HIP kernels behind a C ABI.

``lib`` is the ctypes binding of ``libmoe.so`` (include/moe.h); ``harness``
packs seeded experts into device arenas for tests and benchmarks.
"""

__all__ = ["lib", "harness"]
