"""CPU oracle for the int4 routed-expert MoE layer -- test infrastructure only.

A plain, slow, fp64 NumPy implementation of what the layer computes, written
from the definitions and sharing no code with the GPU library. Only the test
suite, the package smoke check and the benchmark's CPU-baseline leg may import
it; the product path never calls it.

Modules:

* ``moe_ref``   -- router logits, softmax top-k routing, int4 group dequant,
  SwiGLU expert FFN, routing-weighted combine;
* ``arena_ref`` -- an independent model of the fixed-slot expert arena's slot
  policy (least-recently-used with a deterministic tie rule).

Parity status per function is stated in each module's header.
"""

from . import arena_ref, moe_ref  # noqa: F401
