"""Seeded synthetic inputs for the int4 routed-expert MoE layer.

This package only draws inputs (activations, router weights, router logits,
int4 expert codes and fp16 group scales) in the plain interchange formats the
library and the CPU oracle both accept. It holds none of the layer's
arithmetic: no dot products, no selection, no dequantisation.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    activations_bf16,
    bf16_bits_from_f32,
    expert_tensors,
    locality_logits,
    normal_logits,
    router_weight,
    zipf_logits,
)
