"""Seeded synthetic inputs for the MoE routing-align + grouped expert FFN path.

This package only draws inputs: activations, router outputs (top-k ids and
weights) and quantised expert weights.  It holds none of the path's own
arithmetic (no alignment, no dequantisation, no FFN, no blend), so both the
oracle and the HIP path can take their inputs from it without sharing code.

Every array is a pure function of (config, purpose, expert), drawn from numpy
PCG64 streams keyed by ``[seed, purpose_tag, index]``, so any single expert's
weights can be regenerated alone.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    MoeConfig,
    bf16_bits_from_f32,
    expert_matrix,
    fill_expert_weights,
    router_weight_bf16,
    routing,
    shared_gate_bf16,
    shared_matrix,
    weight_shape,
    x_bf16,
)
