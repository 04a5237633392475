"""Seeded synthetic MoE-layer inputs.

This package only draws random numbers and lays them out: hidden states, router
choices, and expert weights in the storage formats the experts forward consumes
(fp32, bf16 bit patterns, or OCP e4m3 codes with 128x128 block scales).  It holds
none of the experts-forward arithmetic, so both the CPU oracle and the GPU path
can be fed from it without sharing any of the method's code.
"""

from .layers import (  # noqa: F401
    CONFIGS,
    Spec,
    spec_for,
    hidden,
    routing,
    expert_gate_up,
    expert_down,
    dense_layer,
    active_experts,
)
