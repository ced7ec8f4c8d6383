"""Seeded synthetic workloads for the null-expert token-choice MoE layer.

This package only draws inputs (activations, router and expert weights, the
null-logit bias) with fixed seeds. It contains none of the layer's arithmetic:
no routing, no selection, no expert FFN. Both the CPU oracle and the HIP path
consume the arrays it produces, so the two sides always see identical values.
"""
from .configs import CONFIGS, SWEEP, MATCHED_PAIR, Config, get_config  # noqa: F401
from .gen import generate, Workload, bf16_round, bf16_bits_to_f32  # noqa: F401
