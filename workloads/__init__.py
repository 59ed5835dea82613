"""Seeded synthetic workloads for the MoE layer: parameter records and input generators.

Shared by the GPU path's tests and bench and by the oracle's tests. Holds no part of the
layer's arithmetic.
"""
from .configs import CONFIGS, HEADLINE, MoEShape
from .generate import (bf16_bits_to_f32, f32_to_bf16_bits, make_inputs, make_shared_expert, make_upstream_grad,
                       normal_f32, to_float64, zipf_router_bias)

__all__ = ["CONFIGS", "HEADLINE", "MoEShape", "make_inputs", "make_shared_expert", "normal_f32", "to_float64",
           "f32_to_bf16_bits", "bf16_bits_to_f32", "zipf_router_bias", "make_upstream_grad"]
