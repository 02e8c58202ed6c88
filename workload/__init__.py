"""Seeded synthetic workloads for the fused LoRA MLP (gated and ReLU^2) / QKV / O paths.

This package only draws random inputs of the right shapes and distributions.
It holds none of the method's arithmetic, so both the CPU oracle (through the
tests) and the HIP path (through the tests, the smoke check and the bench) can
take their inputs from it.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    WorkloadConfig,
    bf16_round,
    make_attn_inputs,
    make_inputs,
    make_mlp_inputs,
    make_relu2_inputs,
    rng_for,
)
