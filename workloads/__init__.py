"""Seeded synthetic inputs shared by the oracle and the GPU path.

This package holds no arithmetic of the decoding method: only model and
workload shapes (``configs``) and a counter-based pseudo-random generator for
weights, prompts and the planted logit bias (``gen``).  Both the CPU oracle and
the HIP library's tests/bench draw their inputs from here, so the two sides see
bit-identical inputs without sharing any method code.
"""
from .configs import ModelShape, Workload, TINY, LLADA_8B, WORKLOADS, workload
from .gen import (
    tensor_names, gen_tensor, gen_weights, gen_prompt, gen_bias,
    bf16_bits_to_f32, f32_to_bf16_bits,
)

__all__ = [
    "ModelShape", "Workload", "TINY", "LLADA_8B", "WORKLOADS", "workload",
    "tensor_names", "gen_tensor", "gen_weights", "gen_prompt", "gen_bias",
    "bf16_bits_to_f32", "f32_to_bf16_bits",
]
