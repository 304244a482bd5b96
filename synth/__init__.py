"""Seeded synthetic inputs for the Stable LatentMoE layer.

This package holds input construction only: shapes, seeded random streams and
the rounding of drawn values to the storage types (bf16, packed e2m1 bytes,
e8m0 bytes).  It holds none of the layer's arithmetic, so that both the CPU
oracle and the HIP path can take their inputs from it without sharing code.
"""
from .inputs import (  # noqa: F401
    LayerShape,
    Workload,
    WORKLOADS,
    K3_SHAPE,
    TINY_SHAPE,
    LAYER0_FFN_SHAPE,
    workload,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    gen_dense,
    gen_gamma_random,
    gen_expert,
    gen_expert_stack,
    gen_expert_affine2,
    gen_expert_affine2_stack,
    gen_expert_paired,
    AFFINE_GROUP,
    gen_tokens,
    gen_bias,
    gen_microbench_counts,
    gen_microbench_activations,
    zipf_permutation,
    zipf_probabilities,
)
