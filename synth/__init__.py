"""Seeded synthetic inputs shared by the oracle tests and the HIP path.

This package draws random numbers and lays them out in the canonical input
format (bitstream bytes, fp16 bit patterns, bf16 bit patterns, int32
permutations).  It contains none of the decode-and-multiply arithmetic:
that lives, independently, in ``oracle/`` (CPU, test infrastructure) and in
the HIP library.
"""
from .workloads import (  # noqa: F401
    MatrixInputs,
    DENSE_LAYER_SHAPES,
    PREFILL_SHAPES,
    MOE_SHAPES,
    MOE_EXPERTS,
    MOE_TOPK,
    WORKLOADS,
    code_bytes,
    n_hot_channels,
    make_codebook,
    make_radius_table,
    make_activations,
    random_activations,
    make_matrix,
    random_matrix,
    single_matrix,
    dense_layer,
    dense_layer_activations,
    DECODE_CALLS,
    DECODE_LAYERS,
    decode_stack,
    PREFILL_TOKENS,
    prompt_activations,
    call_input_widths,
    prefill_set,
    moe_expert_bd,
    moe_expert,
    moe_routing,
    moe_activations,
    bf16_bits_from_f32,
    bf16_bits_to_f64,
    f16_bits_to_f64,
)
