"""Seeded synthetic inputs for DSA sparse-MLA prefill attention.

This package only draws inputs (bf16 tensors as uint16 bit patterns, FP8
latents as E4M3 codes with scales, and int32 top-k index buffers). It contains none of the attention arithmetic, so both
the CPU oracle and the HIP path can take their inputs from it without sharing
any of the method's code.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    Case,
    Config,
    VarlenCase,
    bf16_bits_from_f32,
    bf16_bits_to_f32,
    make_case,
    make_varlen_case,
    normal_fp8,
    topk_locality,
    topk_uniform,
)
