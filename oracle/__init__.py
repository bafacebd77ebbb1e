"""Float64 CPU oracle for the affine group-quantized matmul.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, the smoke check and the CPU-baseline
leg of the bench may import it; the GPU library never does, and the oracle never
imports the GPU package.
"""
from .oracle import (  # noqa: F401
    decode_bf16,
    decode_f32,
    unpack,
    matmul,
    matmul_at,
    bound_terms,
    tolerance,
    accumulation_terms,
    accumulation_terms_at,
    f32_sum_bound,
    BF16_WEIGHT_ROUNDING,
    rounding_step,
    strict_tolerance,
    check_outputs,
    build,
    load_library,
    tolerance_coefficient,
    round_bf16,
    silu_mul_bf16,
    gate_up,
    gate_up_tolerance,
    round_f32,
    residual_rms_norm,
    residual_rms_norm_tolerance,
    group_sums,
    group_sum_tolerance,
    unpack_lsb,
    dequant_rows,
    decode_attention,
    decode_attention_tolerance,
    score_terms,
)
