"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package holds no step of the attention method itself: it only draws
random numbers, rounds them to bfloat16 once, draws packed-sequence lengths,
and states the fixed per-config inputs (shapes, scale, ALiBi slope values).
Both the oracle and the HIP path consume exactly the arrays produced here.
"""
from .gen import (  # noqa: F401
    bf16_round,
    bf16_bits_to_f32,
    draw_varlen_lengths,
    DenseInputs,
    VarlenInputs,
    draw_dense,
    draw_dense_bias,
    draw_fire_theta,
    draw_rmsnorm,
    draw_cross_entropy,
    draw_varlen,
    alibi_slope_values,
)
from .configs import CONFIGS, Config, config_by_name  # noqa: F401
