"""Seeded synthetic inputs for the W4A16 linear layer (shared by tests and bench).

Holds input generation only: no quantization, packing or contraction.
"""
from .cases import (  # noqa: F401
    CONFIGS,
    Case,
    all_cases,
    case_by_name,
    make_bias,
    make_weight,
    make_x,
    to_bits16,
)
