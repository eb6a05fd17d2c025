"""Seeded synthetic workloads for paged attention (no attention arithmetic here)."""

from .synth import (  # noqa: F401
    CONFIGS,
    Case,
    SharedPrefixCase,
    config_case,
    draw_values,
    make_case,
    nan_pool,
    shared_prefix_case,
    to_bf16_bits,
)
