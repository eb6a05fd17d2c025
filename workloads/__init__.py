"""Seeded synthetic workloads for paged attention (no attention arithmetic here)."""

from .synth import CONFIGS, Case, config_case, draw_values, make_case, nan_pool, to_bf16_bits  # noqa: F401
