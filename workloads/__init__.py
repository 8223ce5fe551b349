"""Seeded synthetic workloads (input data only; no step of the method)."""
from .configs import CONFIGS, SHAPES_128, Config, get, padded_variant  # noqa: F401
from .synth import Workload, make, bf16_bits_to_f32, f32_to_bf16_bits  # noqa: F401
