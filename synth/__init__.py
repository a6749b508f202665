"""Seeded synthetic inputs for hybrid-head prefill attention.

This package holds only input preparation: the workload descriptions
(`configs`) and the seeded generator (`generate`).  It contains none of the
attention, scoring, selection or sparsity-ratio arithmetic, so both the fp64
oracle's tests and the GPU path may import it without sharing any method code.
"""

from .configs import CONFIGS, Config, get_config, MODE_FA, MODE_SSA, MODE_XA
from .generate import make_inputs, bf16_bits_to_f64, bf16_bits_to_f32, f32_to_bf16_bits

__all__ = [
    "CONFIGS", "Config", "get_config", "MODE_FA", "MODE_SSA", "MODE_XA",
    "make_inputs", "bf16_bits_to_f64", "bf16_bits_to_f32", "f32_to_bf16_bits",
]
