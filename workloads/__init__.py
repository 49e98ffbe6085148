"""Seeded synthetic inputs shared by the oracle-side tests, the HIP-side
tests and the benchmark.

This module holds only input generation (mask patterns and Gaussian Q/K/V).
It contains none of the attention arithmetic and none of the mask-encoding
arithmetic, so neither the oracle nor the HIP path depends on the other
through it.
"""
from .configs import CONFIGS, Config, get_config
from .gen import make_mask, make_qkv, mask_family, padding_stack, pattern_of

__all__ = ["CONFIGS", "Config", "get_config", "make_mask", "make_qkv",
           "mask_family", "padding_stack", "pattern_of"]
