"""Seeded synthetic inputs for the MoE expert layer.

This package holds the five layer workloads (shapes, dtypes, routing
structure) and the seeded generators that draw their tensors.  It contains
none of the layer's own arithmetic: routing, histograms, permutation, GEMMs
and combine live in the HIP library and in the CPU oracle ``oracle/``, which
never import each other.  Both sides consume the tensors made here.
"""

from .configs import LayerConfig, CONFIGS, get_config, small_variant
from .generate import LayerInputs, generate, quantize_weight_blocks

__all__ = [
    "LayerConfig",
    "CONFIGS",
    "get_config",
    "small_variant",
    "LayerInputs",
    "generate",
    "quantize_weight_blocks",
]
