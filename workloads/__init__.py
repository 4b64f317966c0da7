"""Seeded synthetic inputs for the token-pruned attention layer.

This package only draws random tensors of the shapes, value distributions and
static/moving token structure of the workloads; it holds none of the method's
arithmetic (no scoring, selection, projection or attention).  Both the CPU
oracle's tests and the GPU path take their inputs from here.
"""

from .configs import CONFIGS, Config, get_config
from .generate import hsa_inputs, lipar_eps, lipar_inputs, step_inputs

__all__ = [
    "CONFIGS",
    "Config",
    "get_config",
    "step_inputs",
    "hsa_inputs",
    "lipar_inputs",
    "lipar_eps",
]
