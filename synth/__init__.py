"""Seeded synthetic workloads for the LatentMoE layer forward pass.

This package is shared by the HIP path's tests/bench and by the CPU oracle's
tests.  It holds shapes, seeds and random draws only: none of the layer's
arithmetic lives here.  Every tensor is drawn in float32 and, for bf16
workloads, rounded to bf16 (round to nearest even) once; the rounded values are
the canonical inputs that both sides consume.
"""

from .configs import CONFIGS, LayerShape, get_config  # noqa: F401
from .generate import (  # noqa: F401
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_workload,
    round_to_bf16,
)
