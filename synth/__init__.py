"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package draws random numbers and writes them in the canonical (user-side)
weight format.  It holds none of the method's arithmetic: no dequantisation, no
products, no epilogues.  See ``synth.inputs``.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    WeightSet,
    Workload,
    make_weights,
    make_activations,
    make_residual,
    make_workload,
    pack_canonical,
    bf16_bits,
    make_activations_bf16,
)
