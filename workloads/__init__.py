"""Seeded synthetic inputs for one sequence-parallel rank's share of block-sparse attention.

This package only draws inputs: placements, per-head block masks and bf16 Q/K/V.  It holds none of the
method's arithmetic (no demand union, compaction, pack or attention), so both the HIP path and the CPU
oracle can be fed from it without sharing any of the computation they are compared on.
"""
from .configs import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_from_f32,
    custom,
    make_inputs,
    placement_contiguous,
    placement_periodic,
)
