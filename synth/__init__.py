"""Seeded synthetic inputs shared by the oracle side and the device side.

This module only draws random numbers and lays them out. It contains none of
the quantizer's arithmetic: no rotation is applied, nothing is quantized,
nothing is estimated. Both the CPU oracle (``oracle/``) and the GPU binding
consume exactly the arrays produced here, so a parity test compares the two
paths on identical inputs.

Every draw uses numpy's PCG64 generator seeded through a SeedSequence whose
entropy is a tuple of integers (seed, stream tag, indices...). Any slab of a
large workload can therefore be regenerated alone, in any order.
"""
from .draws import (
    rng_for,
    haar_orthogonal,
    gaussian_sketch,
    standard_normal,
    to_bf16_exact,
    outlier_channels,
    grouped_channel_permutation,
)
from .workloads import (
    QuantizerSpec,
    GroupSpec,
    Workload,
    WORKLOADS,
    workload,
    draw_quantizer,
    draw_kv_slab,
    draw_queries,
    draw_mixture_vectors,
)

__all__ = [
    "rng_for", "haar_orthogonal", "gaussian_sketch", "standard_normal",
    "to_bf16_exact", "outlier_channels", "grouped_channel_permutation",
    "QuantizerSpec", "GroupSpec", "Workload", "WORKLOADS", "workload",
    "draw_quantizer", "draw_kv_slab", "draw_queries", "draw_mixture_vectors",
]
