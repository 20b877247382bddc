"""Seeded synthetic inputs for the fine-grained FP8 path.

This package only draws random numbers and rounds them to BF16 input
tensors.  It holds none of the quantisation or GEMM arithmetic, so both the
CPU oracle and the GPU path can take their inputs from it.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    bf16_bits_from_f32,
    make_workload,
    normal_bf16,
    rng_for,
    route_ids,
    zipf_counts,
)
