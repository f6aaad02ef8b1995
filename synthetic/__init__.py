"""Seeded synthetic inputs for paged decode attention.

This package only draws random numbers and lays them out (block tables,
bf16 bit patterns, NaN poison).  It holds none of the attention, append,
quantisation or merge arithmetic: those live in the HIP library and,
independently, in the CPU oracle.  Both consume the arrays produced here.
"""
from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    PagedInputs,
    MultiQueryInputs,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    generate,
    generate_multiquery,
    make_workload,
    random_partials,
)
