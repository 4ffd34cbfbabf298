"""Seeded synthetic inputs for paged-attention decode.

This package holds only random-number generation and the shapes of the
workloads. It performs none of the method's arithmetic: no block allocation,
no slot computation, no cache write, no attention. Both the float64 oracle
and the GPU library consume what it produces.
"""

from .workloads import (  # noqa: F401
    SEED,
    WORKLOADS,
    Workload,
    draw_lengths,
    free_stack_permutation,
    normal_array,
    cast,
)
