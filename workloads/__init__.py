"""Seeded synthetic inputs for the H-matrix-preconditioned PCG solve.

This package builds the sparse SPD systems, the preconditioner factors and the
right-hand sides that both the HIP path and the CPU oracle consume.  It holds
none of the method's arithmetic (no apply, no SpMV, no PCG): it only assembles
matrices and draws random numbers, so both sides of every parity check start
from the very same fp32 arrays.
"""

from .generate import (  # noqa: F401
    CONFIGS,
    System,
    Batch,
    make_config,
    make_factors,
    make_grid_poisson,
    make_tet_diffusion,
    morton_order,
    build_batch,
)
