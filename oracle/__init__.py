"""CPU fp64 oracle for the H-matrix-preconditioned conjugate-gradient solve.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, obviously checkable
statement of what the solve computes.  Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import it; the product path (the HIP
library and its Python binding) never does, and fails loudly instead of falling
back to it.  It shares no code with the HIP path: both only read the same
seeded fp32 arrays, which the oracle promotes to fp64 exactly.

Modules
  hmatrix  the weak-admissibility partition, the structured apply y = M r,
           a dense assembly of M by its entries, and an SPD certificate
  sparse   CSR matrix-vector product and the true residual
  pcg      preconditioned conjugate gradients
  bridge   the pages' bridge-and-core off-diagonal format and its apply
  forms    M = H H, M = diag(A)^-1, the lambda_min(H) monitor, Jacobi fallback

Every function in this package is pinned by a CPU test against something other
than itself (printed values, closed forms, library routines, brute force).
"""

from .hmatrix import (  # noqa: F401
    tiles,
    tile_count,
    apply_M,
    apply_M_batch,
    apply_M_block,
    dense_M,
    dense_M_entry,
    weyl_lower_bound,
)
from .sparse import spmv, spmv_batch, spmv_block, true_relres, dense_A  # noqa: F401
from .pcg import pcg, pcg_batch, pcg_block, pcg_refined, PCGResult  # noqa: F401
from .bridge import (  # noqa: F401
    apply_M_bridge,
    dense_M_bridge_entry,
    to_slabs,
    pack_bridge,
    weyl_lower_bound_bridge,
    core_count,
)
from .forms import (  # noqa: F401
    apply_M_squared,
    apply_jacobi,
    diag_of,
    h_extreme_eigenvalues,
    pcg_with_fallback,
)
