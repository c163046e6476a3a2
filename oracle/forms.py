"""Preconditioner forms besides M = H: the squared form, the Jacobi form, the
lambda_min(H) monitor and the Jacobi fallback.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"A Neural Hierarchical-Matrix Preconditioner for Real-Time GPU Solves",
section 2 ("SPD by construction"): with the off-diagonal tiles mirrored, H is
symmetric, so M = H^2 is SPD whenever H is nonsingular; the authors watch
lambda_min(H) and keep Jacobi as the fallback.  Readings taken here:

* H is the structured operator of `hmatrix.apply_M` (leaf blocks, mirrored
  tiles, gate); the squared form applies it twice, M r = H (H r).
* Jacobi is M = diag(A)^{-1} (the pages' per-node Jacobi scaling uses the same
  diagonal).
* The monitor's value is the smallest eigenvalue of H (of every system of a
  batch); here it is computed exactly from the dense H.
* The fallback: a solve whose CG breaks down (r.z or p.q not positive and
  finite, which an M that is not SPD can cause) is run again from x = 0 with
  the Jacobi form.
"""

from __future__ import annotations

import numpy as np

from .hmatrix import apply_M, dense_M
from .pcg import pcg


def apply_M_squared(U, W, g, r):
    """M r = H (H r), H the structured apply."""
    return apply_M(U, W, g, apply_M(U, W, g, r))


def diag_of(row_ptr, col, val) -> np.ndarray:
    """diag(A) of a CSR matrix, fp64."""
    row_ptr = np.asarray(row_ptr)
    n = row_ptr.size - 1
    d = np.zeros(n)
    for i in range(n):
        for k in range(row_ptr[i], row_ptr[i + 1]):
            if col[k] == i:
                d[i] += float(val[k])
    return d


def apply_jacobi(diag, r):
    """M r = diag(A)^{-1} r."""
    return np.asarray(r, dtype=np.float64) / np.asarray(diag, dtype=np.float64)


def h_extreme_eigenvalues(U, W, g):
    """(lambda_min(H), lambda_max(H)) from the dense symmetric H (tiny inputs)."""
    w = np.linalg.eigvalsh(dense_M(U, W, g))
    return float(w[0]), float(w[-1])


def pcg_with_fallback(row_ptr, col, val, b, precond, tol: float, maxit: int):
    """PCG with `precond`; on breakdown, PCG again with Jacobi.
    Returns (result, fell_back)."""
    res = pcg(row_ptr, col, val, b, precond, tol, maxit)
    if res.status != "breakdown":
        return res, False
    d = diag_of(row_ptr, col, val)
    return pcg(row_ptr, col, val, b, lambda v: apply_jacobi(d, v), tol, maxit), True
