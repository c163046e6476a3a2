"""Preconditioned conjugate gradients in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages solve A x = b with preconditioned CG and M ~ A^{-1} ("Hierarchical
Transformer Preconditioning for Interactive Physics Simulation", project page,
Introduction and Background, eq. (1)), stopping when ||r_k||_2 / ||r_0||_2 falls
to the tolerance (Supplementary section 1, "Convergence criterion"; main text
section 7.1).  The pages print no listing of the loop, so this is the textbook
preconditioned CG (Saad, "Iterative Methods for Sparse Linear Systems", the
preconditioned CG algorithm in section 9.2) with x_0 = 0, so r_0 = b:

    z = M r,  p = z,  rz = r.z
    repeat:  q = A p;  alpha = rz / p.q;  x += alpha p;  r -= alpha q
             stop if ||r|| / ||b|| <= tol
             z = M r;  beta = (r.z) / rz;  p = z + beta p

Readings taken where the pages are silent: the iteration count is the number
of products q = A p done when the test first passes; the test uses the
recursively updated r; a non-positive or non-finite p.q or r.z stops the loop
as a breakdown.  Everything here is fp64 by default.  The same loop also runs
in extended precision (dtype=np.longdouble, 64-bit significand): CG's
iteration count on a badly conditioned system drifts with rounding, and the
extended run is the near-exact count that a fp64 run with any summation order
should not undercut by much.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .hmatrix import apply_M
from .sparse import spmv, true_relres


@dataclass
class PCGResult:
    x: np.ndarray
    iterations: int
    status: str                  # "converged" | "not_converged" | "breakdown"
    relres: float                # recursive ||r|| / ||b|| at exit
    true_relres: float           # ||b - A x|| / ||b|| from the returned x
    history: list = field(default_factory=list)   # ||r_k|| / ||b|| for k = 1 ..


def pcg(row_ptr, col, val, b, precond, tol: float, maxit: int, dtype=np.float64, store=None) -> PCGResult:
    """Solve A x = b.  precond is either a callable r -> M r or a tuple (U, W, g)
    of preconditioner factors applied with the structured apply.  Vectors and
    scalars are carried in `dtype` (fp64 unless asked otherwise).

    store (e.g. np.float32): the solve vectors r, z, p and q are rounded to
    this type each time one is formed, while every product, dot product,
    scalar and x stay in `dtype`: the vector storage of the pages' precision
    split read as fp32 vectors ("Hierarchical Transformer Preconditioning for
    Interactive Physics Simulation", Supplementary section 7, "Mixed precision
    split": float32 apply path, float64 scalar accumulators)."""
    if store is None:
        def keep(v):
            return v
    else:
        def keep(v):
            return np.asarray(v, dtype=store).astype(dtype)
    if callable(precond):
        apply = precond
    else:
        U, W, g = precond

        def apply(v):
            return apply_M(U, W, g, v, dtype)

    def norm(v):
        return dtype(np.linalg.norm(v))

    b = np.asarray(b, dtype=dtype)
    x = np.zeros_like(b)
    r = b.copy()
    bnorm = norm(b)
    if bnorm == 0.0:
        return PCGResult(x, 0, "converged", 0.0, 0.0, [])

    def out(it, status, rel):
        return PCGResult(x, it, status, float(rel), true_relres(row_ptr, col, val, b, x, dtype), history)

    z = keep(np.asarray(apply(r), dtype=dtype))
    p = z.copy()
    rz = dtype(r @ z)
    history = []
    if not (np.isfinite(rz) and rz > 0.0):
        return PCGResult(x, 0, "breakdown", 1.0, 1.0, history)
    for it in range(1, maxit + 1):
        q = keep(spmv(row_ptr, col, val, p, dtype))
        pq = dtype(p @ q)
        if not (np.isfinite(pq) and pq > 0.0):
            return out(it, "breakdown", norm(r) / bnorm)
        alpha = rz / pq
        x += alpha * p
        r = keep(r - alpha * q)
        rel = norm(r) / bnorm
        history.append(float(rel))
        if rel <= tol:
            return out(it, "converged", rel)
        z = keep(np.asarray(apply(r), dtype=dtype))
        rz_new = dtype(r @ z)
        if not (np.isfinite(rz_new) and rz_new > 0.0):
            return out(it, "breakdown", rel)
        beta = rz_new / rz
        p = keep(z + beta * p)
        rz = rz_new
    return out(maxit, "not_converged", norm(r) / bnorm)


def pcg_refined(row_ptr, col, val, b, precond, tol: float, maxit: int, inner_tol: float, max_outer: int):
    """Outer iterative refinement around PCG ("Hierarchical Transformer
    Preconditioning for Interactive Physics Simulation", Supplementary section 7,
    the loop proposed for rtol <= 1e-10): x = 0; repeat r = b - A x; stop when
    ||r|| <= tol ||b||; solve A d = r / ||r|| to inner_tol; x += ||r|| d.
    Returns (x, inner iterations summed, outer steps, status, true relres)."""
    b = np.asarray(b, dtype=np.float64)
    x = np.zeros_like(b)
    bnorm = float(np.linalg.norm(b))
    iters, outer = 0, 0
    while True:
        r = b - spmv(row_ptr, col, val, x)
        rn = float(np.linalg.norm(r))
        rel = rn / bnorm if bnorm > 0 else 0.0
        if rel <= tol:
            return x, iters, outer, "converged", rel
        if outer >= max_outer or iters >= maxit:
            return x, iters, outer, "not_converged", rel
        inner = pcg(row_ptr, col, val, r / rn, precond, inner_tol, maxit - iters)
        iters += inner.iterations
        outer += 1
        if inner.status == "breakdown":
            return x, iters, outer, "breakdown", rel
        x = x + rn * inner.x


def pcg_block(row_ptr, col, val, Bm, precond, tol: float, maxit: int) -> list:
    """PCG on every column of a node-major block Bm [n, nrhs]: one independent
    solve per column (own step sizes, test and count), the block form of the
    loop above.  Returns one PCGResult per column."""
    Bm = np.asarray(Bm, dtype=np.float64)
    return [pcg(row_ptr, col, val, Bm[:, j], precond, tol, maxit) for j in range(Bm.shape[1])]


def pcg_batch(batch, tol: float | None = None, maxit: int | None = None,
              systems=None) -> list:
    """Independent PCG per system of a workloads.Batch (or the listed systems)."""
    tol = batch.tol if tol is None else tol
    maxit = batch.maxit if maxit is None else maxit
    idx = range(batch.batch) if systems is None else systems
    out = []
    for s in idx:
        sy = batch.system(s)
        out.append(pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), tol, maxit))
    return out
