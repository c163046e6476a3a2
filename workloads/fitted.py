"""Preconditioner factors fitted to a matrix function of A instead of drawn at random.

The pages note that fitting the hierarchical format directly to A^{-1/2}, tile by
tile with a truncated SVD, gives factors that converge in a handful of
iterations on small meshes ("A Neural Hierarchical-Matrix Preconditioner for
Real-Time GPU Solves", section 3, the paragraph on what degrades as N grows).
This module builds such factors as realistic stand-ins for a trained network's
output, without a network:

* T = A^p from a dense symmetric eigendecomposition (p = -1/2 for the squared
  form M = H H, p = -1 for the direct form M = H), so N stays small (a few
  thousand unknowns);
* leaf factor U_k = the lower Cholesky factor of T's diagonal block k, so that
  U_k U_k^T reproduces that block;
* for the tile at level l, index j (row leaves [2jS, 2jS+S), column leaves
  [2jS+S, 2jS+2S), S = 2^l), the rank-r truncated SVD X Sigma Y^T of T's block
  (rows, columns) gives the slabs: the row leaves' slabs stack X Sigma^{1/2},
  the column leaves' slabs stack Y Sigma^{1/2}, so the tile's W_R W_C^T is the
  best rank-r approximation of the block;
* gate 0.

It draws no random numbers and computes nothing of the solve itself (no
apply, no SpMV, no CG): it only turns a matrix into factor arrays in the
library's layout, stored in fp32.
"""

from __future__ import annotations

import numpy as np

from .generate import LEAF, RANK, Batch, build_batch, System


def _dense(row_ptr, col, val, n):
    A = np.zeros((n, n))
    rows = np.repeat(np.arange(n), np.diff(row_ptr))
    A[rows, col] = np.asarray(val, dtype=np.float64)
    return A


def matrix_power(row_ptr, col, val, p: float) -> np.ndarray:
    """Dense A^p of a sparse SPD A (fp64, eigendecomposition)."""
    n = row_ptr.size - 1
    w, Q = np.linalg.eigh(_dense(row_ptr, col, val, n))
    assert w[0] > 0, "A must be positive definite"
    return (Q * w ** p) @ Q.T


def fit_factors(T: np.ndarray, leaf: int = LEAF, rank: int = RANK, levels: int | None = None):
    """(U [K, L, L], W [levels, K, L, rank], g [N]) fitted to the symmetric T."""
    n = T.shape[0]
    K = n // leaf
    assert K * leaf == n and K & (K - 1) == 0
    full = K.bit_length() - 1
    levels = full if levels is None else levels
    U = np.empty((K, leaf, leaf))
    for k in range(K):
        s = slice(k * leaf, (k + 1) * leaf)
        U[k] = np.linalg.cholesky(T[s, s])
    W = np.zeros((levels, K, leaf, rank))
    for lev in range(levels):
        S = 1 << lev
        for j in range(K // (2 * S)):
            r0, c0 = 2 * j * S, 2 * j * S + S
            blk = T[r0 * leaf:(r0 + S) * leaf, c0 * leaf:(c0 + S) * leaf]
            X, sig, Yt = np.linalg.svd(blk, full_matrices=False)
            k_eff = min(rank, sig.size)
            root = np.sqrt(sig[:k_eff])
            Wr = np.zeros((S * leaf, rank))
            Wc = np.zeros((S * leaf, rank))
            Wr[:, :k_eff] = X[:, :k_eff] * root
            Wc[:, :k_eff] = Yt[:k_eff].T * root
            W[lev, r0:r0 + S] = Wr.reshape(S, leaf, rank)
            W[lev, c0:c0 + S] = Wc.reshape(S, leaf, rank)
    return U.astype(np.float32), W.astype(np.float32), np.zeros(n, dtype=np.float32)


def fitted_batch(batch: Batch, power: float, rank: int = RANK) -> Batch:
    """A copy of `batch` whose factors are fitted to A_s^power for every system s."""
    systems = []
    for s in range(batch.batch):
        sy = batch.system(s)
        T = matrix_power(sy.row_ptr, sy.col, sy.val, power)
        U, W, g = fit_factors(T, rank=rank, levels=sy.levels)
        systems.append(System(sy.n, sy.row_ptr, sy.col, sy.val, U, W, g, sy.b, dict(sy.meta, fitted=power)))
    return build_batch(systems, batch.tol, batch.maxit, f"{batch.name}-fit{power:g}")
