"""CSR sparse matrix-vector product in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The system matrix arrives in CSR from the simulator, and A r is the inner
loop's only sparse operation ("Hierarchical Transformer Preconditioning for
Interactive Physics Simulation", section 5 "Preconditioner Application",
stage (iii); Supplementary section 1, "Software stack").  The product is its
definition, y_i = sum over the stored entries (i, j) of A_ij x_j.
"""

from __future__ import annotations

import numpy as np


def spmv(row_ptr, col, val, x, dtype=np.float64):
    """y = A x for a CSR matrix (row_ptr [n+1], col [nnz], val [nnz]), in fp64
    (or in `dtype`; each row is summed in storage order either way)."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    n = row_ptr.size - 1
    rows = np.repeat(np.arange(n), np.diff(row_ptr))
    prods = np.asarray(val, dtype=dtype) * np.asarray(x, dtype=dtype)[np.asarray(col)]
    if np.dtype(dtype) == np.float64:
        return np.bincount(rows, weights=prods, minlength=n)
    y = np.zeros(n, dtype=dtype)
    np.add.at(y, rows, prods)
    return y


def spmv_block(row_ptr, col, val, X):
    """Y = A X for a block X of shape [n, nrhs], column by column."""
    X = np.asarray(X, dtype=np.float64)
    return np.stack([spmv(row_ptr, col, val, X[:, j]) for j in range(X.shape[1])], axis=1)


def spmv_batch(row_ptr, col, val, x):
    """Block-diagonal batch: global CSR over B*n rows, x of shape [B, n]."""
    x = np.asarray(x, dtype=np.float64)
    return spmv(row_ptr, col, val, x.reshape(-1)).reshape(x.shape)


def dense_A(row_ptr, col, val):
    """Dense fp64 copy of a CSR matrix (tiny inputs only)."""
    row_ptr = np.asarray(row_ptr, dtype=np.int64)
    n = row_ptr.size - 1
    A = np.zeros((n, n))
    for i in range(n):
        for e in range(row_ptr[i], row_ptr[i + 1]):
            A[i, col[e]] += float(val[e])
    return A


def true_relres(row_ptr, col, val, b, x, dtype=np.float64) -> float:
    """||b - A x||_2 / ||b||_2 in fp64 (or in `dtype`)."""
    b = np.asarray(b, dtype=dtype)
    res = b - spmv(row_ptr, col, val, x, dtype)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(res) / nb) if nb > 0 else float(np.linalg.norm(res))
