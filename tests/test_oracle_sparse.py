"""Pins for the oracle's SpMV and for the generated systems it multiplies.

The SpMV is checked against scipy.sparse (an independent CSR kernel) and a
hand-built dense matrix; the generators against closed forms: row sums of the
7-point operator, the spectrum of the constant-coefficient operator, and the
null space of the unconstrained tetrahedral stiffness.
"""

import numpy as np
import pytest
import scipy.sparse

import oracle
from workloads import make_config
from workloads.generate import coo_to_csr, make_grid_poisson, make_tet_diffusion


@pytest.mark.parametrize("name", ["N1k", "tet4k"])
def test_spmv_matches_scipy(name):
    b = make_config(name)
    A = scipy.sparse.csr_matrix((b.val.astype(np.float64), b.col, b.row_ptr), shape=(b.n, b.n))
    x = np.random.default_rng(0).standard_normal(b.n)
    np.testing.assert_allclose(oracle.spmv(b.row_ptr, b.col, b.val, x), A @ x,
                               rtol=1e-13, atol=1e-13 * np.abs(A).sum(axis=1).max())


def test_spmv_dense_and_empty_rows():
    rng = np.random.default_rng(3)
    n = 9
    rows = rng.integers(0, n, 30)
    rows = rows[rows != 4]                 # row 4 stays empty
    cols = rng.integers(0, n, rows.size)
    vals = rng.standard_normal(rows.size)
    rp, c, v = coo_to_csr(n, rows, cols, vals)
    D = np.zeros((n, n))
    np.add.at(D, (rows, cols), vals)
    x = rng.standard_normal(n)
    y = oracle.spmv(rp, c, v, x)
    np.testing.assert_allclose(y, D @ x, rtol=1e-13, atol=1e-13)
    assert y[4] == 0.0
    np.testing.assert_allclose(oracle.dense_A(rp, c, v), D, rtol=1e-15, atol=0)


def test_spmv_batch_is_blockwise():
    b = make_config("batch64x2k", batch=3)
    x = np.random.default_rng(1).standard_normal((3, b.n))
    y = oracle.spmv_batch(b.row_ptr, b.col, b.val, x)
    for s in range(3):
        sy = b.system(s)
        np.testing.assert_allclose(y[s], oracle.spmv(sy.row_ptr, sy.col, sy.val, x[s]), rtol=1e-14)


@pytest.mark.parametrize("name", ["N1k", "N8k", "N16k", "tet4k"])
def test_generated_matrix_symmetric_sorted(name):
    b = make_config(name)
    A = scipy.sparse.csr_matrix((b.val, b.col, b.row_ptr), shape=(b.n, b.n))
    assert (A != A.T).nnz == 0
    for i in range(0, b.n, max(1, b.n // 97)):
        c = b.col[b.row_ptr[i]:b.row_ptr[i + 1]]
        assert np.all(np.diff(c) > 0)


def test_grid_row_sums_are_dirichlet_faces():
    dims = (4, 8, 8)
    rng = np.random.default_rng(5)
    rho = np.where(rng.random(np.prod(dims)) < 0.3, 100.0, 1.0)
    rp, c, v, perm = make_grid_poisson(dims, rho)
    ones = np.ones(rp.size - 1)
    rowsum = oracle.spmv(rp, c, v, ones)
    expect_lex = np.zeros(np.prod(dims))
    nx, ny, _ = dims
    expect_lex[: nx * ny] = 1.0 / rho[: nx * ny]          # z = 0 cells
    np.testing.assert_allclose(rowsum, expect_lex[perm], rtol=1e-12, atol=1e-12)


def test_constant_coefficient_spectrum_closed_form():
    dims = (4, 4, 8)
    nx, ny, nz = dims
    rp, c, v, _ = make_grid_poisson(dims, np.ones(nx * ny * nz))
    lam = np.linalg.eigvalsh(oracle.dense_A(rp, c, v))
    lx = 2 - 2 * np.cos(np.pi * np.arange(nx) / nx)                  # Neumann
    ly = 2 - 2 * np.cos(np.pi * np.arange(ny) / ny)
    lz = 2 - 2 * np.cos(np.pi * (2 * np.arange(nz) + 1) / (2 * nz + 1))  # Dirichlet below, Neumann above
    expect = np.sort((lx[:, None, None] + ly[None, :, None] + lz[None, None, :]).ravel())
    np.testing.assert_allclose(lam, expect, rtol=1e-10, atol=1e-12)


def test_tet_stiffness_kills_constants_away_from_dirichlet():
    rng = np.random.default_rng(9)
    rp, c, v, perm, info = make_tet_diffusion(rng, 6, 2)
    n = rp.size - 1
    rowsum = oracle.spmv(rp, c, v, np.ones(n))
    A = oracle.dense_A(rp, c, v)
    lex_z = np.arange(n) // 36                              # iz of lexicographic vertex
    z_of_row = lex_z[perm]
    free = z_of_row > 1                                     # rows with no Dirichlet neighbour
    np.testing.assert_allclose(rowsum[free], 0.0, atol=1e-10 * np.abs(A).max())
    assert np.all(np.linalg.eigvalsh(A) > 0)                # SPD after elimination
    assert info["n_tets"] == 6 * 5 ** 3


def test_spmv_block_matches_scipy():
    b = make_config("N1k")
    A = scipy.sparse.csr_matrix((b.val.astype(np.float64), b.col, b.row_ptr), shape=(b.n, b.n))
    X = np.random.default_rng(1).standard_normal((b.n, 5))
    np.testing.assert_allclose(oracle.spmv_block(b.row_ptr, b.col, b.val, X), A @ X,
                               rtol=1e-13, atol=1e-13 * np.abs(A).sum(axis=1).max() * np.abs(X).max())
