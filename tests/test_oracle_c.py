"""Pins for the plain C fp64 oracle (the CPU baseline's implementation).

It must agree with the numpy oracle, which is pinned on its own (entrywise and
dense definitions of M, scipy's CSR products and CG loops): the apply and the
SpMV to rounding, and the whole PCG with the same iteration count on the grid
systems (x to rounding level over the first 40 steps, to 1e-7 at the end), at
any thread count.
"""

import numpy as np
import pytest
import scipy.sparse

import oracle
from oracle import c_oracle
from workloads import make_config
from workloads.generate import make_factors


@pytest.mark.parametrize("K,L,R,levels", [(1, 8, 3, 0), (2, 8, 3, 1), (8, 4, 3, 3), (8, 16, 4, 2), (16, 6, 2, 4)])
def test_c_apply_matches_oracle(K, L, R, levels):
    rng = np.random.default_rng(K * 7 + levels)
    U = rng.standard_normal((K, L, L)).astype(np.float32)
    W = rng.standard_normal((levels, K, L, R)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, K * L).astype(np.float32)
    r = rng.standard_normal(K * L)
    y = c_oracle.apply_M(U, W if levels else None, g, r)
    ref = oracle.apply_M(U, W, g, r)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    if K * L <= 64:
        M = np.array([[oracle.dense_M_entry(U, W, g, i, j) for j in range(K * L)] for i in range(K * L)])
        np.testing.assert_allclose(y, M @ r, rtol=1e-12, atol=1e-12 * np.abs(M).sum())


def test_c_spmv_matches_scipy():
    b = make_config("tet4k")
    A = scipy.sparse.csr_matrix((b.val.astype(np.float64), b.col, b.row_ptr), shape=(b.n, b.n))
    x = np.random.default_rng(3).standard_normal(b.n)
    np.testing.assert_allclose(c_oracle.spmv(b.row_ptr, b.col, b.val, x), A @ x, rtol=1e-13, atol=1e-12)


@pytest.mark.parametrize("name", ["N1k", "N8k"])
def test_c_pcg_matches_oracle(name):
    b = make_config(name)
    sy = b.system(0)
    ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), b.tol, b.maxit)
    x, it, st, rel = c_oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, sy.U, sy.W, sy.g, b.tol, b.maxit)
    assert st == ref.status == "converged" and it == ref.iterations
    # rounding differences of the two summation orders grow over the solve
    np.testing.assert_allclose(x, ref.x, rtol=0, atol=1e-7 * np.abs(ref.x).max())
    assert rel <= b.tol and abs(rel - ref.relres) <= 0.05 * ref.relres
    # ... and are at rounding level over the first 40 steps
    ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), b.tol, 40)
    x, it, st, rel = c_oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, sy.U, sy.W, sy.g, b.tol, 40)
    assert st == ref.status == "not_converged" and it == 40
    np.testing.assert_allclose(x, ref.x, rtol=0, atol=1e-13 * np.abs(ref.x).max())
    assert abs(rel - ref.relres) <= 1e-12 * ref.relres


def test_c_pcg_edges_and_thread_count():
    b = make_config("N1k")
    sy = b.system(0)
    # b = 0: converged at once with x = 0
    x, it, st, _ = c_oracle.pcg(sy.row_ptr, sy.col, sy.val, 0 * sy.b, sy.U, sy.W, sy.g, 1e-6, 10)
    assert st == "converged" and it == 0 and not x.any()
    # budget too small
    _, it, st, _ = c_oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, sy.U, sy.W, sy.g, 1e-6, 5)
    assert st == "not_converged" and it == 5
    # indefinite M: breakdown, as the numpy oracle reports it
    bad = c_oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, 0 * sy.U, sy.W, np.full(sy.n, -10.0, np.float32), 1e-6, 10)
    ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (0 * sy.U, sy.W, np.full(sy.n, -10.0)), 1e-6, 10)
    assert bad[2] == ref.status == "breakdown" and bad[1] == ref.iterations
    # thread count does not change a bit
    c_oracle.set_threads(1)
    x1 = c_oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, sy.U, sy.W, sy.g, 1e-6, 1000)[0]
    c_oracle.set_threads(4)
    x4 = c_oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, sy.U, sy.W, sy.g, 1e-6, 1000)[0]
    assert np.array_equal(x1, x4)


def test_c_generated_factors_spd_solve():
    # generated factors on a small system: the C loop reaches the tolerance on the
    # true residual like the numpy oracle
    rng = np.random.default_rng(5)
    b = make_config("N1k")
    sy = b.system(0)
    U, W, g = make_factors(rng, sy.n, np.ones(sy.n), leaf=128, rank=32, levels=3)
    x, it, st, _ = c_oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, U, W, g, 1e-6, 1000)
    ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (U, W, g), 1e-6, 1000)
    assert st == "converged" and it == ref.iterations
    assert oracle.true_relres(sy.row_ptr, sy.col, sy.val, sy.b, x) <= 1.05e-6
