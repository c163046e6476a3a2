"""Pins for the oracle's other preconditioner forms (M = H H, M = diag(A)^-1),
the lambda_min(H) monitor, the Jacobi fallback, and for the SVD-fitted factors.

Each pin rests on something other than the function it checks: dense brute
force through the entrywise M, closed forms (a diagonal system that Jacobi
solves in one step, eigenvalues of a block-diagonal H from the leaf factors'
singular values), Cholesky as the SPD test, and an exact fit (full rank) whose
squared form is A^{-1} itself."""

import numpy as np
import pytest

import oracle
from workloads import make_config
from workloads.fitted import fit_factors, fitted_batch, matrix_power
from workloads.generate import random_system


def _dense_from_entries(U, W, g):
    N = U.shape[0] * U.shape[1]
    return np.array([[oracle.dense_M_entry(U, W, g, i, j) for j in range(N)] for i in range(N)])


def _small(K, L, R, levels, seed):
    rng = np.random.default_rng(seed)
    U = np.eye(L) + 0.3 * rng.standard_normal((K, L, L))
    W = 0.2 * rng.standard_normal((levels, K, L, R))
    g = rng.uniform(0.1, 0.2, K * L)
    return U, W, g


@pytest.mark.parametrize("K,L,R,levels", [(1, 5, 2, 0), (2, 4, 2, 1), (4, 6, 3, 2), (8, 3, 2, 3)])
def test_squared_apply_is_H_times_H(K, L, R, levels):
    U, W, g = _small(K, L, R, levels, seed=K + levels)
    H = _dense_from_entries(U, W, g)
    r = np.random.default_rng(1).standard_normal(K * L)
    np.testing.assert_allclose(oracle.apply_M_squared(U, W, g, r), H @ (H @ r), rtol=1e-11,
                               atol=1e-11 * np.abs(H).sum() ** 2)


def test_squared_form_is_spd_for_indefinite_H():
    U, W, g = _small(4, 6, 3, 2, seed=5)
    g = g.copy()
    g[::3] = -6.0                        # pushes some eigenvalues of H below zero
    H = _dense_from_entries(U, W, g)
    with pytest.raises(np.linalg.LinAlgError):
        np.linalg.cholesky(H)
    assert np.linalg.matrix_rank(H) == H.shape[0]
    np.linalg.cholesky(H @ H)            # succeeds: H^2 is SPD
    lo, hi = oracle.h_extreme_eigenvalues(U, W, g)
    assert lo < 0 < hi


def test_monitor_closed_form_without_tiles():
    # W = 0 and a constant gate c: H = blockdiag(U_k U_k^T) + c I has the
    # eigenvalues sigma_i(U_k)^2 + c
    U, W, _ = _small(4, 5, 2, 2, seed=9)
    W = np.zeros_like(W)
    c = 0.37
    g = np.full(20, c)
    sv = np.concatenate([np.linalg.svd(U[k], compute_uv=False) for k in range(4)])
    lo, hi = oracle.h_extreme_eigenvalues(U, W, g)
    assert lo == pytest.approx(sv.min() ** 2 + c, rel=1e-12)
    assert hi == pytest.approx(sv.max() ** 2 + c, rel=1e-12)


def _diagonal_csr(d):
    n = d.size
    return np.arange(n + 1, dtype=np.int32), np.arange(n, dtype=np.int32), d.astype(np.float32)


def test_jacobi_solves_a_diagonal_system_in_one_step():
    d = np.linspace(1.0, 50.0, 64)
    rp, col, val = _diagonal_csr(d)
    assert np.array_equal(oracle.diag_of(rp, col, val), val.astype(np.float64))
    b = np.random.default_rng(2).standard_normal(64)
    res = oracle.pcg(rp, col, val, b, lambda v: oracle.apply_jacobi(oracle.diag_of(rp, col, val), v), 1e-12, 10)
    assert res.status == "converged" and res.iterations == 1
    np.testing.assert_allclose(res.x, b / val.astype(np.float64), rtol=1e-14)


def test_diag_of_matches_dense():
    sy = random_system(256, seed=3, levels=1).system(0)
    np.testing.assert_array_equal(oracle.diag_of(sy.row_ptr, sy.col, sy.val),
                                  np.diag(oracle.dense_A(sy.row_ptr, sy.col, sy.val)))


def test_fallback_after_breakdown():
    sy = random_system(256, seed=4, levels=1).system(0)
    g = -np.abs(sy.g) - 1.0
    U = np.zeros_like(sy.U)
    W = np.zeros_like(sy.W)              # H = diag(g) < 0: r.z < 0 at once
    res = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (U, W, g), 1e-6, 500)
    assert res.status == "breakdown" and res.iterations == 0
    fb, fell = oracle.pcg_with_fallback(sy.row_ptr, sy.col, sy.val, sy.b, (U, W, g), 1e-6, 500)
    d = oracle.diag_of(sy.row_ptr, sy.col, sy.val)
    ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, lambda v: v / d, 1e-6, 500)
    assert fell and fb.status == "converged"
    assert fb.iterations == ref.iterations and np.array_equal(fb.x, ref.x)
    ok, fell = oracle.pcg_with_fallback(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), 1e-6, 500)
    assert not fell and ok.status == "converged"


def test_full_rank_fit_is_exact():
    # K = 2 leaves, one 128 x 128 tile: rank 128 reproduces T exactly, so the
    # squared form of the fit to A^{-1/2} is A^{-1} and CG stops after one step
    b = random_system(256, seed=6, levels=1)
    sy = b.system(0)
    T = matrix_power(sy.row_ptr, sy.col, sy.val, -0.5)
    A = oracle.dense_A(sy.row_ptr, sy.col, sy.val)
    np.testing.assert_allclose(T @ (T @ A), np.eye(256), atol=1e-9)
    U, W, g = fit_factors(T, rank=128)
    H = oracle.dense_M(U, W, g)
    np.testing.assert_allclose(H, T, atol=2e-6 * np.abs(T).max())
    res = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, lambda v: oracle.apply_M_squared(U, W, g, v), 1e-5, 50)
    assert res.status == "converged" and res.iterations <= 2


def test_rank32_fit_converges_in_few_iterations():
    # the pages report 3 to 17 iterations for the format fitted to A^{-1/2}
    b = fitted_batch(make_config("N1k"), -0.5)
    sy = b.system(0)
    res = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, lambda v: oracle.apply_M_squared(sy.U, sy.W, sy.g, v),
                     1e-6, 200)
    assert res.status == "converged" and 3 <= res.iterations <= 17, res.iterations
