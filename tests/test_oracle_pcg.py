"""Pins for the oracle's PCG loop.

scipy.sparse.linalg.cg is an independent textbook (P)CG loop: with M = I and
with M given as a LinearOperator it must take the same number of steps and
return the same x.  Exact preconditioners finish in one step; PCG is invariant
under M -> cM (the scale invariance the pages build their loss on, project
page, Training, Proposition 1); CG ends within n steps in exact arithmetic.
"""

import numpy as np
import pytest
import scipy.sparse
import scipy.sparse.linalg as spla

import oracle
from workloads import make_config
from workloads.generate import random_system


def _scipy_cg(A, b, tol, maxit, M=None):
    count = [0]

    def cb(_x):
        count[0] += 1

    x, info = spla.cg(A, b, rtol=tol, atol=0.0, maxiter=maxit, M=M, callback=cb)
    return x, count[0], info


@pytest.mark.parametrize("name", ["N1k", "tet4k"])
def test_identity_preconditioner_is_textbook_cg(name):
    b = make_config(name)
    sy = b.system(0)
    A = scipy.sparse.csr_matrix((sy.val.astype(np.float64), sy.col, sy.row_ptr), shape=(b.n, b.n))
    rhs = sy.b.astype(np.float64)
    res = oracle.pcg(sy.row_ptr, sy.col, sy.val, rhs, lambda v: v.copy(), 1e-6, 5000)
    xs, its, info = _scipy_cg(A, rhs, 1e-6, 5000)
    assert info == 0 and res.status == "converged"
    assert res.iterations == its
    np.testing.assert_allclose(res.x, xs, rtol=1e-9, atol=1e-9 * np.abs(xs).max())


def test_hmatrix_preconditioner_matches_scipy_pcg():
    b = make_config("N1k")
    sy = b.system(0)
    A = scipy.sparse.csr_matrix((sy.val.astype(np.float64), sy.col, sy.row_ptr), shape=(b.n, b.n))
    Mop = spla.LinearOperator((b.n, b.n), matvec=lambda v: oracle.apply_M(sy.U, sy.W, sy.g, v))
    rhs = sy.b.astype(np.float64)
    res = oracle.pcg(sy.row_ptr, sy.col, sy.val, rhs, (sy.U, sy.W, sy.g), 1e-6, 1000)
    xs, its, info = _scipy_cg(A, rhs, 1e-6, 1000, M=Mop)
    assert info == 0 and res.status == "converged"
    assert res.iterations == its
    np.testing.assert_allclose(res.x, xs, rtol=1e-9, atol=1e-9 * np.abs(xs).max())
    assert res.true_relres <= 1.01e-6


def test_exact_inverse_takes_one_step():
    b = random_system(256, seed=4, leaf=32, rank=4)
    sy = b.system(0)
    Ainv = np.linalg.inv(oracle.dense_A(sy.row_ptr, sy.col, sy.val))
    res = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, lambda v: Ainv @ v, 1e-10, 50)
    assert res.status == "converged" and res.iterations == 1
    assert res.true_relres < 1e-11


def test_format_exact_block_diagonal_inverse():
    # keep only the in-leaf couplings of A; U_k = chol(A_kk)^{-T} gives M = A^{-1}
    b = random_system(512, seed=8, leaf=64, rank=4)
    sy = b.system(0)
    L = 64
    A = oracle.dense_A(sy.row_ptr, sy.col, sy.val)
    K = sy.n // L
    Ab = np.zeros_like(A)
    U = np.zeros((K, L, L))
    for k in range(K):
        blk = A[k * L:(k + 1) * L, k * L:(k + 1) * L]
        Ab[k * L:(k + 1) * L, k * L:(k + 1) * L] = blk
        U[k] = np.linalg.inv(np.linalg.cholesky(blk)).T
    S = scipy.sparse.csr_matrix(Ab)
    W = np.zeros((3, K, L, 4))
    res = oracle.pcg(S.indptr, S.indices, S.data, sy.b, (U, W, np.zeros(sy.n)), 1e-10, 50)
    assert res.status == "converged" and res.iterations == 1


def test_scale_invariance():
    b = make_config("N1k")
    sy = b.system(0)
    r1 = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), 1e-6, 1000)
    c = 37.5
    r2 = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b,
                    lambda v: c * oracle.apply_M(sy.U, sy.W, sy.g, v), 1e-6, 1000)
    assert r1.iterations == r2.iterations
    np.testing.assert_allclose(r1.x, r2.x, rtol=1e-8, atol=1e-8 * np.abs(r1.x).max())


def test_finite_termination_small_system():
    rng = np.random.default_rng(12)
    n = 48
    Q = np.linalg.qr(rng.standard_normal((n, n)))[0]
    A = Q @ np.diag(np.linspace(1.0, 4.0, n)) @ Q.T
    A = (A + A.T) / 2
    S = scipy.sparse.csr_matrix(A)
    rhs = rng.standard_normal(n)
    res = oracle.pcg(S.indptr, S.indices, S.data, rhs, lambda v: v.copy(), 1e-12, 500)
    assert res.status == "converged" and res.iterations <= n
    # two distinct eigenvalues: CG converges in two steps
    A2 = Q @ np.diag(np.where(np.arange(n) < n // 2, 1.0, 3.0)) @ Q.T
    S2 = scipy.sparse.csr_matrix((A2 + A2.T) / 2)
    res2 = oracle.pcg(S2.indptr, S2.indices, S2.data, rhs, lambda v: v.copy(), 1e-10, 500)
    assert res2.iterations == 2


def test_edge_cases():
    b = make_config("N1k")
    sy = b.system(0)
    zero = oracle.pcg(sy.row_ptr, sy.col, sy.val, np.zeros(sy.n), (sy.U, sy.W, sy.g), 1e-6, 10)
    assert zero.status == "converged" and zero.iterations == 0 and not zero.x.any()
    one = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), 1e-6, 1)
    assert one.status == "not_converged" and one.iterations == 1 and one.x.any()
    bad = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b,
                     (0 * sy.U, sy.W, np.full(sy.n, -10.0)), 1e-6, 10)
    assert bad.status == "breakdown"


def test_batch_equals_per_system():
    # pcg_batch against scipy's independent PCG loop on each system's diagonal
    # block, cut by hand from the batch's global (block-diagonal) CSR, with M
    # applied from that system's own factors: a system or axis mix-up fails
    b = make_config("batch64x2k", batch=3)
    res = oracle.pcg_batch(b)
    A = scipy.sparse.csr_matrix((b.val.astype(np.float64), b.col, b.row_ptr), shape=(b.batch * b.n,) * 2)
    for s in range(b.batch):
        As = A[s * b.n:(s + 1) * b.n, s * b.n:(s + 1) * b.n]
        assert A[s * b.n:(s + 1) * b.n].nnz == As.nnz          # block-diagonal batch
        Mop = spla.LinearOperator((b.n, b.n), matvec=lambda v, s=s: oracle.apply_M(b.U[s], b.W[s], b.g[s], v))
        rhs = b.b[s].astype(np.float64)
        xs, its, info = _scipy_cg(As, rhs, b.tol, b.maxit, M=Mop)
        assert info == 0 and res[s].status == "converged"
        assert res[s].iterations == its, (s, res[s].iterations, its)
        np.testing.assert_allclose(res[s].x, xs, rtol=1e-9, atol=1e-9 * np.abs(xs).max())
    assert len({r.iterations for r in res}) > 1 or not np.allclose(res[0].x, res[1].x)


def test_extended_precision_run():
    # The same loop carried in np.longdouble: on a well-conditioned system it
    # agrees with fp64 (count and x); it really runs in the wider type.
    sy = make_config("N1k").system(0)
    d = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), 1e-6, 1000)
    e = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), 1e-6, 1000, dtype=np.longdouble)
    assert e.x.dtype == np.longdouble and e.status == "converged"
    assert e.iterations == d.iterations
    # rounding differences stay at 1e-15 for the first ~50 steps, then grow
    d = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), 1e-6, 40)
    e = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), 1e-6, 40, dtype=np.longdouble)
    np.testing.assert_allclose(e.x.astype(np.float64), d.x, rtol=0, atol=1e-12 * np.abs(d.x).max())
    assert not np.array_equal(e.x, d.x.astype(np.longdouble))
    # exact preconditioner: one step in either precision
    b = random_system(256, seed=4, leaf=32, rank=4)
    sy = b.system(0)
    Ainv = np.linalg.inv(oracle.dense_A(sy.row_ptr, sy.col, sy.val))
    e1 = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, lambda v: (Ainv @ v.astype(np.float64)).astype(np.longdouble),
                    1e-10, 50, dtype=np.longdouble)
    assert e1.iterations == 1


def test_rounding_sensitivity_of_iteration_counts():
    # On the tetrahedral system (a 100:1 coefficient jump) rounding differences
    # grow by orders of magnitude within tens of steps, so the iteration count
    # depends on the arithmetic: fewer steps in extended precision than in fp64.
    # The first steps still agree closely.
    sy = make_config("tet4k").system(0)
    d = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), 1e-6, 2000)
    e = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), 1e-6, 2000, dtype=np.longdouble)
    assert d.status == e.status == "converged"
    assert e.iterations < d.iterations - 2
    np.testing.assert_allclose(d.history[:5], e.history[:5], rtol=1e-12)


def test_refinement_reaches_tight_tolerance():
    # outer refinement with a loose inner tolerance reaches 1e-10 on the true
    # residual; the number of outer steps is about log(tol) / log(inner_tol)
    sy = make_config("N1k").system(0)
    x, its, outer, status, rel = oracle.pcg_refined(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g),
                                                    1e-10, 5000, 1e-4, 10)
    assert status == "converged" and rel <= 1e-10
    assert 3 <= outer <= 4
    assert rel == pytest.approx(oracle.true_relres(sy.row_ptr, sy.col, sy.val, sy.b, x), rel=1e-12)
    # with the inner tolerance at the outer one, one step is plain PCG
    x1, its1, outer1, status1, _ = oracle.pcg_refined(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g),
                                                      1e-6, 1000, 1e-6, 10)
    plain = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), 1e-6, 1000)
    assert its1 >= plain.iterations and outer1 >= 1
    # against a direct solve: the refined x is the solution to ~ cond(A) * 1e-10
    A = oracle.dense_A(sy.row_ptr, sy.col, sy.val)
    xs = np.linalg.solve(A, sy.b.astype(np.float64))
    assert np.linalg.norm(x - xs) <= 1e-6 * np.linalg.norm(xs)


def test_block_pcg_columns_are_independent_solves():
    # block PCG = one solve per column: equal columns give equal results, a zero
    # column stops at once, a permutation of the columns permutes the results,
    # and a scaled column gives the scaled solution with the same count
    from workloads.generate import random_system
    sy = random_system(256, seed=31, levels=1).system(0)
    rng = np.random.default_rng(5)
    b0, b1 = rng.standard_normal(256), rng.standard_normal(256)
    Bm = np.stack([b0, np.zeros(256), b1, b0, 4.0 * b1], axis=1)
    res = oracle.pcg_block(sy.row_ptr, sy.col, sy.val, Bm, (sy.U, sy.W, sy.g), 1e-8, 300)
    assert [r.status for r in res] == ["converged"] * 5
    assert res[1].iterations == 0 and not res[1].x.any()
    assert res[0].iterations == res[3].iterations and np.array_equal(res[0].x, res[3].x)
    assert res[4].iterations == res[2].iterations
    np.testing.assert_allclose(res[4].x, 4.0 * res[2].x, rtol=1e-12, atol=1e-14)
    perm = oracle.pcg_block(sy.row_ptr, sy.col, sy.val, Bm[:, ::-1], (sy.U, sy.W, sy.g), 1e-8, 300)
    for a, b in zip(res, perm[::-1]):
        assert a.iterations == b.iterations and np.array_equal(a.x, b.x)
    # each column solves its own system
    A = oracle.dense_A(sy.row_ptr, sy.col, sy.val)
    for j in (0, 2):
        np.testing.assert_allclose(A @ res[j].x, Bm[:, j], atol=1e-7 * np.linalg.norm(Bm[:, j]))


def test_fp32_vector_storage_option():
    # store=np.float32 keeps r, z, p and q as fp32 values (the pages' fp32
    # vectors) with fp64 products, scalars and x.  store=np.float64 changes
    # nothing; an exact inverse still stops after one step (at a tolerance
    # above the fp32 rounding of z times the condition number); a
    # well-conditioned grid system keeps the fp64 count within 2; on the
    # tetrahedral system the
    # fp32 storage alone costs about a quarter more iterations (the reason the
    # fp32-vector mode is not held to the fp64 count there).
    sy = make_config("N1k").system(0)
    pre = (sy.U, sy.W, sy.g)
    d = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, pre, 1e-6, 1000)
    same = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, pre, 1e-6, 1000, store=np.float64)
    assert same.iterations == d.iterations and np.array_equal(same.x, d.x)
    f = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, pre, 1e-6, 1000, store=np.float32)
    assert f.status == "converged" and abs(f.iterations - d.iterations) <= 2
    assert not np.array_equal(f.x, d.x)
    np.testing.assert_allclose(f.x, d.x, rtol=0, atol=1e-4 * np.abs(d.x).max())
    assert f.true_relres <= 1.1e-6
    b = random_system(256, seed=4, leaf=32, rank=4)
    s2 = b.system(0)
    Ainv = np.linalg.inv(oracle.dense_A(s2.row_ptr, s2.col, s2.val))
    one = oracle.pcg(s2.row_ptr, s2.col, s2.val, s2.b, lambda v: Ainv @ v, 1e-4, 10, store=np.float32)
    assert one.iterations == 1
    t = make_config("tet4k").system(0)
    pre = (t.U, t.W, t.g)
    d = oracle.pcg(t.row_ptr, t.col, t.val, t.b, pre, 1e-6, 2000)
    f = oracle.pcg(t.row_ptr, t.col, t.val, t.b, pre, 1e-6, 2000, store=np.float32)
    assert f.status == "converged" and f.iterations >= 1.15 * d.iterations, (f.iterations, d.iterations)
