"""Pins for the oracle's partition and structured apply y = M r.

Each check ties the oracle to something other than itself: the tile counts and
factor sizes the pages print, an entrywise definition of M derived from the
tree geometry, a second dense assembly through W Pi W^T, scipy's block_diag,
symmetry and linearity, and a Cholesky factorization.
"""

import os

import numpy as np
import pytest
import scipy.linalg
from hypothesis import given, settings, strategies as st

import oracle
from workloads.generate import make_factors

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "factor_tensor_sizes.txt")


def _factors(K, L, R, levels, seed, gate=True):
    rng = np.random.default_rng(seed)
    U = rng.standard_normal((K, L, L))
    W = rng.standard_normal((levels, K, L, R))
    g = rng.uniform(0.5, 1.5, K * L) if gate else np.zeros(K * L)
    return U, W, g


def test_tile_count_matches_printed_table():
    rows = [list(map(float, line.split())) for line in open(GOLDEN)
            if line.strip() and not line.startswith("#")]
    L, Ls = 128, 32
    for N, K, MH, KL2, P, MB in rows:
        N, K, MH = int(N), int(K), int(MH)
        assert N // L == K
        got = oracle.tile_count(K)
        assert got == MH
        packed = K * L * L + got * Ls * Ls + 2 * N * Ls + N
        assert round(K * L * L / 1e6, 3) == pytest.approx(KL2)
        assert round(packed / 1e6, 2) == pytest.approx(P)
        mb = packed * 4 / 1e6
        assert round(mb, 2 if mb < 10 else 1) == pytest.approx(MB)


@pytest.mark.parametrize("K", [1, 2, 4, 8, 16, 64, 128])
def test_every_leaf_in_one_tile_per_level(K):
    levels = K.bit_length() - 1
    ts = oracle.tiles(K, levels)
    assert len(ts) == K - 1
    for lev in range(levels):
        seen = []
        for lv, _j, rows, cols in ts:
            if lv == lev:
                assert len(rows) == len(cols) == 1 << lev
                assert rows.stop == cols.start
                seen += list(rows) + list(cols)
        assert sorted(seen) == list(range(K))


@pytest.mark.parametrize("K,L,R,levels", [(1, 8, 3, 0), (2, 8, 3, 1), (4, 6, 2, 2),
                                          (8, 4, 3, 3), (8, 4, 3, 1), (16, 4, 2, 4)])
def test_apply_equals_entrywise_definition(K, L, R, levels):
    U, W, g = _factors(K, L, R, levels, seed=K * 100 + levels)
    N = K * L
    M = np.array([[oracle.dense_M_entry(U, W, g, i, j) for j in range(N)] for i in range(N)])
    rng = np.random.default_rng(7)
    for _ in range(3):
        r = rng.standard_normal(N)
        y = oracle.apply_M(U, W, g, r)
        np.testing.assert_allclose(y, M @ r, rtol=1e-12, atol=1e-12 * np.abs(M).sum())
    np.testing.assert_allclose(M, oracle.dense_M(U, W, g), rtol=1e-13, atol=1e-13)


def test_leaf_only_is_scipy_block_diagonal():
    U, W, g = _factors(8, 16, 4, 0, seed=3, gate=False)
    r = np.random.default_rng(1).standard_normal(8 * 16)
    B = scipy.linalg.block_diag(*[U[k] @ U[k].T for k in range(8)])
    np.testing.assert_allclose(oracle.apply_M(U, W, g, r), B @ r, rtol=1e-12)


def test_single_tile_two_leaves_explicit():
    # K = 2: M = [[U0 U0^T, W0 W1^T], [W1 W0^T, U1 U1^T]] + diag(g)
    U, W, g = _factors(2, 5, 2, 1, seed=11)
    top = np.hstack([U[0] @ U[0].T, W[0, 0] @ W[0, 1].T])
    bot = np.hstack([W[0, 1] @ W[0, 0].T, U[1] @ U[1].T])
    M = np.vstack([top, bot]) + np.diag(g)
    r = np.random.default_rng(2).standard_normal(10)
    np.testing.assert_allclose(oracle.apply_M(U, W, g, r), M @ r, rtol=1e-12)


@settings(max_examples=25, deadline=None)
@given(logK=st.integers(0, 4), L=st.integers(1, 9), R=st.integers(1, 4),
       seed=st.integers(0, 2 ** 31 - 1), data=st.data())
def test_symmetric_and_linear(logK, L, R, seed, data):
    K = 1 << logK
    levels = data.draw(st.integers(0, logK))
    U, W, g = _factors(K, L, R, levels, seed)
    rng = np.random.default_rng(seed ^ 0x5A5A)
    u, v = rng.standard_normal((2, K * L))
    a, b = rng.standard_normal(2)
    Mu, Mv = oracle.apply_M(U, W, g, u), oracle.apply_M(U, W, g, v)
    scale = np.linalg.norm(Mu) * np.linalg.norm(v) + np.linalg.norm(Mv) * np.linalg.norm(u)
    assert abs(u @ Mv - v @ Mu) <= 1e-12 * scale
    np.testing.assert_allclose(oracle.apply_M(U, W, g, a * u + b * v), a * Mu + b * Mv,
                               rtol=1e-10, atol=1e-10 * (np.abs(Mu).max() + np.abs(Mv).max()))


@pytest.mark.parametrize("K,L,levels", [(8, 32, 3), (16, 16, 4), (4, 64, 1)])
def test_generated_factors_spd_and_weyl_bound(K, L, levels):
    rng = np.random.default_rng(K + L)
    n = K * L
    diag_a = rng.uniform(0.5, 700.0, n)
    U, W, g = make_factors(rng, n, diag_a, leaf=L, rank=8, levels=levels)
    M = oracle.dense_M(U, W, g)
    assert np.array_equal(M, M.T) or np.abs(M - M.T).max() < 1e-14
    np.linalg.cholesky(M)                      # raises unless SPD
    lam_min = np.linalg.eigvalsh(M)[0]
    bound = oracle.weyl_lower_bound(U, W, g)
    assert 0.0 < bound <= lam_min + 1e-12


def test_weyl_bound_is_a_true_lower_bound_on_rough_factors():
    # large off-diagonal factors: the bound must stay below lambda_min even when negative
    U, W, g = _factors(8, 6, 3, 3, seed=5)
    M = oracle.dense_M(U, W, g)
    assert oracle.weyl_lower_bound(U, W, g) <= np.linalg.eigvalsh(M)[0] + 1e-10


@pytest.mark.parametrize("K,L,R,levels", [(4, 6, 2, 2), (8, 4, 3, 3)])
def test_block_apply_is_dense_product(K, L, R, levels):
    # the block apply against the dense closed form times the whole block
    U, W, g = _factors(K, L, R, levels, seed=31 + K)
    R_blk = np.random.default_rng(5).standard_normal((K * L, 7))
    np.testing.assert_allclose(oracle.apply_M_block(U, W, g, R_blk), oracle.dense_M(U, W, g) @ R_blk,
                               rtol=1e-12, atol=1e-12 * np.abs(R_blk).max())


def test_batch_apply_is_per_system_dense_product():
    # three systems with their own factors, gates and inputs: every row of the
    # batched apply must be that system's own entrywise M times its own r (an
    # axis mix-up between systems, leaves or levels lands on another system's
    # factors and fails)
    K, L, R, levels, B = 4, 6, 2, 2, 3
    fac = [_factors(K, L, R, levels, seed=70 + s) for s in range(B)]
    U = np.stack([f[0] for f in fac])
    W = np.stack([f[1] for f in fac])
    g = np.stack([f[2] for f in fac])
    r = np.random.default_rng(9).standard_normal((B, K * L))
    y = oracle.apply_M_batch(U, W, g, r)
    assert y.shape == (B, K * L)
    N = K * L
    for s in range(B):
        M = np.array([[oracle.dense_M_entry(U[s], W[s], g[s], i, j) for j in range(N)] for i in range(N)])
        np.testing.assert_allclose(y[s], M @ r[s], rtol=1e-12, atol=1e-12 * np.abs(M).sum())
    # the systems really differ, so a swap would have been seen
    assert np.abs(y[0] - y[1]).max() > 1e-3
