"""Pins for the oracle's bridge-format apply (the pages' per-leaf bridges and
per-tile cores): an entrywise definition of M from the partition geometry,
symmetry, the packed width the pages print (Supplementary Table 3), and an SPD
certificate checked against Cholesky."""

import os

import numpy as np
import pytest

import oracle
from workloads.generate import make_bridge_factors, make_factors

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "factor_tensor_sizes.txt")


def _bridge(K, L, Ls, levels, seed):
    rng = np.random.default_rng(seed)
    F = rng.standard_normal((K, L, L))
    Ub = rng.standard_normal((K, L, Ls))
    Vb = rng.standard_normal((K, L, Ls))
    Bc = rng.standard_normal((oracle.core_count(K, levels), Ls, Ls))
    g = rng.uniform(0.5, 1.5, K * L)
    return F, Ub, Vb, Bc, g


@pytest.mark.parametrize("K,L,Ls,levels", [(1, 6, 2, 0), (2, 5, 2, 1), (4, 6, 3, 2), (8, 4, 3, 3), (8, 4, 2, 1),
                                           (16, 3, 2, 4)])
def test_bridge_apply_equals_entrywise_definition(K, L, Ls, levels):
    F, Ub, Vb, Bc, g = _bridge(K, L, Ls, levels, seed=K * 10 + levels)
    N = K * L
    M = np.array([[oracle.dense_M_bridge_entry(F, Ub, Vb, Bc, g, i, j) for j in range(N)] for i in range(N)])
    np.testing.assert_allclose(M, M.T, rtol=1e-12, atol=1e-12)
    rng = np.random.default_rng(3)
    for _ in range(3):
        r = rng.standard_normal(N)
        np.testing.assert_allclose(oracle.apply_M_bridge(F, Ub, Vb, Bc, g, r), M @ r,
                                   rtol=1e-12, atol=1e-12 * np.abs(M).sum())


def test_two_leaves_one_core_explicit():
    # K = 2: M = [[F0 F0^T, U0 B V1^T], [V1 B^T U0^T, F1 F1^T]] + diag(g)
    F, Ub, Vb, Bc, g = _bridge(2, 4, 2, 1, seed=5)
    top = np.hstack([F[0] @ F[0].T, Ub[0] @ Bc[0] @ Vb[1].T])
    bot = np.hstack([Vb[1] @ Bc[0].T @ Ub[0].T, F[1] @ F[1].T])
    M = np.vstack([top, bot]) + np.diag(g)
    r = np.random.default_rng(1).standard_normal(8)
    np.testing.assert_allclose(oracle.apply_M_bridge(F, Ub, Vb, Bc, g, r), M @ r, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("K,levels", [(4, 2), (8, 3), (16, 2)])
def test_slab_expansion_gives_the_same_M(K, levels):
    F, Ub, Vb, Bc, g = _bridge(K, 5, 3, levels, seed=K + 100)
    W = oracle.to_slabs(Ub, Vb, Bc, K, levels)
    r = np.random.default_rng(2).standard_normal(K * 5)
    np.testing.assert_allclose(oracle.apply_M(F, W, g, r), oracle.apply_M_bridge(F, Ub, Vb, Bc, g, r),
                               rtol=1e-12, atol=1e-12 * np.abs(r).sum())


def test_packed_width_matches_printed_table():
    rows = [list(map(float, line.split())) for line in open(GOLDEN)
            if line.strip() and not line.startswith("#")]
    L, Ls = 128, 32
    for N, K, MH, _kl2, P, _mb in rows:
        N, K = int(N), int(K)
        levels = K.bit_length() - 1
        F = np.zeros((K, L, L), np.float32)
        Ub = np.zeros((K, L, Ls), np.float32)
        Bc = np.zeros((oracle.core_count(K, levels), Ls, Ls), np.float32)
        packed = oracle.pack_bridge(F, Ub, Ub, Bc, np.zeros(N, np.float32))
        assert Bc.shape[0] == int(MH)
        assert round(packed.size / 1e6, 2) == pytest.approx(P)


@pytest.mark.parametrize("K,levels", [(4, 2), (8, 3), (16, 4)])
def test_generated_bridge_factors_spd(K, levels):
    rng = np.random.default_rng(K)
    L = 16
    diag = np.full(K * L, 6.0)
    F, _W, g = make_factors(rng, K * L, diag, leaf=L, rank=4, levels=0)
    Ub, Vb, Bc = make_bridge_factors(rng, K, levels, leaf=L, rank=4)
    bound = oracle.weyl_lower_bound_bridge(F, Ub, Vb, Bc, g)
    M = np.array([[oracle.dense_M_bridge_entry(F, Ub, Vb, Bc, g, i, j) for j in range(K * L)]
                  for i in range(K * L)])
    np.linalg.cholesky(M)
    assert 0 < bound <= np.linalg.eigvalsh(M)[0] + 1e-12
