"""Weak-admissibility H-matrix preconditioner M, in plain fp64 numpy.

TEST INFRASTRUCTURE ONLY (see the package docstring): imported by tests, the
smoke check and the benchmark's CPU baseline, never by the product path.

Definitions followed
--------------------
Partition.  Unknowns are cut into K = N/L contiguous leaves of L nodes; the
weak-admissibility partition with eta = 1 holds the K diagonal leaf blocks and
off-diagonal tiles spanning S x S leaves with S = 2^l, l = 0, 1, ...; their
count is K/2 + K/4 + ... + 1 = K - 1 ("Hierarchical Transformer Preconditioning
for Interactive Physics Simulation", Supplementary section 2, "Apply-path
tensor layout"; project page, Method, "Notation and pipeline").  Read as a
binary tree: tile j of level l couples the row leaves [2jS, 2jS+S) with the
column leaves [2jS+S, 2jS+2S).

Blocks.  Diagonal block k is the PSD product U_k U_k^T ("A Neural
Hierarchical-Matrix Preconditioner for Real-Time GPU Solves", section 2,
"Network"; project page, Method, "Diagonal and off-diagonal attention
stacks").  The upper tile (l, j) is U_{l,j} V_{l,j}^T with rank-32 factors and
the lower tile mirrors it as V_{l,j} U_{l,j}^T, which makes M symmetric
("A Neural Hierarchical-Matrix Preconditioner", section 2, "SPD by
construction").  Per-tile factors of SL x 32 with the identity as the coupling
core are the reading of the pages' bridge-and-core chain taken here: U_{l,j}
stacks the slabs W_l[k] of the row leaves and V_{l,j} those of the column
leaves, so every leaf carries exactly one L x 32 slab per level.  A per-node
gate adds diag(g) (project page, Method, "Decoder, geometric picture, and
complexity").

Apply.  M is never assembled: a diagonal stage applies each leaf block to its
slice of r, then each tile applies U (V^T r_C) to its row strip and its mirror
V (U^T r_R) to its column strip, then the gate is added ("Hierarchical
Transformer Preconditioning", section 5 "Preconditioner Application",
stages (i) and (ii), eqs. (2)-(5) with the coupling core equal to identity).
"""

from __future__ import annotations

import numpy as np


def tiles(K: int, levels: int):
    """Tiles of the partition as (level, j, row_leaves, col_leaves) ranges."""
    assert K >= 1 and K & (K - 1) == 0, "leaf count must be a power of two"
    assert 0 <= levels <= K.bit_length() - 1
    out = []
    for lev in range(levels):
        S = 1 << lev
        for j in range(K // (2 * S)):
            out.append((lev, j, range(2 * j * S, 2 * j * S + S),
                        range(2 * j * S + S, 2 * j * S + 2 * S)))
    return out


def tile_count(K: int, levels: int | None = None) -> int:
    """Number of unique off-diagonal tiles (the pages' M_H)."""
    if levels is None:
        levels = K.bit_length() - 1
    return len(tiles(K, levels))


def apply_M(U, W, g, r, dtype=np.float64):
    """y = M r for one system, structured (M is never formed).

    U: [K, L, L] leaf factors; W: [levels, K, L, R] per-level slabs;
    g: [N] gate; r: [N].  Everything is promoted to fp64 (or to `dtype`, e.g.
    np.longdouble for an extended-precision reference run).
    """
    U = np.asarray(U, dtype=dtype)
    W = np.asarray(W, dtype=dtype)
    g = np.asarray(g, dtype=dtype)
    r = np.asarray(r, dtype=dtype)
    K, L, _ = U.shape
    levels = W.shape[0]
    R = W.shape[3] if levels else 0
    assert r.shape == (K * L,)
    y = np.zeros_like(r)
    # (i) diagonal stage: y_k = U_k (U_k^T r_k)
    for k in range(K):
        rk = r[k * L:(k + 1) * L]
        y[k * L:(k + 1) * L] += U[k] @ (U[k].T @ rk)
    # (ii) off-diagonal stage, one tile at a time, upper tile and its mirror
    for lev, _j, rows, cols in tiles(K, levels):
        Ut = W[lev, rows.start:rows.stop].reshape(-1, R)      # SL x R
        Vt = W[lev, cols.start:cols.stop].reshape(-1, R)      # SL x R
        rs = slice(rows.start * L, rows.stop * L)
        cs = slice(cols.start * L, cols.stop * L)
        y[rs] += Ut @ (Vt.T @ r[cs])
        y[cs] += Vt @ (Ut.T @ r[rs])
    # gate
    y += g * r
    return y


def apply_M_batch(U, W, g, r):
    """apply_M over a leading batch axis: U [B,K,L,L], W [B,lev,K,L,R], g/r [B,N]."""
    return np.stack([apply_M(U[s], W[s], g[s], r[s]) for s in range(U.shape[0])])


def apply_M_block(U, W, g, R):
    """Y = M R for a block R of shape [N, nrhs]: M applied to every column
    (the probe-block product of the pages' training objective, project page,
    "Cosine Hutchinson Probe Loss")."""
    R = np.asarray(R, dtype=np.float64)
    return np.stack([apply_M(U, W, g, R[:, j]) for j in range(R.shape[1])], axis=1)


def dense_M_entry(U, W, g, i: int, j: int) -> float:
    """One entry M[i, j], written from the partition's geometry rather than its tiles.

    Nodes i and j in the same leaf meet in that leaf's block.  Otherwise their
    leaves k_i != k_j first split at the tree level l = msb(k_i XOR k_j): that is
    the only tile holding (i, j), and whichever of the two is in the row half,
    the entry is the dot product of node i's and node j's rows of their level-l
    slabs.  The gate sits on the diagonal.
    """
    U = np.asarray(U, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    L = U.shape[1]
    ki, kj = i // L, j // L
    if ki == kj:
        v = float(U[ki, i % L] @ U[kj, j % L])
    else:
        lev = (ki ^ kj).bit_length() - 1
        v = float(W[lev, ki, i % L] @ W[lev, kj, j % L]) if lev < W.shape[0] else 0.0
    if i == j:
        v += float(g[i])
    return v


def dense_M(U, W, g):
    """Dense M assembled as blockdiag(U_k U_k^T) + diag(g) + sum_l W_l Pi_l W_l^T.

    W_l = blockdiag_k(W_l[k]) is N x RK and Pi_l holds an R x R identity at leaf
    pair (k, k') exactly when k >> l and k' >> l are the two halves of one tile
    ((k >> l) == (k' >> l) XOR 1).  For tiny inputs only.
    """
    U = np.asarray(U, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    K, L, _ = U.shape
    N = K * L
    M = np.zeros((N, N))
    for k in range(K):
        M[k * L:(k + 1) * L, k * L:(k + 1) * L] = U[k] @ U[k].T
    M += np.diag(np.asarray(g, dtype=np.float64))
    for lev in range(W.shape[0]):
        R = W.shape[3]
        Wl = np.zeros((N, R * K))
        for k in range(K):
            Wl[k * L:(k + 1) * L, k * R:(k + 1) * R] = W[lev, k]
        Pi = np.zeros((R * K, R * K))
        for k in range(K):
            for kp in range(K):
                if (k >> lev) == ((kp >> lev) ^ 1):
                    Pi[k * R:(k + 1) * R, kp * R:(kp + 1) * R] = np.eye(R)
        M += Wl @ Pi @ Wl.T
    return M


def weyl_lower_bound(U, W, g) -> float:
    """A lower bound on lambda_min(M) that needs no dense M.

    M = D + G + sum_l O_l with D = blockdiag(U_k U_k^T), G = diag(g) and O_l the
    level-l tiles with their mirrors.  At a fixed level every leaf lies in
    exactly one tile, so O_l is block-diagonal with blocks [[0, U V^T], [V U^T, 0]]
    whose spectral norm is ||U V^T||_2.  Weyl's inequality then gives
    lambda_min(M) >= min_k sigma_min(U_k)^2 + min(g) - sum_l max_j ||U_{l,j} V_{l,j}^T||_2.
    A positive value certifies that M is SPD.
    """
    U = np.asarray(U, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    K, L, _ = U.shape
    smin = min(np.linalg.svd(U[k], compute_uv=False)[-1] for k in range(K))
    bound = smin ** 2 + float(np.min(g))
    levels = W.shape[0]
    R = W.shape[3] if levels else 0
    for lev in range(levels):
        worst = 0.0
        for _l, _j, rows, cols in tiles(K, levels):
            if _l != lev:
                continue
            Ut = W[lev, rows.start:rows.stop].reshape(-1, R)
            Vt = W[lev, cols.start:cols.stop].reshape(-1, R)
            # ||U V^T|| = ||R_U R_V^T|| with U = Q_U R_U, V = Q_V R_V
            ru = np.linalg.qr(Ut, mode="r")
            rv = np.linalg.qr(Vt, mode="r")
            worst = max(worst, np.linalg.norm(ru @ rv.T, 2))
        bound -= worst
    return float(bound)
