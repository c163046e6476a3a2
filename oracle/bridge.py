"""The pages' own off-diagonal factor format: per-leaf bridges and tile cores.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Hierarchical Transformer Preconditioning for Interactive Physics Simulation",
section 4.4 / project page "Decoder, geometric picture, and complexity": the
decoder emits, besides the leaf factors F_k (block F_k F_k^T), two per-leaf
bridges U~_k, V~_k of L x L_s between node and tile resolution, and per tile m
two L_s x L_s factors U_m, V_m whose product B_m = U_m V_m^T couples the tile's
row strip R_m with its column strip J_m; all factors pack into one tensor of
width P = K L^2 + M_H L_s^2 + 2 N L_s + N (Supplementary section 2, Table 3).
The apply (section 5, "Preconditioner Application", eqs. (2)-(5)):

    restriction          u^_k = U~_k^T r_k,   v^_k = V~_k^T r_k
    strip aggregation    s^r_m = sum_{k in R_m} u^_k,   s^c_m = sum_{k in C_m} v^_k
    coarse coupling      t^c_m = B_m^T s^r_m,  t^r_m = B_m s^c_m
    prolongation         dy_k = U~_k sum_{m: k in R_m} t^r_m + V~_k sum_{m: k in C_m} t^c_m

so tile m contributes U~_R B_m V~_C^T to M and its mirror V~_C B_m^T U~_R^T.
Here the cores are given directly as B_m (the product the apply uses), the
tiles are those of the binary partition in `hmatrix.tiles` in that order, and
the gate is the additive diag(g) of the per-tile format.

Equivalence used by the library: with slabs W_l[k] = U~_k B_m for a leaf in
the row half of its level-l tile m, and W_l[k] = V~_k for a leaf in the
column half, the per-tile apply (identity core) gives the same M.
"""

from __future__ import annotations

import numpy as np

from .hmatrix import tiles


def core_count(K: int, levels: int) -> int:
    return len(tiles(K, levels))


def apply_M_bridge(F, Ub, Vb, Bc, g, r, dtype=np.float64):
    """y = M r in the bridge format.  F [K, L, L], Ub/Vb [K, L, Ls], Bc [M_H, Ls, Ls]
    (tile order of hmatrix.tiles), g and r [N]."""
    F, Ub, Vb, Bc = (np.asarray(a, dtype=dtype) for a in (F, Ub, Vb, Bc))
    g = np.asarray(g, dtype=dtype)
    r = np.asarray(r, dtype=dtype)
    K, L, _ = F.shape
    levels = 0
    while len(tiles(K, levels)) < Bc.shape[0]:
        levels += 1
    assert len(tiles(K, levels)) == Bc.shape[0]
    rk = r.reshape(K, L)
    # (i) diagonal stage
    y = np.einsum("kij,kj->ki", F, np.einsum("kji,kj->ki", F, rk))
    # (ii) restriction
    u_hat = np.einsum("kji,kj->ki", Ub, rk)          # [K, Ls]
    v_hat = np.einsum("kji,kj->ki", Vb, rk)
    tr = np.zeros_like(u_hat)                        # sum over tiles with k in R_m of t^r_m
    tc = np.zeros_like(v_hat)
    for m, (_lev, _j, rows, cols) in enumerate(tiles(K, levels)):
        s_r = u_hat[rows.start:rows.stop].sum(axis=0)    # strip aggregation
        s_c = v_hat[cols.start:cols.stop].sum(axis=0)
        t_c = Bc[m].T @ s_r                              # coarse coupling
        t_r = Bc[m] @ s_c
        tr[rows.start:rows.stop] += t_r
        tc[cols.start:cols.stop] += t_c
    # prolongation
    y += np.einsum("kij,kj->ki", Ub, tr) + np.einsum("kij,kj->ki", Vb, tc)
    return y.reshape(-1) + g * r


def dense_M_bridge_entry(F, Ub, Vb, Bc, g, i: int, j: int) -> float:
    """M[i, j] from the geometry: same leaf -> F F^T; else the one tile holding
    (i, j) at level l = msb(k_i XOR k_j), row-half leaf uses U~ and B, column-half
    leaf uses V~."""
    F, Ub, Vb, Bc = (np.asarray(a, dtype=np.float64) for a in (F, Ub, Vb, Bc))
    K, L, _ = F.shape
    ki, kj = i // L, j // L
    if ki == kj:
        v = float(F[ki, i % L] @ F[kj, j % L])
    else:
        lev = (ki ^ kj).bit_length() - 1
        m = sum(K >> (l + 1) for l in range(lev)) + (ki >> (lev + 1))
        if m >= Bc.shape[0] or (K >> (lev + 1)) == 0:
            v = 0.0
        elif (ki >> lev) & 1 == 0:        # i in the row half
            v = float(Ub[ki, i % L] @ Bc[m] @ Vb[kj, j % L])
        else:                              # i in the column half
            v = float(Vb[ki, i % L] @ Bc[m].T @ Ub[kj, j % L])
    if i == j:
        v += float(g[i])
    return v


def to_slabs(Ub, Vb, Bc, K: int, levels: int):
    """Per-level slabs W [levels, K, L, Ls] of the per-tile format that give the
    same M: W_l[k] = U~_k B_m (row half of tile m) or V~_k (column half)."""
    Ub, Vb, Bc = (np.asarray(a, dtype=np.float64) for a in (Ub, Vb, Bc))
    L, Ls = Ub.shape[1], Ub.shape[2]
    W = np.zeros((levels, K, L, Ls))
    for m, (lev, _j, rows, cols) in enumerate(tiles(K, levels)):
        for k in rows:
            W[lev, k] = Ub[k] @ Bc[m]
        for k in cols:
            W[lev, k] = Vb[k]
    return W


def pack_bridge(F, Ub, Vb, Bc, g) -> np.ndarray:
    """One flat tensor in the order F, cores, U~, V~, gate: K L^2 + M_H Ls^2 + 2 N Ls + N."""
    return np.concatenate([np.asarray(a, dtype=np.float32).reshape(-1) for a in (F, Bc, Ub, Vb, g)])


def weyl_lower_bound_bridge(F, Ub, Vb, Bc, g) -> float:
    """lambda_min(M) >= min_k sigma_min(F_k)^2 + min(g) - sum_l max_m ||U~_R B_m V~_C^T||_2
    (per level the tiles are disjoint diagonal blocks of the off-diagonal part)."""
    F, Ub, Vb, Bc = (np.asarray(a, dtype=np.float64) for a in (F, Ub, Vb, Bc))
    K, L, _ = F.shape
    Ls = Ub.shape[2]
    levels = 0
    while len(tiles(K, levels)) < Bc.shape[0]:
        levels += 1
    bound = min(np.linalg.svd(F[k], compute_uv=False)[-1] for k in range(K)) ** 2 + float(np.min(g))
    worst = [0.0] * levels
    for m, (lev, _j, rows, cols) in enumerate(tiles(K, levels)):
        ur = np.linalg.qr(Ub[rows.start:rows.stop].reshape(-1, Ls), mode="r")
        vc = np.linalg.qr(Vb[cols.start:cols.stop].reshape(-1, Ls), mode="r")
        worst[lev] = max(worst[lev], np.linalg.norm(ur @ Bc[m] @ vc.T, 2))
    return float(bound - sum(worst))
