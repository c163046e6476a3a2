"""Seeded generators for the five benchmark systems and their preconditioner factors.

What the pages fix and what is read into them
---------------------------------------------
* Unknowns are laid out along a space-filling (Morton / Z-order) curve and cut
  into leaves of L = 128 consecutive nodes ("Neural H-Matrix Preconditioner"
  page, section 2 "Structure and apply"; "Hierarchical Transformer
  Preconditioning" project page, Introduction, "From PCG geometry to
  hierarchical structure").  Morton codes interleave x, y, z bits with x in the
  lowest position; cells are sorted by code.
* The system matrices are the 3D stand-ins for the pages' 2D multiphase
  pressure-Poisson benchmark (Supplementary section 4, "Multiphase Poisson
  Benchmark Generation") and for the v3 tetrahedral diffusion ladder
  ("Neural H-Matrix Preconditioner" page, section 4 "Results").  The face
  coefficient of the grid systems is 1/rho_h with rho_h the harmonic mean of
  the two cell densities; a Dirichlet face at z = 0 adds 1/rho_i to the
  diagonal of a bottom cell; every other boundary face is zero-flux.
* Factors stand in for the network's output: leaf factors U_k = I + 0.05 G/sqrt(L),
  off-diagonal slab entries 0.01 G/sqrt(S L) at level S = 2^l, and a diagonal
  gate g = 0.1/diag(A) (the pages' per-node Jacobi gate, project page,
  Method, "Decoder, geometric picture, and complexity").  These scales keep
  M symmetric positive definite with a wide margin (see the oracle's Weyl bound).

Everything is drawn from numpy's PCG64 generator seeded through SeedSequence,
with separate child streams for geometry, factors and right-hand side, and is
stored in fp32 (int32 for indices): both the oracle (which promotes the fp32
values to fp64 exactly) and the HIP path read the same arrays.
"""

from __future__ import annotations

import itertools
from dataclasses import dataclass, field

import numpy as np

LEAF = 128          # L, nodes per leaf block
RANK = 32           # R, columns of every off-diagonal slab (the pages' L_s = 32)

# name -> recipe.  dims are (nx, ny, nz) in cells; seeds are the ones the
# workload descriptions name.
CONFIGS = {
    "N1k": dict(kind="grid", dims=(8, 8, 16), feature="spheres", count=3,
                seed=1024, batch=1, tol=1e-6, maxit=1000),
    "N8k": dict(kind="grid", dims=(16, 16, 32), feature="spheres", count=8,
                seed=8192, batch=1, tol=1e-6, maxit=1000),
    "N16k": dict(kind="grid", dims=(32, 32, 16), feature="seam", count=1,
                 seed=16384, batch=1, tol=1e-6, maxit=1000),
    "tet4k": dict(kind="tet", lattice=16, count=4, seed=4096, batch=1,
                  tol=1e-6, maxit=1000),
    "batch64x2k": dict(kind="grid", dims=(8, 16, 16), feature="spheres", count=3,
                       seed=2048, batch=64, tol=1e-6, maxit=1000),
}


@dataclass
class System:
    """One sparse SPD system in Morton order with its preconditioner factors."""

    n: int
    row_ptr: np.ndarray          # int32 [n+1]
    col: np.ndarray              # int32 [nnz], sorted within each row
    val: np.ndarray              # float32 [nnz]
    U: np.ndarray                # float32 [K, L, L]   leaf factors, row = node in leaf
    W: np.ndarray                # float32 [levels, K, L, R] per-level off-diagonal slabs
    g: np.ndarray                # float32 [n] diagonal gate
    b: np.ndarray                # float32 [n] right-hand side
    meta: dict = field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1])

    @property
    def K(self) -> int:
        return self.U.shape[0]

    @property
    def levels(self) -> int:
        return self.W.shape[0]


@dataclass
class Batch:
    """B independent systems of equal size, stored block-diagonally.

    The CSR uses global row and column indices (system s owns rows
    [s*n, (s+1)*n)); factors and vectors are stacked along a leading batch axis.
    """

    n: int
    batch: int
    row_ptr: np.ndarray          # int32 [B*n+1]
    col: np.ndarray              # int32 [nnz_total]
    val: np.ndarray              # float32 [nnz_total]
    U: np.ndarray                # float32 [B, K, L, L]
    W: np.ndarray                # float32 [B, levels, K, L, R]
    g: np.ndarray                # float32 [B, n]
    b: np.ndarray                # float32 [B, n]
    tol: float = 1e-6
    maxit: int = 1000
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def nnz(self) -> int:
        return int(self.row_ptr[-1])

    @property
    def K(self) -> int:
        return self.U.shape[1]

    @property
    def levels(self) -> int:
        return self.W.shape[1]

    def system(self, s: int) -> System:
        """System s with its own local CSR (row and column indices from 0)."""
        r0, r1 = s * self.n, (s + 1) * self.n
        a, z = int(self.row_ptr[r0]), int(self.row_ptr[r1])
        rp = (self.row_ptr[r0:r1 + 1] - a).astype(np.int32)
        col = (self.col[a:z] - r0).astype(np.int32)
        return System(self.n, rp, col, self.val[a:z].copy(), self.U[s], self.W[s],
                      self.g[s], self.b[s], dict(self.meta))


# ----------------------------------------------------------------------------
# ordering and sparse assembly helpers (no method arithmetic)
# ----------------------------------------------------------------------------

def morton_order(nx: int, ny: int, nz: int) -> np.ndarray:
    """perm[new] = lexicographic index (x fastest) of the cell at Morton rank new."""
    z, y, x = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx), indexing="ij")
    x, y, z = x.ravel().astype(np.int64), y.ravel().astype(np.int64), z.ravel().astype(np.int64)
    bits = max(int(nx - 1).bit_length(), int(ny - 1).bit_length(), int(nz - 1).bit_length(), 1)
    code = np.zeros_like(x)
    for bit in range(bits):
        code |= ((x >> bit) & 1) << (3 * bit)
        code |= ((y >> bit) & 1) << (3 * bit + 1)
        code |= ((z >> bit) & 1) << (3 * bit + 2)
    perm = np.argsort(code, kind="stable")
    assert len(np.unique(code)) == code.size
    return perm


def coo_to_csr(n: int, rows: np.ndarray, cols: np.ndarray, vals: np.ndarray):
    """Sum duplicate (row, col) entries in fp64 and emit a column-sorted CSR."""
    key = rows.astype(np.int64) * n + cols.astype(np.int64)
    uniq, inv = np.unique(key, return_inverse=True)
    summed = np.bincount(inv, weights=vals.astype(np.float64), minlength=uniq.size)
    r = (uniq // n).astype(np.int64)
    c = (uniq % n).astype(np.int32)
    row_ptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(np.bincount(r, minlength=n), out=row_ptr[1:])
    return row_ptr.astype(np.int32), c, summed


# ----------------------------------------------------------------------------
# 3D variable-coefficient 7-point Poisson on a Morton-ordered grid
# ----------------------------------------------------------------------------

def _density_spheres(rng, dims, count):
    nx, ny, nz = dims
    box = np.array(dims, dtype=np.float64)
    z, y, x = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx), indexing="ij")
    pts = np.stack([x.ravel(), y.ravel(), z.ravel()], axis=1) + 0.5
    rho = np.ones(nx * ny * nz)
    for _ in range(count):
        centre = rng.uniform(0.0, 1.0, 3) * box
        radius = rng.uniform(0.15, 0.30) * min(dims)
        inside = np.sum((pts - centre) ** 2, axis=1) <= radius ** 2
        rho[inside] = 100.0
    return rho


def _density_seam(rng, dims):
    nx, ny, nz = dims
    box = np.array(dims, dtype=np.float64)
    z, y, x = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx), indexing="ij")
    pts = np.stack([x.ravel(), y.ravel(), z.ravel()], axis=1) + 0.5
    normal = rng.standard_normal(3)
    normal /= np.linalg.norm(normal)
    point = rng.uniform(0.25, 0.75, 3) * box
    dist = (pts - point) @ normal
    rho = np.ones(nx * ny * nz)
    rho[np.abs(dist) <= 1.0] = 100.0
    return rho


def make_grid_poisson(dims, rho_lex: np.ndarray):
    """Assemble the Morton-ordered 7-point operator for a lexicographic density field.

    Returns (row_ptr, col, val_fp64, perm) where perm[new] = lexicographic index.
    """
    nx, ny, nz = dims
    n = nx * ny * nz
    perm = morton_order(nx, ny, nz)
    inv = np.empty(n, dtype=np.int64)
    inv[perm] = np.arange(n)
    lex = np.arange(n).reshape(nz, ny, nx)
    rows, cols, vals = [], [], []
    diag = np.zeros(n)
    for axis in range(3):  # numpy axes of lex are (z, y, x)
        a = np.take(lex, np.arange(lex.shape[axis] - 1), axis=axis).ravel()
        b = np.take(lex, np.arange(1, lex.shape[axis]), axis=axis).ravel()
        ra, rb = rho_lex[a], rho_lex[b]
        w = (ra + rb) / (2.0 * ra * rb)        # 1 / harmonic mean of the two densities
        rows += [a, b]
        cols += [b, a]
        vals += [-w, -w]
        np.add.at(diag, a, w)
        np.add.at(diag, b, w)
    bottom = lex[0].ravel()                    # z = 0 layer: Dirichlet ghost face
    diag[bottom] += 1.0 / rho_lex[bottom]
    rows.append(np.arange(n))
    cols.append(np.arange(n))
    vals.append(diag)
    r = inv[np.concatenate(rows)]
    c = inv[np.concatenate(cols)]
    row_ptr, col, v = coo_to_csr(n, r, c, np.concatenate(vals))
    return row_ptr, col, v, perm


# ----------------------------------------------------------------------------
# P1 tetrahedral diffusion on a jittered Kuhn lattice
# ----------------------------------------------------------------------------

def make_tet_diffusion(rng, lattice: int, count: int):
    """Stiffness matrix of P1 elements on a jittered lattice split into Kuhn tets.

    Returns (row_ptr, col, val_fp64, perm, info).
    """
    m = lattice
    h = 1.0
    n = m ** 3
    iz, iy, ix = np.meshgrid(np.arange(m), np.arange(m), np.arange(m), indexing="ij")
    ix, iy, iz = ix.ravel(), iy.ravel(), iz.ravel()
    pos = np.stack([ix, iy, iz], axis=1) * h + rng.uniform(-0.3 * h, 0.3 * h, (n, 3))

    def vid(x, y, z):
        return x + m * (y + m * z)

    cz, cy, cx = np.meshgrid(np.arange(m - 1), np.arange(m - 1), np.arange(m - 1), indexing="ij")
    cx, cy, cz = cx.ravel(), cy.ravel(), cz.ravel()
    unit = np.eye(3, dtype=np.int64)
    tets = []
    for order in itertools.permutations(range(3)):
        e0, e1 = unit[order[0]], unit[order[0]] + unit[order[1]]
        tets.append(np.stack([vid(cx, cy, cz),
                              vid(cx + e0[0], cy + e0[1], cz + e0[2]),
                              vid(cx + e1[0], cy + e1[1], cz + e1[2]),
                              vid(cx + 1, cy + 1, cz + 1)], axis=1))
    tets = np.concatenate(tets, axis=0)                       # [n_tet, 4]
    X = pos[tets]                                             # [n_tet, 4, 3]
    E = X[:, 1:, :] - X[:, :1, :]                             # rows are edge vectors
    det = np.linalg.det(E)
    Einv = np.linalg.inv(E)
    G = np.empty((tets.shape[0], 4, 3))
    G[:, 1:, :] = np.transpose(Einv, (0, 2, 1))               # grad of barycentric 1..3
    G[:, 0, :] = -G[:, 1:, :].sum(axis=1)
    vol = np.abs(det) / 6.0

    box = (m - 1) * h
    centroid = X.mean(axis=1)
    kappa = np.full(tets.shape[0], 100.0)
    for _ in range(count):
        centre = rng.uniform(0.2, 0.8, 3) * box
        axes = rng.uniform(0.1, 0.3, 3) * (m * h)
        inside = np.sum(((centroid - centre) / axes) ** 2, axis=1) <= 1.0
        kappa[inside] = 1.0
    Ke = (kappa * vol)[:, None, None] * np.einsum("tad,tbd->tab", G, G)

    rows = np.repeat(tets, 4, axis=1).ravel()
    cols = np.tile(tets, (1, 4)).ravel()
    vals = Ke.reshape(-1)
    dirichlet = iz == 0
    off = rows != cols
    drop = off & (dirichlet[rows] | dirichlet[cols])
    rows, cols, vals = rows[~drop], cols[~drop], vals[~drop]

    perm = np.argsort(_morton_codes(ix, iy, iz), kind="stable")
    inv = np.empty(n, dtype=np.int64)
    inv[perm] = np.arange(n)
    row_ptr, col, v = coo_to_csr(n, inv[rows], inv[cols], vals)
    info = dict(n_tets=int(tets.shape[0]), min_abs_det=float(np.abs(det).min()),
                n_dirichlet=int(dirichlet.sum()))
    return row_ptr, col, v, perm, info


def _morton_codes(x, y, z):
    x, y, z = x.astype(np.int64), y.astype(np.int64), z.astype(np.int64)
    bits = max(int(max(x.max(), y.max(), z.max())).bit_length(), 1)
    code = np.zeros_like(x)
    for bit in range(bits):
        code |= ((x >> bit) & 1) << (3 * bit)
        code |= ((y >> bit) & 1) << (3 * bit + 1)
        code |= ((z >> bit) & 1) << (3 * bit + 2)
    return code


# ----------------------------------------------------------------------------
# preconditioner factors (stand-in for the network's output)
# ----------------------------------------------------------------------------

def make_factors(rng, n: int, diag_a: np.ndarray, leaf: int = LEAF, rank: int = RANK,
                 levels: int | None = None, leaf_noise: float = 0.05,
                 tile_scale: float = 0.01, gate_scale: float = 0.1):
    """Leaf factors, per-level slabs and gate for one system.

    levels defaults to log2(n/leaf) (every tile level S = 1 .. K/2 present).
    """
    assert n % leaf == 0
    K = n // leaf
    assert K & (K - 1) == 0, "leaf count must be a power of two"
    full = K.bit_length() - 1
    levels = full if levels is None else levels
    assert 0 <= levels <= full
    U = np.eye(leaf)[None, :, :] + leaf_noise * rng.standard_normal((K, leaf, leaf)) / np.sqrt(leaf)
    W = np.empty((levels, K, leaf, rank))
    for lev in range(levels):
        S = 1 << lev
        W[lev] = tile_scale * rng.standard_normal((K, leaf, rank)) / np.sqrt(S * leaf)
    g = gate_scale / diag_a
    return U.astype(np.float32), W.astype(np.float32), g.astype(np.float32)


def make_bridge_factors(rng, K: int, levels: int, leaf: int = LEAF, rank: int = RANK,
                        bridge_scale: float = 1.0, core_scale: float = 0.005):
    """Off-diagonal factors in the pages' bridge format for one system: per-leaf
    bridges U~_k, V~_k [K, L, Ls] with entries N(0,1) bridge_scale/sqrt(L), and
    one Ls x Ls core per tile (tile order: level by level, j ascending) with
    entries N(0,1) core_scale/(sqrt(Ls) 2^l) at level l, so that every level's
    tiles have about the same operator norm."""
    Ub = bridge_scale * rng.standard_normal((K, leaf, rank)) / np.sqrt(leaf)
    Vb = bridge_scale * rng.standard_normal((K, leaf, rank)) / np.sqrt(leaf)
    cores = [core_scale * rng.standard_normal((rank, rank)) / (np.sqrt(rank) * (1 << lev))
             for lev in range(levels) for _j in range(K >> (lev + 1))]
    Bc = np.stack(cores) if cores else np.zeros((0, rank, rank))
    return Ub.astype(np.float32), Vb.astype(np.float32), Bc.astype(np.float32)


def bridge_factors_for(batch: "Batch", seed: int = 7):
    """Bridge-format off-diagonal factors for every system of a batch (its leaf
    factors and gate stay as they are): Ub, Vb [B, K, L, Ls], Bc [B, M_H, Ls, Ls]."""
    out = []
    for s in range(batch.batch):
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, s, batch.n])))
        out.append(make_bridge_factors(rng, batch.K, batch.levels))
    return tuple(np.stack([o[i] for o in out]) for i in range(3))


def _diag_of(row_ptr, col, val):
    n = row_ptr.size - 1
    rows = np.repeat(np.arange(n), np.diff(row_ptr))
    d = np.zeros(n)
    on = rows == col
    d[rows[on]] = val[on]
    return d


def _one_system(recipe: dict, seed: int) -> System:
    ss = np.random.SeedSequence(seed)
    geo_ss, fac_ss, rhs_ss = ss.spawn(3)
    geo, fac, rhs = (np.random.Generator(np.random.PCG64(s)) for s in (geo_ss, fac_ss, rhs_ss))
    meta = dict(seed=seed)
    if recipe["kind"] == "grid":
        dims = recipe["dims"]
        if recipe["feature"] == "spheres":
            rho = _density_spheres(geo, dims, recipe["count"])
        else:
            rho = _density_seam(geo, dims)
        row_ptr, col, v, perm = make_grid_poisson(dims, rho)
        meta.update(dims=dims, heavy_fraction=float(np.mean(rho > 1.0)))
    else:
        row_ptr, col, v, perm, info = make_tet_diffusion(geo, recipe["lattice"], recipe["count"])
        meta.update(info)
    val = v.astype(np.float32)
    n = row_ptr.size - 1
    diag = _diag_of(row_ptr, col, val.astype(np.float64))
    U, W, g = make_factors(fac, n, diag)
    b = rhs.standard_normal(n).astype(np.float32)
    return System(n, row_ptr, col, val, U, W, g, b, meta)


def build_batch(systems: list[System], tol=1e-6, maxit=1000, name="") -> Batch:
    """Stack equally sized systems into one block-diagonal batch."""
    n = systems[0].n
    assert all(s.n == n for s in systems)
    rps, cols, vals = [np.zeros(1, dtype=np.int64)], [], []
    base = 0
    for i, s in enumerate(systems):
        rps.append(s.row_ptr[1:].astype(np.int64) + base)
        cols.append(s.col.astype(np.int64) + i * n)
        vals.append(s.val)
        base += s.nnz
    assert base < 2 ** 31
    return Batch(
        n=n, batch=len(systems),
        row_ptr=np.concatenate(rps).astype(np.int32),
        col=np.concatenate(cols).astype(np.int32),
        val=np.concatenate(vals).astype(np.float32),
        U=np.stack([s.U for s in systems]), W=np.stack([s.W for s in systems]),
        g=np.stack([s.g for s in systems]), b=np.stack([s.b for s in systems]),
        tol=tol, maxit=maxit, name=name, meta=dict(systems[0].meta),
    )


def make_config(name: str, batch: int | None = None) -> Batch:
    """Build one of the named workloads.  batch overrides the batch size
    (the batched workload's systems are seeded seed*100 + s, s = 0..B-1)."""
    recipe = CONFIGS[name]
    B = recipe["batch"] if batch is None else batch
    if recipe["batch"] == 1 and B == 1:
        systems = [_one_system(recipe, recipe["seed"])]
    else:
        systems = [_one_system(recipe, recipe["seed"] * 100 + s) for s in range(B)]
    return build_batch(systems, recipe["tol"], recipe["maxit"], name)


def random_system(n: int, seed: int, leaf: int = LEAF, rank: int = RANK,
                  levels: int | None = None, dims=None) -> Batch:
    """Small grid system for tests: a dims grid (default: n cells as 4 x 4 x n/16)
    with 2 spheres, and factors at the given leaf size and rank."""
    if dims is None:
        dims = (4, 4, n // 16)
    assert dims[0] * dims[1] * dims[2] == n
    ss = np.random.SeedSequence(seed)
    geo_ss, fac_ss, rhs_ss = ss.spawn(3)
    geo, fac, rhs = (np.random.Generator(np.random.PCG64(s)) for s in (geo_ss, fac_ss, rhs_ss))
    rho = _density_spheres(geo, dims, 2)
    row_ptr, col, v, _ = make_grid_poisson(dims, rho)
    val = v.astype(np.float32)
    diag = _diag_of(row_ptr, col, val.astype(np.float64))
    U, W, g = make_factors(fac, n, diag, leaf=leaf, rank=rank, levels=levels)
    b = rhs.standard_normal(n).astype(np.float32)
    s = System(n, row_ptr, col, val, U, W, g, b, dict(seed=seed, dims=dims))
    return build_batch([s], name=f"random{n}")
