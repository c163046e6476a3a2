"""GPU parity of the single-vector path on seeded random shapes, through the C
ABI: 1 .. 128 leaves per system, any number of tile levels up to log2 K (none,
partial, full), 1 .. 4 systems (at most 16,384 unknowns in all), near-cubic power-of-two grids
(sides within a factor of 8) in Morton order.

Per shape: the apply on the automatic path and on the streaming path, and the
SpMV, elementwise within 1e-5 of (|M| |r|)_i (|A| |x|) and 1e-5 relative L2
against the fp64 oracle; the solve on the automatic engine or the graph engine
within 2 iterations of the oracle's count for every system, recursive residual
<= tol and true residual <= 1.05 tol."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads.generate import build_batch, random_system  # noqa: E402

from matrix_preconditioned_pcg_amd import hpcg  # noqa: E402
from test_gpu_parity import ITER_TOL, _check_apply, _check_spmv, _log, _solver  # noqa: E402


def _shapes(count, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        a = int(rng.integers(0, 8))                       # K = 2^a leaves
        n = 128 << a
        levels = 0 if a == 0 or rng.random() < 0.2 else int(rng.integers(1, a + 1))
        batch = int(rng.integers(1, max(1, min(4, 16384 // n)) + 1))
        e = n.bit_length() - 1                            # n = 2^e cells
        ex = [e // 3 + (1 if d < e % 3 else 0) for d in range(3)]   # near-cubic, then a
        i, j = rng.choice(3, size=2, replace=False)                # factor 2 moved between sides
        ex[i] += 1
        ex[j] -= 1
        rng.shuffle(ex)
        dims = tuple(1 << int(x) for x in ex)
        engine = [hpcg.HPCG_ENGINE_AUTO, hpcg.HPCG_ENGINE_GRAPH][int(rng.integers(0, 2))]
        out.append((n, levels, batch, dims, engine))
    return out


@pytest.mark.parametrize("case,shape", list(enumerate(_shapes(24, 4711))))
def test_random_shape(case, shape):
    n, levels, batch, dims, engine = shape
    _log(f"random case {case}: n={n} levels={levels} batch={batch} dims={dims} engine={engine}")
    systems = [random_system(n, seed=5000 + 10 * case + i, levels=levels, dims=dims).system(0)
               for i in range(batch)]
    b = build_batch(systems, name=f"rand{case}")
    s = _solver(b)
    rng = np.random.default_rng(case)
    r = rng.standard_normal((batch, n)).astype(np.float32)
    _check_apply(b, s, r)
    s.set_option(hpcg.HPCG_OPT_APPLY_PATH, hpcg.HPCG_APPLY_STREAMING)
    _check_apply(b, s, r)
    s.set_option(hpcg.HPCG_OPT_APPLY_PATH, hpcg.HPCG_APPLY_AUTO)
    _check_spmv(b, s, r)
    s.set_option(hpcg.HPCG_OPT_ENGINE, engine)
    res = s.solve(b.b.reshape(-1), tol=b.tol, maxit=b.maxit)
    assert res.status == hpcg.HPCG_OK, (res.status, hpcg.hpcg_last_error(s.handle))
    for i in range(batch):
        sy = b.system(i)
        ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), b.tol, b.maxit)
        assert ref.status == "converged"
        assert abs(res.iterations[i] - ref.iterations) <= ITER_TOL, (i, res.iterations[i], ref.iterations)
        assert res.relres[i] <= b.tol
        tr = oracle.true_relres(sy.row_ptr, sy.col, sy.val, sy.b, res.x[i].cpu().numpy())
        assert tr <= 1.05 * b.tol, (i, tr)
    s.close()
