"""GPU parity at the largest partitions the library takes.

A system holds at most eight tile levels.  n = 32,768 on a 32 x 32 x 32 grid
is the full eight-level hierarchy of 256 leaves: every one of the device's 256
compute units holds a leaf, so the single-pass apply and the register-resident
solve run at their widest grid and with their largest partner stage (255 rows
of restrictions).  n = 65,536 (a 32 x 32 x 64 grid, 512 leaves, eight levels:
a partial hierarchy) has more leaves than compute units, so the apply takes
the streaming path and the solve the graph engine.  Bars as in
test_gpu_parity: apply and SpMV elementwise 1e-5 of |M| |r| (|A| |x|) and
relative L2 1e-5; x after 40 steps to 1e-9 of the oracle's; the full solve
within 2 iterations of the oracle's count, true residual <= 1.05 tol.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads.generate import random_system  # noqa: E402

from matrix_preconditioned_pcg_amd import hpcg  # noqa: E402
from test_gpu_parity import ITER_TOL, _check_apply, _check_spmv, _log, _solver  # noqa: E402

SHAPES = {32768: (32, 32, 32), 65536: (32, 32, 64)}


@pytest.fixture(scope="module")
def system():
    cache = {}

    def get(n):
        if n not in cache:
            cache[n] = random_system(n, seed=900 + n // 32768, levels=8, dims=SHAPES[n])
        return cache[n]
    return get


@pytest.mark.parametrize("n", [32768, 65536])
def test_max_apply_spmv(system, n):
    batch = system(n)
    _log(f"max-size apply / SpMV n={n} levels={batch.levels}")
    s = _solver(batch)
    rng = np.random.default_rng(n + 3)
    r = rng.standard_normal((1, n)).astype(np.float32)
    _check_apply(batch, s, r)
    want = hpcg.HPCG_APPLY_FUSED if n // 128 <= 256 else hpcg.HPCG_APPLY_STREAMING
    assert hpcg.hpcg_last_apply_path(s.handle) == want
    s.set_option(hpcg.HPCG_OPT_APPLY_PATH, hpcg.HPCG_APPLY_STREAMING)
    _check_apply(batch, s, r)
    _check_spmv(batch, s, r)
    s.close()


@pytest.mark.parametrize("n,engine", [(32768, hpcg.HPCG_ENGINE_PERSISTENT), (32768, hpcg.HPCG_ENGINE_GRAPH),
                                      (65536, hpcg.HPCG_ENGINE_AUTO)])
def test_max_truncated_solve(system, n, engine):
    batch = system(n)
    steps = 40
    _log(f"max-size truncated solve n={n} engine={engine}")
    s = _solver(batch)
    s.set_option(hpcg.HPCG_OPT_ENGINE, engine)
    res = s.solve(batch.b.reshape(-1), tol=batch.tol, maxit=steps)
    assert res.status == hpcg.HPCG_ERR_NOT_CONVERGED, (res.status, hpcg.hpcg_last_error(s.handle))
    if engine == hpcg.HPCG_ENGINE_AUTO:
        assert s.last_engine == hpcg.HPCG_ENGINE_GRAPH   # more leaves than compute units
    else:
        assert s.last_engine == engine
    _log(f"  launch grid, LDS: {hpcg.hpcg_last_launch_info(s.handle)}")
    sy = batch.system(0)
    ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), batch.tol, steps)
    assert ref.status == "not_converged" and res.iterations[0] == steps
    x = res.x[0].cpu().numpy()
    scale = np.abs(ref.x).max()
    assert np.abs(x - ref.x).max() <= 1e-9 * scale, np.abs(x - ref.x).max() / scale
    assert abs(res.relres[0] - ref.relres) <= 1e-9 * ref.relres, (res.relres[0], ref.relres)
    s.close()


def test_max_solve_parity(system):
    # both vector precisions on the resident engine at its widest (256
    # workgroups, one per CU, with the 255-row partner stage of W^T r in LDS)
    batch = system(32768)
    _log("max-size solve n=32768 (oracle solve takes ~15 s)")
    sy = batch.system(0)
    ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), batch.tol, batch.maxit)
    assert ref.status == "converged"
    s = _solver(batch)
    for prec in (hpcg.HPCG_PREC_VEC64, hpcg.HPCG_PREC_VEC32):
        s.set_option(hpcg.HPCG_OPT_PRECISION, prec)
        res = s.solve(batch.b.reshape(-1), tol=batch.tol, maxit=batch.maxit)
        assert res.status == hpcg.HPCG_OK, (res.status, hpcg.hpcg_last_error(s.handle))
        grid, lds = hpcg.hpcg_last_launch_info(s.handle)
        _log(f"  precision {prec}: engine {s.last_engine} (grid {grid}, LDS {lds}), "
             f"{res.iterations[0]} iterations (oracle {ref.iterations})")
        assert s.last_engine == hpcg.HPCG_ENGINE_PERSISTENT and grid == 256
        assert abs(res.iterations[0] - ref.iterations) <= ITER_TOL, (res.iterations[0], ref.iterations)
        assert res.relres[0] <= batch.tol
        tr = oracle.true_relres(sy.row_ptr, sy.col, sy.val, sy.b, res.x[0].cpu().numpy())
        assert tr <= 1.05 * batch.tol, tr
    s.close()
