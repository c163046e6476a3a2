"""Tight tolerances (rtol 1e-10) on the GPU: the fp64-vector solve directly, and
the outer fp64 refinement around fp32-vector inner solves (hpcg_solve_refined),
both against the oracle's loops and the true residual."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import make_config  # noqa: E402

from matrix_preconditioned_pcg_amd import hpcg  # noqa: E402

TIGHT = 1e-10


def _log(msg):
    print(msg, flush=True)


def _solver(b):
    s = hpcg.Solver(b.n, b.row_ptr, b.col, b.val, batch=b.batch, levels=b.levels)
    s.set_factors(b.U, b.W, b.g)
    return s


@pytest.mark.parametrize("name", ["N1k", "N8k"])
def test_fp64_vectors_reach_1e_10(name):
    b = make_config(name)
    _log(f"direct 1e-10 {name}")
    s = _solver(b)
    res = s.solve(b.b.reshape(-1), tol=TIGHT, maxit=3000)
    assert res.status == hpcg.HPCG_OK, hpcg.hpcg_last_error(s.handle)
    sy = b.system(0)
    ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b, (sy.U, sy.W, sy.g), TIGHT, 3000)
    assert abs(res.iterations[0] - ref.iterations) <= 2, (res.iterations, ref.iterations)
    tr = oracle.true_relres(sy.row_ptr, sy.col, sy.val, sy.b, res.x[0].cpu().numpy())
    assert tr <= 1.05 * TIGHT, tr
    s.close()


@pytest.mark.parametrize("prec", [hpcg.HPCG_PREC_VEC32, hpcg.HPCG_PREC_VEC64])
@pytest.mark.parametrize("name,batch", [("N1k", None), ("N8k", None), ("N16k", None), ("tet4k", None),
                                        ("batch64x2k", 4)])
def test_refined_solve(name, batch, prec):
    b = make_config(name, batch=batch)
    _log(f"refined 1e-10 {name} prec={prec}")
    s = _solver(b)
    s.set_option(hpcg.HPCG_OPT_PRECISION, prec)
    res, outer = s.solve_refined(b.b.reshape(-1), tol=TIGHT, maxit=20000, inner_tol=1e-5, max_outer=10)
    assert res.status == hpcg.HPCG_OK, hpcg.hpcg_last_error(s.handle)
    for i in range(b.batch):
        sy = b.system(i)
        x = res.x[i].cpu().numpy()
        tr = oracle.true_relres(sy.row_ptr, sy.col, sy.val, sy.b, x)
        assert tr <= TIGHT and res.relres[i] == pytest.approx(tr, rel=1e-6, abs=1e-13), (i, tr, res.relres[i])
        xr, its, outer_ref, status, rel = oracle.pcg_refined(sy.row_ptr, sy.col, sy.val, sy.b,
                                                             (sy.U, sy.W, sy.g), TIGHT, 20000, 1e-5, 10)
        assert status == "converged"
        assert abs(outer[i] - outer_ref) <= 1, (outer[i], outer_ref)
        # both satisfy ||b - A x|| <= 1e-10 ||b||: the solutions agree to cond(A) x 1e-10
        assert np.linalg.norm(x - xr) <= 1e-5 * np.linalg.norm(xr)
        assert res.system_status[i] == hpcg.HPCG_SYS_CONVERGED
    s.close()


def test_refined_budget_and_arguments():
    b = make_config("N1k")
    s = _solver(b)
    res, outer = s.solve_refined(b.b.reshape(-1), tol=TIGHT, maxit=20000, inner_tol=1e-3, max_outer=1)
    assert res.status == hpcg.HPCG_ERR_NOT_CONVERGED and outer == [1]
    assert res.relres[0] > TIGHT
    with pytest.raises(hpcg.HPCGError):
        s.solve_refined(b.b.reshape(-1), inner_tol=1.5)
    with pytest.raises(hpcg.HPCGError):
        s.solve_refined(b.b.reshape(-1), max_outer=0)
    zero, outer = s.solve_refined(np.zeros(b.n, np.float32))
    assert zero.status == hpcg.HPCG_OK and zero.iterations == [0] and outer == [0]
    s.close()
