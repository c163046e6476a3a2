"""GPU parity with factors in the pages' bridge format (per-leaf bridges U~_k,
V~_k and per-tile cores B_m), loaded through hpcg_set_factors_bridge and
expanded on the device.  The references are the oracle's bridge apply (the
pages' four stages in fp64) and its PCG with that apply.  Bars as for the
per-tile format: 1e-5 relative per apply, iteration count within 2, true
residual within 1.05 tol."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import make_config  # noqa: E402
from workloads.generate import bridge_factors_for  # noqa: E402

from matrix_preconditioned_pcg_amd import hpcg  # noqa: E402

TOL = 1e-5


def _log(msg):
    print(msg, flush=True)


def _setup(name, batch=None):
    b = make_config(name, batch=batch)
    Ub, Vb, Bc = bridge_factors_for(b)
    s = hpcg.Solver(b.n, b.row_ptr, b.col, b.val, batch=b.batch, levels=b.levels)
    s.set_factors_bridge(b.U, Ub, Vb, Bc, b.g)
    return b, (Ub, Vb, Bc), s


@pytest.mark.parametrize("name,batch", [("N1k", None), ("N8k", None), ("N16k", None), ("tet4k", None),
                                        ("batch64x2k", 4)])
def test_bridge_apply_parity(name, batch):
    b, (Ub, Vb, Bc), s = _setup(name, batch)
    _log(f"bridge apply {name}")
    r = np.random.default_rng(17).standard_normal((b.batch, b.n)).astype(np.float32)
    y = s.apply_M(r.reshape(-1)).cpu().numpy().astype(np.float64).reshape(b.batch, b.n)
    for i in range(b.batch):
        ref = oracle.apply_M_bridge(b.U[i], Ub[i], Vb[i], Bc[i], b.g[i], r[i])
        mag = oracle.apply_M_bridge(np.abs(b.U[i]), np.abs(Ub[i]), np.abs(Vb[i]), np.abs(Bc[i]), np.abs(b.g[i]),
                                    np.abs(r[i]))
        rel = np.linalg.norm(y[i] - ref) / np.linalg.norm(ref)
        assert rel <= TOL, (i, rel)
        assert not (np.abs(y[i] - ref) > TOL * mag + 1e-30).any()
    s.close()


@pytest.mark.parametrize("engine", [hpcg.HPCG_ENGINE_AUTO, hpcg.HPCG_ENGINE_GRAPH])
@pytest.mark.parametrize("name", ["N1k", "N8k", "N16k"])
def test_bridge_solve_parity(name, engine):
    b, (Ub, Vb, Bc), s = _setup(name)
    _log(f"bridge solve {name} engine={engine}")
    s.set_option(hpcg.HPCG_OPT_ENGINE, engine)
    res = s.solve(b.b.reshape(-1), tol=b.tol, maxit=b.maxit)
    assert res.status == hpcg.HPCG_OK, (res.status, hpcg.hpcg_last_error(s.handle))
    sy = b.system(0)
    ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b,
                     lambda v: oracle.apply_M_bridge(b.U[0], Ub[0], Vb[0], Bc[0], b.g[0], v), b.tol, b.maxit)
    assert ref.status == "converged"
    assert abs(res.iterations[0] - ref.iterations) <= 2, (res.iterations, ref.iterations)
    tr = oracle.true_relres(sy.row_ptr, sy.col, sy.val, sy.b, res.x[0].cpu().numpy())
    assert res.relres[0] <= b.tol and tr <= 1.05 * b.tol, (res.relres, tr)
    s.close()


def test_bridge_truncated_solve_matches_oracle():
    b, (Ub, Vb, Bc), s = _setup("N8k")
    _log("bridge truncated solve N8k")
    res = s.solve(b.b.reshape(-1), tol=b.tol, maxit=30)
    sy = b.system(0)
    ref = oracle.pcg(sy.row_ptr, sy.col, sy.val, sy.b,
                     lambda v: oracle.apply_M_bridge(b.U[0], Ub[0], Vb[0], Bc[0], b.g[0], v), b.tol, 30)
    x = res.x[0].cpu().numpy()
    # the device slabs U~ B are rounded to fp32 once, so the operator itself
    # differs from the fp64 one by ~1e-7 relative
    assert np.abs(x - ref.x).max() <= 1e-5 * np.abs(ref.x).max()
    assert abs(res.relres[0] - ref.relres) <= 1e-5 * ref.relres
    s.close()


def test_bridge_block_apply():
    b, (Ub, Vb, Bc), s = _setup("N8k")
    _log("bridge block apply N8k")
    R = np.random.default_rng(18).standard_normal((b.n, 32)).astype(np.float32)
    Y = s.apply_M_block(R.reshape(-1), 32).cpu().numpy().astype(np.float64).reshape(b.n, 32)
    for j in (0, 9, 31):
        ref = oracle.apply_M_bridge(b.U[0], Ub[0], Vb[0], Bc[0], b.g[0], R[:, j])
        assert np.linalg.norm(Y[:, j] - ref) <= TOL * np.linalg.norm(ref)
    s.close()
