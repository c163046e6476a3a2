"""GPU parity with factors in the pages' bridge format (per-leaf bridges U~_k,
V~_k and per-tile cores B_m), loaded through hpcg_set_factors_bridge: the
native bridge apply (the default apply path for such factors), the slab
paths and the solve engines on the device expansion.  The references are the
oracle's bridge apply (the pages' four stages in fp64) and its PCG with that
apply.  Bars as for the per-tile format: 1e-5 relative per apply and
elementwise against |M| |r|, iteration count within 2, true residual within
1.05 tol."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from workloads import make_config  # noqa: E402
from workloads.generate import bridge_factors_for, build_batch, random_system  # noqa: E402

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
    assert hpcg.hpcg_last_apply_path(s.handle) == hpcg.HPCG_APPLY_BRIDGE
    s.close()


def _check_bridge_apply(b, fac, y, r):
    Ub, Vb, Bc = fac
    for i in range(b.batch):
        ref = oracle.apply_M_bridge(b.U[i], Ub[i], Vb[i], Bc[i], b.g[i], r[i])
        mag = oracle.apply_M_bridge(np.abs(b.U[i]), np.abs(Ub[i]), np.abs(Vb[i]), np.abs(Bc[i]), np.abs(b.g[i]),
                                    np.abs(r[i]))
        assert np.linalg.norm(y[i] - ref) <= TOL * np.linalg.norm(ref), i
        assert not (np.abs(y[i] - ref) > TOL * mag + 1e-30).any(), i


@pytest.mark.parametrize("path", [hpcg.HPCG_APPLY_BRIDGE, hpcg.HPCG_APPLY_FUSED, hpcg.HPCG_APPLY_STREAMING])
@pytest.mark.parametrize("name,batch", [("N8k", None), ("N16k", None), ("batch64x2k", None), ("batch64x2k", 17)])
def test_bridge_apply_paths(name, batch, path):
    # every apply path on bridge-format factors: the native one (one or two
    # workgroups per leaf; the full batch in launches of whole systems, the
    # ragged 17-system batch in one launch of 16 and one of 1) and the slab
    # paths on the device expansion
    b, fac, s = _setup(name, batch)
    _log(f"bridge apply path={path} {name} batch={b.batch}")
    s.set_option(hpcg.HPCG_OPT_APPLY_PATH, path)
    r = np.random.default_rng(23).standard_normal((b.batch, b.n)).astype(np.float32)
    y = s.apply_M(r.reshape(-1)).cpu().numpy().astype(np.float64).reshape(b.batch, b.n)
    assert hpcg.hpcg_last_apply_path(s.handle) == path
    _check_bridge_apply(b, fac, y, r)
    assert s.apply_status() == hpcg.HPCG_OK
    s.close()


@pytest.mark.parametrize("n,levels,batch", [(256, 1, 1), (256, 1, 3), (1024, 2, 1), (1024, 3, 2), (2048, 4, 3),
                                            (4096, 2, 1)])
def test_bridge_apply_small_and_partial(n, levels, batch):
    # two leaves (one level), hierarchies with fewer levels than log2 K, batches
    systems = [random_system(n, seed=500 + i, levels=levels).system(0) for i in range(batch)]
    b = build_batch(systems, name=f"bridge_small{n}_{levels}_{batch}")
    _log(f"bridge apply small n={n} levels={levels} batch={batch}")
    fac = bridge_factors_for(b)
    s = hpcg.Solver(b.n, b.row_ptr, b.col, b.val, batch=b.batch, levels=b.levels)
    s.set_factors_bridge(b.U, *fac, b.g)
    r = np.random.default_rng(29).standard_normal((b.batch, b.n)).astype(np.float32)
    y = s.apply_M(r.reshape(-1)).cpu().numpy().astype(np.float64).reshape(b.batch, b.n)
    assert hpcg.hpcg_last_apply_path(s.handle) == hpcg.HPCG_APPLY_BRIDGE
    _check_bridge_apply(b, fac, y, r)
    s.close()


def test_bridge_apply_replays_and_path_switches():
    # graph replays of the native bridge apply interleaved with the slab
    # single pass on the same handle, eager calls in between: every call
    # bit-identical to the first of its path (the flagged words' epochs stay
    # consistent across the two kernels)
    b = make_config("N8k")
    _log("bridge apply replays N8k")
    fac = bridge_factors_for(b)
    stream = torch.cuda.Stream()
    s = hpcg.Solver(b.n, b.row_ptr, b.col, b.val, batch=1, levels=b.levels, stream=stream)
    s.set_factors_bridge(b.U, *fac, b.g)
    r = torch.as_tensor(np.random.default_rng(31).standard_normal(b.n).astype(np.float32)).cuda()
    torch.cuda.synchronize()
    ys = {}
    for path in (hpcg.HPCG_APPLY_BRIDGE, hpcg.HPCG_APPLY_FUSED):
        s.set_option(hpcg.HPCG_OPT_APPLY_PATH, path)
        y0 = s.apply_M(r)
        torch.cuda.synchronize()
        ys[path] = y0.clone()
    for path in (hpcg.HPCG_APPLY_BRIDGE, hpcg.HPCG_APPLY_FUSED, hpcg.HPCG_APPLY_BRIDGE):
        s.set_option(hpcg.HPCG_OPT_APPLY_PATH, path)
        y = torch.empty_like(r)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(5):
                hpcg.hpcg_apply_M(s.handle, s.part, r, y)
        for _ in range(4):
            y.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, ys[path]), path
            other = hpcg.HPCG_APPLY_FUSED if path == hpcg.HPCG_APPLY_BRIDGE else hpcg.HPCG_APPLY_BRIDGE
            s.set_option(hpcg.HPCG_OPT_APPLY_PATH, other)      # an eager call of the other kernel
            yo = s.apply_M(r)
            torch.cuda.synchronize()
            assert torch.equal(yo, ys[other])
            s.set_option(hpcg.HPCG_OPT_APPLY_PATH, path)
        del g
    assert s.apply_status() == hpcg.HPCG_OK
    s.close()


def test_bridge_apply_errors_and_poll_limit():
    b = make_config("N8k")
    _log("bridge apply errors N8k")
    s = hpcg.Solver(b.n, b.row_ptr, b.col, b.val, batch=1, levels=b.levels)
    s.set_factors(b.U, b.W, b.g)
    r = np.random.default_rng(37).standard_normal(b.n).astype(np.float32)
    s.apply_M(r)
    assert hpcg.hpcg_last_apply_path(s.handle) == hpcg.HPCG_APPLY_FUSED     # slab factors: no bridge
    s.set_option(hpcg.HPCG_OPT_APPLY_PATH, hpcg.HPCG_APPLY_BRIDGE)
    with pytest.raises(hpcg.HPCGError) as err:
        s.apply_M(r)
    assert err.value.status == hpcg.HPCG_ERR_STATE
    with pytest.raises(hpcg.HPCGError):
        s.set_option(hpcg.HPCG_OPT_APPLY_PATH, 4)
    s.close()
    # a tight poll bound on the native path: reported or bit-identical
    b, fac, s = _setup("N16k")
    rr = torch.as_tensor(np.random.default_rng(38).standard_normal(b.n).astype(np.float32)).cuda()
    ref = s.apply_M(rr).clone()
    s.set_option(hpcg.HPCG_OPT_APPLY_POLL_LIMIT, 1)
    for _ in range(3):
        y = s.apply_M(rr)
        st = s.apply_status()
        assert st == hpcg.HPCG_OK and torch.equal(y, ref) or st == hpcg.HPCG_ERR_HIP
    s.set_option(hpcg.HPCG_OPT_APPLY_POLL_LIMIT, 0)
    assert torch.equal(s.apply_M(rr), ref) and s.apply_status() == hpcg.HPCG_OK
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
