"""ctypes front end of the plain C fp64 oracle (oracle/c/pcg_oracle.c).

TEST INFRASTRUCTURE ONLY (see the package docstring).  Same definitions as
hmatrix.apply_M, sparse.spmv and pcg.pcg, written as C loops so that the
oracle can be timed on host cores; pinned against those functions by the CPU
tests.
"""

from __future__ import annotations

import ctypes

import numpy as np

from .build import lib

_STATUS = {0: "converged", 1: "not_converged", 2: "breakdown"}


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def set_threads(t: int) -> None:
    lib().orc_set_threads(int(t))


def max_threads() -> int:
    return int(lib().orc_max_threads())


def spmv(row_ptr, col, val, x):
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    cl = np.ascontiguousarray(col, dtype=np.int32)
    vl = np.ascontiguousarray(val, dtype=np.float32)
    xx = np.ascontiguousarray(x, dtype=np.float64)
    n = rp.size - 1
    y = np.empty(n)
    lib().orc_spmv(n, _p(rp), _p(cl), _p(vl), _p(xx), _p(y))
    return y


def apply_M(U, W, g, r):
    U = np.ascontiguousarray(U, dtype=np.float32)
    K, L, _ = U.shape
    levels = 0 if W is None else W.shape[0]
    R = W.shape[3] if levels else 32
    Wc = np.ascontiguousarray(W if levels else np.zeros(1), dtype=np.float32)
    gg = np.ascontiguousarray(g, dtype=np.float32)
    rr = np.ascontiguousarray(r, dtype=np.float64)
    y = np.empty(K * L)
    lib().orc_apply_M(K, L, R, levels, _p(U), _p(Wc), _p(gg), _p(rr), _p(y))
    return y


def pcg(row_ptr, col, val, b, U, W, g, tol: float, maxit: int):
    """Returns (x, iterations, status, recursive relres) of one system."""
    rp = np.ascontiguousarray(row_ptr, dtype=np.int32)
    cl = np.ascontiguousarray(col, dtype=np.int32)
    vl = np.ascontiguousarray(val, dtype=np.float32)
    U = np.ascontiguousarray(U, dtype=np.float32)
    K, L, _ = U.shape
    levels = 0 if W is None else W.shape[0]
    R = W.shape[3] if levels else 32
    Wc = np.ascontiguousarray(W if levels else np.zeros(1), dtype=np.float32)
    gg = np.ascontiguousarray(g, dtype=np.float32)
    bb = np.ascontiguousarray(b, dtype=np.float32)
    n = rp.size - 1
    x = np.empty(n)
    it, rel = ctypes.c_int32(), ctypes.c_double()
    st = lib().orc_pcg(n, _p(rp), _p(cl), _p(vl), L, R, levels, _p(U), _p(Wc), _p(gg), _p(bb), float(tol),
                       int(maxit), _p(x), ctypes.byref(it), ctypes.byref(rel))
    return x, it.value, _STATUS[st], rel.value
