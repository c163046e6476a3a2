"""ctypes binding of the hpcg C ABI (include/hpcg.h).

Argument marshalling only: every function here checks tensor dtypes, devices,
sizes and contiguity, passes raw device pointers and the current HIP stream to
the library of the same name, and turns status codes into exceptions.  All
arithmetic of the solve runs in the library's HIP kernels; there is no CPU or
PyTorch fallback, and a missing library raises instead of degrading.

PyTorch supplies device memory and streams.  It is imported before the library
is loaded so that the library binds to the same HIP runtime as torch.
"""

from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

from .build import LIB

HPCG_OK = 0
HPCG_ERR_INVALID_ARG = 1
HPCG_ERR_SHAPE = 2
HPCG_ERR_HIP = 3
HPCG_ERR_BREAKDOWN = 4
HPCG_ERR_NOT_CONVERGED = 5
HPCG_ERR_WORKSPACE = 6
HPCG_ERR_STATE = 7

HPCG_SYS_RUNNING = 0
HPCG_SYS_CONVERGED = 1
HPCG_SYS_NOT_CONVERGED = 2
HPCG_SYS_BREAKDOWN = 3

HPCG_ENGINE_AUTO = 0
HPCG_ENGINE_GRAPH = 1
HPCG_ENGINE_PERSISTENT = 2

HPCG_OPT_ENGINE = 1
HPCG_OPT_GRAPH_UNROLL = 2
HPCG_OPT_PRECISION = 4
HPCG_OPT_LEAF_SPLIT = 8
HPCG_OPT_BLOCK_SPLIT = 512
HPCG_OPT_APPLY_PATH = 16

HPCG_OPT_FORM = 32

HPCG_OPT_FALLBACK = 64
HPCG_OPT_POLL_LIMIT = 128
HPCG_OPT_APPLY_POLL_LIMIT = 256

HPCG_FORM_DIRECT = 0
HPCG_FORM_SQUARED = 1
HPCG_FORM_JACOBI = 2

HPCG_APPLY_AUTO = 0
HPCG_APPLY_STREAMING = 1
HPCG_APPLY_FUSED = 2
HPCG_APPLY_BRIDGE = 3

HPCG_PREC_VEC64 = 0
HPCG_PREC_VEC32 = 1

LEAF = 128
RANK = 32


class HPCGError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"hpcg status {status}: {message}")
        self.status = status


class hpcg_partition(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("leaf", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("levels", ctypes.c_int32), ("batch", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    """The library this process loads: libhpcg.so, or the file named by the
    HPCG_LIBRARY environment variable (e.g. the timeline build)."""
    return os.environ.get("HPCG_LIBRARY") or LIB


def lib() -> ctypes.CDLL:
    """Load the library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m matrix_preconditioned_pcg_amd.build`")
    L = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp, i32, i64, dbl, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_size_t
    sig = {
        "hpcg_workspace_bytes": (sz, [P(hpcg_partition), i64]),
        "hpcg_create": (i32, [P(hpcg_partition), vp, vp, vp, i64, vp, sz, vp, P(vp)]),
        "hpcg_set_values": (i32, [vp, vp]),
        "hpcg_set_factors": (i32, [vp, vp, vp, vp]),
        "hpcg_set_factors_bridge": (i32, [vp, vp, vp, vp, vp, vp]),
        "hpcg_apply_M": (i32, [vp, vp, vp]),
        "hpcg_apply_status": (i32, [vp]),
        "hpcg_read_probe": (i32, [vp, sz, vp, i32, vp]),
        "hpcg_trace_read": (i32, [vp, sz, i32]),
        "hpcg_spmv": (i32, [vp, vp, vp]),
        "hpcg_block_workspace_bytes": (sz, [vp, i32]),
        "hpcg_apply_M_block": (i32, [vp, vp, vp, i32, vp, sz]),
        "hpcg_spmv_block": (i32, [vp, vp, vp, i32]),
        "hpcg_apply_M_block_noalloc": (i32, [vp, vp, vp, i32]),
        "hpcg_solve": (i32, [vp, vp, vp, dbl, i32, P(i32), P(dbl)]),
        "hpcg_last_solve_status": (i32, [vp, P(i32)]),
        "hpcg_solve_refined": (i32, [vp, vp, vp, dbl, i32, dbl, i32, P(i32), P(i32), P(dbl)]),
        "hpcg_set_option": (i32, [vp, i32, i32]),
        "hpcg_last_engine": (i32, [vp]),
        "hpcg_last_apply_path": (i32, [vp]),
        "hpcg_last_fallback": (i32, [vp]),
        "hpcg_block_solve_workspace_bytes": (sz, [vp, i32]),
        "hpcg_solve_block": (i32, [vp, vp, vp, i32, dbl, i32, vp, sz, P(i32), P(dbl)]),
        "hpcg_estimate_spectrum": (i32, [vp, i32, P(dbl), P(dbl)]),
        "hpcg_last_launch_info": (i32, [vp, P(i32), P(i32)]),
        "hpcg_status_string": (ctypes.c_char_p, [i32]),
        "hpcg_last_error": (ctypes.c_char_p, [vp]),
        "hpcg_destroy": (None, [vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def declared_functions(header: str) -> list:
    """Names of the functions a C header declares (used to check the exports)."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hpcg_[a-zA-Z_]+)\s*\(", text)))


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

def _ptr(t: torch.Tensor | None, dtype, numel: int, name: str, allow_none=False) -> int | None:
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is None")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, handle=None):
    if status != HPCG_OK:
        msg = lib().hpcg_last_error(handle).decode()
        raise HPCGError(status, msg or lib().hpcg_status_string(status).decode())


def partition(n: int, levels: int | None = None, batch: int = 1) -> hpcg_partition:
    K = n // LEAF
    if levels is None:
        levels = max(K.bit_length() - 1, 0)
    return hpcg_partition(n, LEAF, RANK, levels, batch)


# ----------------------------------------------------------------------------
# the C ABI, same names
# ----------------------------------------------------------------------------

def hpcg_workspace_bytes(part: hpcg_partition, nnz_total: int) -> int:
    return int(lib().hpcg_workspace_bytes(ctypes.byref(part), int(nnz_total)))


def hpcg_create(part: hpcg_partition, row_ptr, col, val, workspace, stream=None):
    """Returns an opaque handle (int).  workspace: uint8 device tensor whose
    data pointer is 256-byte aligned and at least hpcg_workspace_bytes long."""
    N = part.n * part.batch
    nnz = int(col.numel())
    rp = _ptr(row_ptr, torch.int32, N + 1, "row_ptr")
    cp = _ptr(col, torch.int32, nnz, "col")
    vp = _ptr(val, torch.float32, nnz, "val")
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda":
        raise TypeError("workspace must be a uint8 device tensor")
    h = ctypes.c_void_p()
    st = lib().hpcg_create(ctypes.byref(part), rp, cp, vp, nnz, workspace.data_ptr(),
                           workspace.numel(), _stream(stream), ctypes.byref(h))
    _check(st, None)
    return h.value


def hpcg_set_values(h, val, nnz: int):
    _check(lib().hpcg_set_values(h, _ptr(val, torch.float32, nnz, "val")), h)


def hpcg_set_factors(h, part: hpcg_partition, U, W, g):
    K = part.n // LEAF
    up = _ptr(U, torch.float32, part.batch * K * LEAF * LEAF, "U")
    wp = _ptr(W, torch.float32, part.batch * part.levels * K * LEAF * RANK, "W", allow_none=part.levels == 0)
    gp = _ptr(g, torch.float32, part.batch * part.n, "g")
    _check(lib().hpcg_set_factors(h, up, wp, gp), h)


def hpcg_set_factors_bridge(h, part: hpcg_partition, F, Ub, Vb, Bc, g):
    K = part.n // LEAF
    cores = sum(K >> (l + 1) for l in range(part.levels))
    none_ok = part.levels == 0
    fp = _ptr(F, torch.float32, part.batch * K * LEAF * LEAF, "F")
    up = _ptr(Ub, torch.float32, part.batch * K * LEAF * RANK, "Ub", allow_none=none_ok)
    vq = _ptr(Vb, torch.float32, part.batch * K * LEAF * RANK, "Vb", allow_none=none_ok)
    bp = _ptr(Bc, torch.float32, part.batch * cores * RANK * RANK, "Bc", allow_none=none_ok)
    gp = _ptr(g, torch.float32, part.batch * part.n, "g")
    _check(lib().hpcg_set_factors_bridge(h, fp, up, vq, bp, gp), h)


def hpcg_apply_M(h, part: hpcg_partition, r, y):
    N = part.n * part.batch
    _check(lib().hpcg_apply_M(h, _ptr(r, torch.float32, N, "r"), _ptr(y, torch.float32, N, "y")), h)


def hpcg_apply_status(h) -> int:
    """Synchronizes; returns the status code (HPCG_ERR_HIP when an earlier
    single-pass apply gave up a bounded wait), without raising."""
    return int(lib().hpcg_apply_status(h))


def hpcg_read_probe(src, nbytes: int, sink, workgroups: int, stream=None):
    """Measurement aid: one launch reading nbytes of the device tensor src
    (sink: float32 device tensor of `workgroups` elements)."""
    if src.device.type != "cuda" or nbytes > src.numel() * src.element_size():
        raise ValueError("src must be a device tensor of at least nbytes bytes")
    _check(lib().hpcg_read_probe(src.data_ptr(), int(nbytes), _ptr(sink, torch.float32, int(workgroups), "sink"),
                                 int(workgroups), _stream(stream)), None)


def hpcg_trace_read(count: int, clear: bool = True):
    """The first `count` timeline entries (uint64) of a HPCG_TRACE build, as a list."""
    out = (ctypes.c_uint64 * max(int(count), 1))()
    _check(lib().hpcg_trace_read(out, int(count), int(bool(clear))), None)
    return list(out)[:count]


def hpcg_spmv(h, part: hpcg_partition, x, y):
    N = part.n * part.batch
    _check(lib().hpcg_spmv(h, _ptr(x, torch.float32, N, "x"), _ptr(y, torch.float32, N, "y")), h)


def hpcg_block_workspace_bytes(h, nrhs: int) -> int:
    return int(lib().hpcg_block_workspace_bytes(h, int(nrhs)))


def hpcg_apply_M_block(h, part: hpcg_partition, R, Y, nrhs: int, work=None):
    """R, Y: float32 device tensors of batch*n*nrhs elements, node-major; work:
    uint8 device tensor of hpcg_block_workspace_bytes(h, nrhs) bytes (or None
    when levels == 0)."""
    N = part.n * part.batch
    wp, wb = (None, 0) if work is None else (work.data_ptr(), work.numel())
    _check(lib().hpcg_apply_M_block(h, _ptr(R, torch.float32, N * nrhs, "R"), _ptr(Y, torch.float32, N * nrhs, "Y"),
                                    int(nrhs), wp, wb), h)


def hpcg_apply_M_block_noalloc(h, part: hpcg_partition, R, Y, nrhs: int):
    """hpcg_apply_M_block with the library's fixed scratch instead of a caller workspace."""
    N = part.n * part.batch
    _check(lib().hpcg_apply_M_block_noalloc(h, _ptr(R, torch.float32, N * nrhs, "R"),
                                            _ptr(Y, torch.float32, N * nrhs, "Y"), int(nrhs)), h)


def hpcg_spmv_block(h, part: hpcg_partition, X, Y, nrhs: int):
    N = part.n * part.batch
    _check(lib().hpcg_spmv_block(h, _ptr(X, torch.float32, N * nrhs, "X"), _ptr(Y, torch.float32, N * nrhs, "Y"),
                                 int(nrhs)), h)


def hpcg_solve(h, part: hpcg_partition, b, x, tol: float, maxit: int):
    """Returns (status, iters[list], relres[list]); raises on argument/HIP errors,
    not on HPCG_ERR_NOT_CONVERGED or HPCG_ERR_BREAKDOWN."""
    N = part.n * part.batch
    iters = (ctypes.c_int32 * part.batch)()
    rel = (ctypes.c_double * part.batch)()
    st = lib().hpcg_solve(h, _ptr(b, torch.float32, N, "b"), _ptr(x, torch.float64, N, "x"),
                          float(tol), int(maxit), iters, rel)
    if st not in (HPCG_OK, HPCG_ERR_NOT_CONVERGED, HPCG_ERR_BREAKDOWN):
        _check(st, h)
    return st, list(iters), list(rel)


def hpcg_solve_refined(h, part: hpcg_partition, b, x, tol: float, maxit: int, inner_tol: float, max_outer: int):
    """Returns (status, inner iterations[list], outer steps[list], true relres[list])."""
    N = part.n * part.batch
    iters = (ctypes.c_int32 * part.batch)()
    outer = (ctypes.c_int32 * part.batch)()
    rel = (ctypes.c_double * part.batch)()
    st = lib().hpcg_solve_refined(h, _ptr(b, torch.float32, N, "b"), _ptr(x, torch.float64, N, "x"),
                                  float(tol), int(maxit), float(inner_tol), int(max_outer), iters, outer, rel)
    if st not in (HPCG_OK, HPCG_ERR_NOT_CONVERGED, HPCG_ERR_BREAKDOWN):
        _check(st, h)
    return st, list(iters), list(outer), list(rel)


def hpcg_last_solve_status(h, batch: int) -> list:
    out = (ctypes.c_int32 * batch)()
    _check(lib().hpcg_last_solve_status(h, out), h)
    return list(out)


def hpcg_set_option(h, option: int, value: int):
    _check(lib().hpcg_set_option(h, int(option), int(value)), h)


def hpcg_last_engine(h) -> int:
    return int(lib().hpcg_last_engine(h))


def hpcg_block_solve_workspace_bytes(h, nrhs: int) -> int:
    return int(lib().hpcg_block_solve_workspace_bytes(h, int(nrhs)))


def hpcg_solve_block(h, part: hpcg_partition, B, X, nrhs: int, tol: float, maxit: int, work):
    """Returns (status, iters[batch*nrhs], relres[batch*nrhs]); raises on
    argument/HIP errors, not on HPCG_ERR_NOT_CONVERGED or HPCG_ERR_BREAKDOWN."""
    N = part.n * part.batch
    cnt = part.batch * nrhs
    iters = (ctypes.c_int32 * cnt)()
    rel = (ctypes.c_double * cnt)()
    st = lib().hpcg_solve_block(h, _ptr(B, torch.float32, N * nrhs, "B"), _ptr(X, torch.float64, N * nrhs, "X"),
                                int(nrhs), float(tol), int(maxit), _ptr(work, torch.uint8, work.numel(), "work"),
                                int(work.numel()), iters, rel)
    if st not in (HPCG_OK, HPCG_ERR_NOT_CONVERGED, HPCG_ERR_BREAKDOWN):
        _check(st, h)
    return st, list(iters), list(rel)


def hpcg_last_fallback(h) -> int:
    return int(lib().hpcg_last_fallback(h))


def hpcg_estimate_spectrum(h, steps: int = 40) -> tuple:
    """(lambda_min, lambda_max) Lanczos estimates for H, the factor operator."""
    lo, hi = ctypes.c_double(), ctypes.c_double()
    _check(lib().hpcg_estimate_spectrum(h, int(steps), ctypes.byref(lo), ctypes.byref(hi)), h)
    return lo.value, hi.value


def hpcg_last_apply_path(h) -> int:
    return int(lib().hpcg_last_apply_path(h))


def hpcg_last_launch_info(h) -> tuple:
    """(workgroups per phase launch, largest dynamic LDS bytes) of the last solve."""
    grid, lds = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().hpcg_last_launch_info(h, ctypes.byref(grid), ctypes.byref(lds)), h)
    return grid.value, lds.value


def hpcg_status_string(status: int) -> str:
    return lib().hpcg_status_string(int(status)).decode()


def hpcg_last_error(h) -> str:
    return lib().hpcg_last_error(h).decode()


def hpcg_destroy(h):
    if h:
        lib().hpcg_destroy(h)


# ----------------------------------------------------------------------------
# convenience owner of a handle and its device buffers
# ----------------------------------------------------------------------------

@dataclass
class SolveResult:
    x: torch.Tensor          # fp64 [batch, n]
    iterations: list
    relres: list
    status: int              # hpcg_status of the call
    system_status: list      # hpcg_system_status per system


class Solver:
    """Owns one hpcg handle, its workspace and its CSR copy on the device.

    row_ptr/col/val may be numpy arrays or tensors; they are moved to the
    device and handed to hpcg_create.
    """

    def __init__(self, n: int, row_ptr, col, val, batch: int = 1, levels: int | None = None,
                 device="cuda", stream=None):
        self.device = torch.device(device)
        self.part = partition(n, levels, batch)
        self.stream = stream
        self.n, self.batch = n, batch
        rp = torch.as_tensor(row_ptr, dtype=torch.int32).to(self.device).contiguous()
        cl = torch.as_tensor(col, dtype=torch.int32).to(self.device).contiguous()
        vl = torch.as_tensor(val, dtype=torch.float32).to(self.device).contiguous()
        self.nnz = int(cl.numel())
        nbytes = hpcg_workspace_bytes(self.part, self.nnz)
        if nbytes == 0:
            raise HPCGError(HPCG_ERR_SHAPE, "invalid partition")
        raw = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        pad = (-raw.data_ptr()) % 256
        self._raw = raw
        self.workspace = raw[pad:pad + nbytes]
        self.handle = hpcg_create(self.part, rp, cl, vl, self.workspace, stream)
        self._keep = (rp, cl, vl)

    def set_option(self, option: int, value: int):
        hpcg_set_option(self.handle, option, value)

    def set_values(self, val):
        v = torch.as_tensor(val, dtype=torch.float32).to(self.device).contiguous()
        hpcg_set_values(self.handle, v, self.nnz)
        self._keep = self._keep[:2] + (v,)

    def set_factors(self, U, W, g):
        self._factors = tuple(
            None if a is None else torch.as_tensor(a, dtype=torch.float32).to(self.device).contiguous()
            for a in (U, W, g))
        hpcg_set_factors(self.handle, self.part, *self._factors)

    def set_factors_bridge(self, F, Ub, Vb, Bc, g):
        """Bridge-format factors (per-leaf bridges and per-tile cores)."""
        self._factors = tuple(
            None if a is None else torch.as_tensor(a, dtype=torch.float32).to(self.device).contiguous()
            for a in (F, Ub, Vb, Bc, g))
        hpcg_set_factors_bridge(self.handle, self.part, *self._factors)

    def _vec(self, v):
        return torch.as_tensor(v, dtype=torch.float32).to(self.device).contiguous().reshape(-1)

    def apply_M(self, r, y=None):
        r = self._vec(r)
        y = torch.empty_like(r) if y is None else y
        hpcg_apply_M(self.handle, self.part, r, y)
        return y

    def apply_status(self) -> int:
        """HPCG_OK, or HPCG_ERR_HIP if a single-pass apply since the last call
        gave up its bounded wait (synchronizes the stream)."""
        return hpcg_apply_status(self.handle)

    def spmv(self, x, y=None):
        x = self._vec(x)
        y = torch.empty_like(x) if y is None else y
        hpcg_spmv(self.handle, self.part, x, y)
        return y

    def _block(self, V, nrhs):
        V = torch.as_tensor(V, dtype=torch.float32).to(self.device).contiguous()
        if V.numel() != self.batch * self.n * nrhs:
            raise ValueError(f"block must have batch*n*nrhs = {self.batch * self.n * nrhs} elements")
        return V

    def apply_M_block(self, R, nrhs: int, Y=None):
        """Y = M R for a node-major block [batch*n, nrhs]."""
        R = self._block(R, nrhs)
        Y = torch.empty_like(R) if Y is None else Y
        nbytes = hpcg_block_workspace_bytes(self.handle, nrhs)
        if nbytes == 0:
            raise HPCGError(HPCG_ERR_SHAPE, "nrhs must be a multiple of 16 in [16, 1024]")
        work = getattr(self, "_bwork", None)
        if work is None or work.numel() < nbytes:
            work = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._bwork = work
        hpcg_apply_M_block(self.handle, self.part, R, Y, nrhs, work)
        return Y

    def spmv_block(self, X, nrhs: int, Y=None):
        """Y = A X for a node-major block [batch*n, nrhs]."""
        X = self._block(X, nrhs)
        Y = torch.empty_like(X) if Y is None else Y
        hpcg_spmv_block(self.handle, self.part, X, Y, nrhs)
        return Y

    def solve(self, b, tol: float = 1e-6, maxit: int = 1000, x=None) -> SolveResult:
        b = self._vec(b)
        x = torch.empty(b.numel(), dtype=torch.float64, device=self.device) if x is None else x
        st, iters, rel = hpcg_solve(self.handle, self.part, b, x, tol, maxit)
        sys_st = hpcg_last_solve_status(self.handle, self.batch)
        return SolveResult(x.reshape(self.batch, self.n), iters, rel, st, sys_st)

    def solve_block(self, B, nrhs: int, tol: float = 1e-6, maxit: int = 1000, X=None):
        """Block PCG on a node-major block [batch*n, nrhs]; returns
        (X fp64 [batch*n, nrhs], iterations, relres, status), the lists
        system-major over (system, column)."""
        B = self._block(B, nrhs)
        X = torch.empty(B.numel(), dtype=torch.float64, device=self.device) if X is None else X
        nbytes = hpcg_block_solve_workspace_bytes(self.handle, nrhs)
        if nbytes == 0:
            raise HPCGError(HPCG_ERR_SHAPE, "nrhs must be a multiple of 16 in [16, 1024]")
        work = getattr(self, "_bswork", None)
        if work is None or work.numel() < nbytes:
            work = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._bswork = work
        st, iters, rel = hpcg_solve_block(self.handle, self.part, B, X, nrhs, tol, maxit, work)
        return X.reshape(-1, nrhs), iters, rel, st

    def solve_refined(self, b, tol: float = 1e-10, maxit: int = 5000, inner_tol: float = 1e-5,
                      max_outer: int = 10, x=None):
        """Outer fp64 refinement around the configured solve; returns
        (SolveResult with the true relative residual, outer steps per system)."""
        b = self._vec(b)
        x = torch.empty(b.numel(), dtype=torch.float64, device=self.device) if x is None else x
        st, iters, outer, rel = hpcg_solve_refined(self.handle, self.part, b, x, tol, maxit, inner_tol, max_outer)
        sys_st = hpcg_last_solve_status(self.handle, self.batch)
        return SolveResult(x.reshape(self.batch, self.n), iters, rel, st, sys_st), outer

    def estimate_spectrum(self, steps: int = 40) -> tuple:
        return hpcg_estimate_spectrum(self.handle, steps)

    @property
    def last_fallback(self) -> int:
        return hpcg_last_fallback(self.handle)

    @property
    def last_engine(self) -> int:
        return hpcg_last_engine(self.handle)

    def close(self):
        if getattr(self, "handle", None):
            torch.cuda.synchronize(self.device)
            hpcg_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
