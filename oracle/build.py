"""Build the plain C fp64 oracle (oracle/c/pcg_oracle.c) with gcc, in-tree.

TEST INFRASTRUCTURE ONLY: loaded by the tests and by the benchmark's CPU
baseline, never by the product path.  OpenMP splits rows, leaves and the tiles
of a level; sums keep a fixed order, so results do not depend on the thread
count.

    python -m oracle.build
"""

from __future__ import annotations

import ctypes
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "c", "pcg_oracle.c")
LIB = os.path.join(HERE, "_build", "liborc.so")


def build(verbose: bool = False) -> str:
    """Compile liborc.so (always recompiles) and return its path."""
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError("gcc failed:\n" + proc.stdout + proc.stderr)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib() -> ctypes.CDLL:
    """Load liborc.so, building it first if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        build()
    L = ctypes.CDLL(LIB)
    vp, i32, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double
    P = ctypes.POINTER
    L.orc_set_threads.argtypes, L.orc_set_threads.restype = [i32], None
    L.orc_max_threads.argtypes, L.orc_max_threads.restype = [], i32
    L.orc_spmv.argtypes, L.orc_spmv.restype = [i32, vp, vp, vp, vp, vp], None
    L.orc_apply_M.argtypes, L.orc_apply_M.restype = [i32, i32, i32, i32, vp, vp, vp, vp, vp], None
    L.orc_pcg.argtypes = [i32, vp, vp, vp, i32, i32, i32, vp, vp, vp, vp, dbl, i32, vp, P(i32), P(dbl)]
    L.orc_pcg.restype = i32
    _lib = L
    return L


if __name__ == "__main__":
    print(build(verbose=True))
