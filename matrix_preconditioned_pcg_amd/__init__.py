"""MI355X-native H-matrix-preconditioned conjugate gradients.

The solve runs in a HIP library (csrc/, built for gfx950 into _lib/libhpcg.so)
behind the C ABI of include/hpcg.h; `hpcg` is its ctypes binding with the same
function names plus a small `Solver` owner class.  Import the binding with

    from matrix_preconditioned_pcg_amd import hpcg

Building: `python -m matrix_preconditioned_pcg_amd.build`.
"""

__all__ = ["hpcg", "build"]
