"""Build the HIP library libhpcg.so for gfx950, in-tree.

    python -m matrix_preconditioned_pcg_amd.build

The library is one translation unit (csrc/hpcg.hip, which pulls in the device
code) compiled with hipcc for gfx950 only.  Packed-fp32 VALU instructions are
disabled (target feature -packed-fp32-ops) so every fp32 operation is a plain
scalar-lane instruction.  The result is written atomically to _lib/libhpcg.so.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "hpcg.hip")
DEPS = [os.path.join(HERE, "csrc", f) for f in ("hpcg.hip", "hpcg_device.hpp", "hpcg_kernels.hpp", "hpcg_leaf.hpp",
                                                 "hpcg_apply.hpp", "hpcg_bridge.hpp", "hpcg_resident.hpp", "hpcg_block.hpp",
                                                 "hpcg_bsolve.hpp")]
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(HERE, "_lib")
LIB = os.path.join(LIB_DIR, "libhpcg.so")
TRACE_LIB = os.path.join(LIB_DIR, "libhpcg_trace.so")   # the same sources with HPCG_TRACE (timeline)
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def command(out: str, trace: bool = False) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument"] + (["-DHPCG_TRACE"] if trace else []) + [
            "-I", INCLUDE, "-o", out, SRC]


def build(verbose: bool = False, trace: bool = False) -> str:
    """Compile libhpcg.so (or, with trace, the timeline build libhpcg_trace.so;
    always recompiles) and return its path."""
    os.makedirs(LIB_DIR, exist_ok=True)
    target = TRACE_LIB if trace else LIB
    tmp = target + f".tmp{os.getpid()}"
    cmd = command(tmp, trace)
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + proc.stdout + proc.stderr)
    os.replace(tmp, target)
    return target


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, trace="--trace" in sys.argv))
