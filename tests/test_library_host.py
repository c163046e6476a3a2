"""CPU checks of the C ABI library: it loads, exports what include/hpcg.h
declares, and its host-side argument validation answers without touching a GPU."""

import ctypes
import os

import pytest

from matrix_preconditioned_pcg_amd import build as build_mod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hpcg.h")


@pytest.fixture(scope="module")
def hp():
    if not os.path.exists(build_mod.LIB):
        build_mod.build()
    from matrix_preconditioned_pcg_amd import hpcg
    hpcg.lib()
    return hpcg


def test_exports_every_declared_symbol(hp):
    names = hp.declared_functions(HEADER)
    assert len(names) >= 13
    L = ctypes.CDLL(build_mod.LIB)
    for n in names:
        assert hasattr(L, n), n


def test_binding_mirrors_the_abi_names(hp):
    for n in hp.declared_functions(HEADER):
        assert callable(getattr(hp, n)), n


def test_header_is_plain_c():
    import re
    text = open(HEADER).read()
    assert 'extern "C"' in text
    code = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    for banned in ("torch", "hipStream_t", "#include <hip", "Tensor"):
        assert banned not in code


@pytest.mark.parametrize("kw", [dict(leaf=64), dict(rank=16), dict(n=1000), dict(n=384),
                                dict(levels=4), dict(levels=-1), dict(batch=0), dict(n=0)])
def test_workspace_bytes_rejects_bad_partitions(hp, kw):
    p = dict(n=1024, leaf=128, rank=32, levels=3, batch=1)
    p.update(kw)
    part = hp.hpcg_partition(p["n"], p["leaf"], p["rank"], p["levels"], p["batch"])
    assert hp.hpcg_workspace_bytes(part, 100) == 0


@pytest.mark.parametrize("n,levels", [(32768, 8), (65536, 8), (65536, 5), (1 << 20, 8), (1 << 20, 0)])
def test_workspace_bytes_accepts_large_partitions(hp, n, levels):
    # more leaves than the full eight levels cover (a partial hierarchy): the
    # partner stages hold 2^levels - 1 rows, not one per leaf, so the
    # partition fits a compute unit's LDS and is accepted
    part = hp.hpcg_partition(n, 128, 32, levels, 1)
    assert hp.hpcg_workspace_bytes(part, 7 * n) > n * (128 + 32 * levels) * 4


def test_workspace_bytes_covers_the_buffers(hp):
    part = hp.partition(16384)
    nnz = 110592
    nbytes = hp.hpcg_workspace_bytes(part, nnz)
    factors = 128 * 128 * 128 * 4 + 7 * 128 * 128 * 32 * 4
    # block apply: dense leaf blocks U_k U_k^T and the slabs (also transposed) as
    # fp16 pairs, one exponent per leaf and per slab
    factors += 128 * 128 * 128 * 4 + 128 * 4 + 2 * 7 * 128 * 128 * 32 * 4 + 7 * 128 * 4
    csr = (16385 + 2 * nnz) * 4
    vectors = 16384 * (2 * 4 + 7 * 8)            # g, b fp32; r (two), z, q, p0, p1, x fp64
    # per leaf: diagonal shares of up to 8 slots and two copies of W_l[k]^T r_k, fp64
    restrictions = 128 * (8 * 128 + 2 * 7 * 32) * 8
    flagged = 128 * 7 * 32 * 8 + 128 * 128 * 8   # single-pass apply: (value, epoch) words
    barrier_lines = 128 * 128                     # resident solve: one 128-byte line per leaf
    # resident solve: leaf-local CSR columns, halo lists (at most one slot per
    # entry), z as two flagged words per row, four flagged partials per leaf
    resident = 2 * nnz * 4 + 129 * 4 + 16384 * 16 + 128 * 32
    # resident solve: W^T q and p.q as flagged words, two step parities
    resident += 2 * 7 * 128 * 32 * 8 + 2 * 128 * 16
    # the bridge format as given (native bridge apply): U~, V~ and K - 1 cores
    bridge = 2 * 128 * 128 * 32 * 4 + 127 * 32 * 32 * 4
    need = factors + csr + vectors + restrictions + flagged + barrier_lines + resident + bridge
    assert need <= nbytes <= need + (1 << 20)
    assert hp.hpcg_workspace_bytes(hp.partition(2048, batch=64), 851968) > 64 * hp.hpcg_workspace_bytes(
        hp.partition(2048), 13312) * 0.9


def test_create_validates_before_touching_the_device(hp):
    L = hp.lib()
    h = ctypes.c_void_p()
    bad = hp.hpcg_partition(1000, 128, 32, 0, 1)
    st = L.hpcg_create(ctypes.byref(bad), 8, 8, 8, 10, 256, 1 << 20, None, ctypes.byref(h))
    assert st == hp.HPCG_ERR_SHAPE
    assert "multiple of 128" in hp.hpcg_last_error(None)
    good = hp.partition(1024)
    st = L.hpcg_create(ctypes.byref(good), None, 8, 8, 10, 256, 1 << 20, None, ctypes.byref(h))
    assert st == hp.HPCG_ERR_INVALID_ARG
    st = L.hpcg_create(ctypes.byref(good), 8, 8, 8, 10, 256 + 4, 1 << 30, None, ctypes.byref(h))
    assert st == hp.HPCG_ERR_WORKSPACE
    st = L.hpcg_create(ctypes.byref(good), 8, 8, 8, 10, 256, 16, None, ctypes.byref(h))
    assert st == hp.HPCG_ERR_WORKSPACE
    st = L.hpcg_create(ctypes.byref(good), 8, 8, 8, 10, 256, 1 << 30, None, None)
    assert st == hp.HPCG_ERR_INVALID_ARG
    assert h.value is None


def test_null_handle_calls(hp):
    L = hp.lib()
    assert L.hpcg_set_option(None, 1, 0) == hp.HPCG_ERR_INVALID_ARG
    assert L.hpcg_apply_M(None, None, None) == hp.HPCG_ERR_INVALID_ARG
    assert L.hpcg_spmv(None, None, None) == hp.HPCG_ERR_INVALID_ARG
    assert L.hpcg_solve(None, None, None, 1e-6, 10, None, None) == hp.HPCG_ERR_INVALID_ARG
    assert L.hpcg_last_engine(None) == 0
    assert L.hpcg_apply_status(None) == hp.HPCG_ERR_INVALID_ARG
    assert L.hpcg_apply_M_block_noalloc(None, None, None, 16) == hp.HPCG_ERR_INVALID_ARG
    # the read probe validates before it launches (no device touched)
    assert L.hpcg_read_probe(None, 16, None, 1, None) == hp.HPCG_ERR_INVALID_ARG
    assert L.hpcg_read_probe(16, 24, 16, 1, None) == hp.HPCG_ERR_INVALID_ARG
    assert L.hpcg_read_probe(16, 32, 16, 0, None) == hp.HPCG_ERR_INVALID_ARG
    L.hpcg_destroy(None)
    for code in range(8):
        assert hp.hpcg_status_string(code) not in ("", "unknown status")
