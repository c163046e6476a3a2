"""The benchmark's roofline accounting against the arrays it stands for: the
algorithmic bytes of an apply and of an SpMV are the bytes of the factors, the
gate, the CSR arrays and the vectors each read or written once, and the block
apply's flops are two per multiply-add of every factor entry per column."""

import numpy as np
import pytest

import bench
from workloads import CONFIGS, make_config


@pytest.mark.parametrize("name", ["N1k", "N8k", "tet4k"])
def test_apply_and_spmv_bytes(name):
    b = make_config(name)
    vec = 4 * b.batch * b.n                       # one fp32 vector
    factors = b.U.astype(np.float32).nbytes + b.W.astype(np.float32).nbytes + b.g.astype(np.float32).nbytes
    assert bench.apply_bytes(b.n, b.K, b.levels, b.batch) == factors + 2 * vec
    csr = (b.val.astype(np.float32).nbytes + b.col.astype(np.int32).nbytes
           + b.row_ptr.astype(np.int32).nbytes)
    assert bench.spmv_bytes(b.n, b.nnz, b.batch) == csr + 2 * vec


def test_n8k_pair_bytes_match_the_quoted_figure():
    b = make_config("N8k")
    total = bench.apply_bytes(b.n, b.K, b.levels, b.batch) + bench.spmv_bytes(b.n, b.nnz, b.batch)
    assert total == 11120644                      # 10.58 MB apply + 0.54 MB SpMV


@pytest.mark.parametrize("name,nrhs", [("N1k", 16), ("N8k", 96)])
def test_block_apply_flops(name, nrhs):
    b = make_config(name)
    # one product with the dense leaf blocks (F_k = U_k U_k^T, U's shape), two
    # with every slab (restriction and prolongation), the gate
    per_column = 2 * b.U.size + 4 * b.W.size + 2 * b.g.size
    assert bench.block_apply_flops(b.n, b.levels, nrhs, b.batch) == nrhs * per_column


def test_every_config_is_known():
    assert set(CONFIGS) == {"N1k", "N8k", "N16k", "tet4k", "batch64x2k"}
