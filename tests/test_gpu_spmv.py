"""GPU SpMV vs the oracle.  Both sides form every row sum in ascending slot
order from 0 with separately rounded multiplies and adds, so the results are
compared bit for bit."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import csr_handle, say, t

pytestmark = pytest.mark.gpu


def _check(rowptr, col, vals, x):
    import torch
    import krylov_solvers_adjoint_amd as K
    n = len(rowptr) - 1
    P = csr_handle(rowptr, col)
    y = K.sla_spmv(P, t(vals), t(x))
    torch.cuda.synchronize()
    A = oracle.CSR(n, rowptr.astype(np.int64), col.astype(np.int32), vals)
    yo = oracle.spmv(A, x)
    assert np.array_equal(y.cpu().numpy(), yo), np.abs(y.cpu().numpy() - yo).max()


@pytest.mark.parametrize("N", [1, 3, 16, 100, 257])
def test_poisson(N):
    rp, c, v = W.poisson_csr(N, np.int32)
    _check(rp, c, v, W.uniform_rhs(N * N, N))


def test_poisson_int64_rowptr():
    rp, c, v = W.poisson_csr(50, np.int64)
    _check(rp, c, v, W.uniform_rhs(2500, 1))


def test_rgg():
    n = 30000
    row, col, val, _ = W.rgg_coo(n, 4, 5)
    rp, c, perm = oracle.csr_from_coo(n, row, col)
    vals = oracle.values_from_coo(perm, int(rp[-1]), val)
    _check(rp.astype(np.int32), c, vals, W.normal_rhs(n, 6))


def test_long_rows_bypass_lds():
    """Tiles with more slots than the LDS stage holds read from memory."""
    rng = np.random.default_rng(5)
    n = 5000  # tiles holding rows 3, 4 and 2600 exceed the 4096-slot stage
    dense_rows = {3, 4, 2600}
    rows = []
    for i in range(n):
        if i in dense_rows:
            cols = np.arange(n)
        else:
            cols = np.unique(np.concatenate([[i], rng.integers(0, n, 4)]))
        rows.append(cols)
    rowptr = np.zeros(n + 1, np.int64)
    rowptr[1:] = np.cumsum([len(r) for r in rows])
    col = np.concatenate(rows).astype(np.int32)
    vals = rng.standard_normal(col.shape[0])
    say(f"long rows: nnz={col.shape[0]}")
    _check(rowptr.astype(np.int32), col, vals, rng.standard_normal(n))


def test_batched_values():
    import torch
    import krylov_solvers_adjoint_amd as K
    N, B = 40, 5
    rp, c, vals, b, _ = W.batched_poisson(N, B, 2, 3)
    P = csr_handle(rp, c)
    y = K.sla_spmv(P, t(vals), t(b))
    torch.cuda.synchronize()
    for s in range(B):
        yo = oracle.spmv(oracle.CSR(N * N, rp.astype(np.int64), c, vals[s]), b[s])
        assert np.array_equal(y[s].cpu().numpy(), yo)
