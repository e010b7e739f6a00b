"""The differentiable .matvec on the GPU: the transposed product and the
SpMV backward (grad_x = A^T g, grad_vals = g_i x_j) bit for bit against the
oracle's explicit transpose, the batch, the autograd node, and a chain
through the solve."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_X, csr_handle, rel, say, t

pytestmark = pytest.mark.gpu


def _nonsym_csr(n, per_row, seed, empty_rows=()):
    """A random non-symmetric sparse matrix (ascending columns, no
    duplicates), some rows empty, one stored zero."""
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    for i in range(n):
        if i in empty_rows:
            continue
        k = rng.integers(1, 2 * per_row)
        cs = np.unique(rng.integers(0, n, k))
        rows.append(np.full(cs.shape[0], i))
        cols.append(cs)
    rows = np.concatenate(rows)
    cols = np.concatenate(cols)
    vals = rng.uniform(-2, 2, rows.shape[0])
    vals[rows.shape[0] // 2] = 0.0
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    return np.cumsum(rp).astype(np.int32), cols.astype(np.int32), vals


def _check(rp, c, v, x, g):
    import torch
    import krylov_solvers_adjoint_amd as K
    n = len(rp) - 1
    P = csr_handle(rp, c)
    vt = t(v)
    yt = K.sla_spmv_transpose(P, vt, t(g))
    gx, gv = K.sla_matvec_grad(P, vt, t(x), t(g))
    torch.cuda.synchronize()
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    gxo, gvo = oracle.matvec_grad(A, x, g)
    assert np.array_equal(yt.cpu().numpy(), gxo)
    assert np.array_equal(gx.cpu().numpy(), gxo)
    assert np.array_equal(gv.cpu().numpy(), gvo)


@pytest.mark.parametrize("n,per_row,seed", [(1, 1, 0), (257, 5, 1), (20000, 9, 2)])
def test_random_nonsymmetric(n, per_row, seed):
    rp, c, v = _nonsym_csr(n, per_row, seed, empty_rows={0, n // 3} if n > 3 else set())
    _check(rp, c, v, W.normal_rhs(n, 50), W.normal_rhs(n, 51))


def test_poisson_and_random_graph():
    """A banded pattern (its transpose is banded too) and the irregular
    random geometric graph with non-symmetric values."""
    rp, c, v = W.poisson_csr(300, np.int32)
    n = 300 * 300
    rng = np.random.default_rng(52)
    _check(rp, c, v * rng.uniform(0.5, 1.5, v.shape[0]), W.normal_rhs(n, 53),
           W.normal_rhs(n, 54))
    n = 200000
    row, col, val, _ = W.rgg_coo(n, 4, 5)
    rpg, cg_, perm = oracle.csr_from_coo(n, row, col)
    vg = oracle.values_from_coo(perm, int(rpg[-1]), val) * rng.uniform(0.5, 1.5, int(rpg[-1]))
    _check(rpg.astype(np.int32), cg_, vg, W.normal_rhs(n, 55), W.normal_rhs(n, 56))


def test_batch():
    import torch
    import krylov_solvers_adjoint_amd as K
    n, B = 3000, 4
    rp, c, v = _nonsym_csr(n, 6, 57)
    rng = np.random.default_rng(58)
    vb = np.stack([v * rng.uniform(0.5, 2.0, v.shape[0]) for _ in range(B)])
    xb = rng.standard_normal((B, n))
    gb = rng.standard_normal((B, n))
    P = csr_handle(rp, c)
    gx, gv = K.sla_matvec_grad(P, t(vb), t(xb), t(gb))
    torch.cuda.synchronize()
    for s in range(B):
        gxo, gvo = oracle.matvec_grad(oracle.CSR(n, rp.astype(np.int64), c, vb[s]), xb[s], gb[s])
        assert np.array_equal(gx[s].cpu().numpy(), gxo) and np.array_equal(gv[s].cpu().numpy(), gvo)


def test_autograd_matvec():
    import torch
    import krylov_solvers_adjoint_amd as K
    n = 5000
    rp, c, v = _nonsym_csr(n, 7, 59)
    x = W.normal_rhs(n, 60)
    g = W.normal_rhs(n, 61)
    P = csr_handle(rp, c)
    vals = t(v).requires_grad_(True)
    xt = t(x).requires_grad_(True)
    y = K.SparseTensor(P, vals).matvec(xt)
    (y * t(g)).sum().backward()
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    gxo, gvo = oracle.matvec_grad(A, x, g)
    assert np.array_equal(y.detach().cpu().numpy(), oracle.spmv(A, x))
    assert np.array_equal(xt.grad.cpu().numpy(), gxo)
    assert np.array_equal(vals.grad.cpu().numpy(), gvo)


def test_chain_through_the_solve():
    """L = g . (A (A^-1 b)) = g . b: dL/db = g and dL/dvals = 0, up to the
    solve's tolerance; both backward passes run in one autograd graph."""
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 60
    rp, c, v = W.poisson_csr(N, np.int32)
    n = N * N
    b = W.uniform_rhs(n, 62)
    g = W.normal_rhs(n, 63)
    P = csr_handle(rp, c)
    vals = t(v).requires_grad_(True)
    bt = t(b).requires_grad_(True)
    A = K.SparseTensor(P, vals)
    y = A.matvec(A.solve(bt, tol=1e-13, maxit=10000))
    (y * t(g)).sum().backward()
    say(f"chain: |db - g| {rel(bt.grad.cpu().numpy(), g):.1e}, |dvals| "
        f"{float(vals.grad.abs().max()):.1e}")
    assert rel(y.detach().cpu().numpy(), b) <= 1e-11
    assert rel(bt.grad.cpu().numpy(), g) <= 1e-10
    assert float(vals.grad.abs().max()) <= 1e-9 * float(np.abs(g).max() * np.abs(b).max() + 1)
