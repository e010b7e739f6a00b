"""Edge cases of the .matvec backward, .eigsh, BiCGStab and list paths: int64
row pointers (every kernel family has an int64 instantiation) and batched
autograd through eigsh and BiCGStab, each against the oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_GRAD, TOL_X, csr_handle, rel, t

pytestmark = pytest.mark.gpu


def test_int64_row_pointers():
    import torch
    import krylov_solvers_adjoint_amd as K
    # .matvec backward and A^T x: bit for bit
    N = 40
    rp, c, v = W.poisson_csr(N, np.int64)
    n = N * N
    rng = np.random.default_rng(3)
    v = v * rng.uniform(0.5, 1.5, v.shape[0])     # non-symmetric values
    A = oracle.CSR(n, rp, c, v)
    P = csr_handle(rp, c)
    assert P.rowptr_dtype == torch.int64
    x, g = W.normal_rhs(n, 1), W.normal_rhs(n, 2)
    gx, gv = K.sla_matvec_grad(P, t(v), t(x), t(g))
    torch.cuda.synchronize()
    gxo, gvo = oracle.matvec_grad(A, x, g)
    assert np.array_equal(gx.cpu().numpy(), gxo) and np.array_equal(gv.cpu().numpy(), gvo)
    # eigsh and the eigenvalue gradient on the symmetric Poisson values
    rp, c, v = W.poisson_csr(N, np.int64)
    A = oracle.CSR(n, rp, c, v)
    P = csr_handle(rp, c)
    v0 = W.normal_rhs(n, 4)
    th, X, res, infos = K.sla_eigsh(P, t(v), 3, "LA", 200, t(v0))
    torch.cuda.synchronize()
    tho, Xo, _ = oracle.eigsh(A, 3, "LA", v0, 200)
    assert np.max(np.abs(th.cpu().numpy() - tho)) <= 1e-9
    gv = K.sla_eig_grad(P, t(v), X[2:3].contiguous(), t(np.ones(1)))
    torch.cuda.synchronize()
    assert np.array_equal(gv.cpu().numpy(), oracle.eig_grad(A, X[2].cpu().numpy()))
    # BiCGStab
    rp, c, v = W.convection_diffusion_csr(N, rowptr_dtype=np.int64)
    A = oracle.CSR(n, rp, c, v)
    P = csr_handle(rp, c)
    b = W.normal_rhs(n, 5)
    xg, info = K.sla_bicgstab_solve(P, t(v), t(b), 1e-12, 3000)
    torch.cuda.synchronize()
    xo, io = oracle.bicgstab(A, b, 1e-12, 3000)
    assert info[0].converged and rel(xg.cpu().numpy(), xo) <= TOL_X
    # a list mixing int64 and int32 handles
    rp2, c2, v2 = W.poisson_csr(25)
    P2 = csr_handle(rp2, c2)
    b2 = W.normal_rhs(625, 6)
    xs, infos = K.sla_solve_list([P, P2], [t(v), t(v2)], [t(b), t(b2)], 1e-12, 3000,
                                 method="bicgstab")
    torch.cuda.synchronize()
    assert rel(xs[0].cpu().numpy(), xo) <= TOL_X
    xo2, _ = oracle.bicgstab(oracle.CSR(625, rp2.astype(np.int64), c2, v2), b2, 1e-12, 3000)
    assert rel(xs[1].cpu().numpy(), xo2) <= TOL_X


def test_batched_autograd_eigsh_and_bicgstab():
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 30
    n = N * N
    rp, c, v = W.poisson_csr(N)
    rows = np.repeat(np.arange(n), np.diff(rp))
    vb = np.stack([v, 0.5 * v + np.where(rows == c, 0.3, 0.0)])
    P = csr_handle(rp, c)
    vals = t(vb).requires_grad_(True)
    v0 = t(np.stack([W.normal_rhs(n, 7), W.normal_rhs(n, 8)]))
    th, X = K.SparseTensor(P, vals).eigsh(k=1, which="LA", m=n, v0=v0)
    th.sum().backward()
    for s in range(2):
        A = oracle.CSR(n, rp.astype(np.int64), c, vb[s])
        tho, Xo, _ = oracle.eigsh(A, 1, "LA", v0[s].cpu().numpy(), n)
        assert abs(th[s, 0].item() - tho[0]) <= 1e-10
        assert rel(vals.grad[s].cpu().numpy(), oracle.eig_grad(A, Xo[0])) <= 1e-8
    # BiCGStab: values [2, nnz], b [2, n]
    rp, c, v = W.convection_diffusion_csr(N)
    rows = np.repeat(np.arange(n), np.diff(rp))
    vb = np.stack([v, v + np.where(rows == c, 20.0, 0.0)])
    P = csr_handle(rp, c)
    vals = t(vb).requires_grad_(True)
    b = np.stack([W.normal_rhs(n, 9), W.normal_rhs(n, 10)])
    g = np.stack([W.normal_rhs(n, 11), W.normal_rhs(n, 12)])
    bt = t(b).requires_grad_(True)
    x = K.SparseTensor(P, vals).solve(bt, tol=1e-12, maxit=3000, method="bicgstab")
    (x * t(g)).sum().backward()
    for s in range(2):
        A = oracle.CSR(n, rp.astype(np.int64), c, vb[s])
        xo, _ = oracle.bicgstab(A, b[s], 1e-12, 3000)
        lo, gvo, _ = oracle.adjoint_bicgstab(A, xo, g[s], 1e-12, 3000)
        assert rel(x[s].detach().cpu().numpy(), xo) <= TOL_X
        assert rel(bt.grad[s].cpu().numpy(), lo) <= TOL_X
        assert rel(vals.grad[s].cpu().numpy(), gvo) <= TOL_GRAD
