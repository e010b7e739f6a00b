"""Jacobi-preconditioned CG on the GPU (SLA_FLAG_JACOBI) against the
oracle's pcg_jacobi / adjoint_jacobi: the exact identity with CG when the
diagonal is 4, badly scaled matrices, the random geometric graph, every
SpMV-step kernel family, the batch, statuses, reproducibility, autograd."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_GRAD, TOL_X, csr_handle, iters_close, rel, say, t

pytestmark = pytest.mark.gpu


def _scaled_spd(n, seed, per_row=8, spread=2.0):
    """S M S for a random sparse diagonally dominant SPD M, S = diag(10^U(-spread, spread));
    values symmetric bit for bit."""
    import scipy.sparse as sp
    rng = np.random.default_rng(seed)
    m = n * per_row // 2
    i = rng.integers(0, n, m)
    j = rng.integers(0, n, m)
    keep = i != j
    i, j = i[keep], j[keep]
    w = rng.uniform(-1, 1, i.shape[0])
    U = sp.coo_matrix((w, (np.minimum(i, j), np.maximum(i, j))), shape=(n, n)).tocsr()
    U.sum_duplicates()
    M = (U + U.T).tocsr()
    M.sum_duplicates()
    diag = np.asarray(abs(M).sum(axis=1)).ravel() + rng.uniform(0.5, 1.5, n)
    M = (M + sp.diags(diag)).tocsr()
    M.sort_indices()
    sd = 10.0 ** rng.uniform(-spread, spread, n)
    rows = np.repeat(np.arange(n), np.diff(M.indptr))
    vals = M.data * (sd[rows] * sd[M.indices])
    return M.indptr.astype(np.int32), M.indices.astype(np.int32), vals


def _pair(rp, c, v, b, g, tol, maxit, variant="auto"):
    import torch
    import krylov_solvers_adjoint_amd as K
    P = csr_handle(rp, c)
    P.set_spmv_variant(variant)
    vt = t(v)
    x, info = K.sla_cg_solve(P, vt, t(b), tol, maxit, jacobi=True)
    gb, gv, ai = K.sla_cg_adjoint(P, vt, x, t(g), tol, maxit, jacobi=True)
    torch.cuda.synchronize()
    return x.cpu().numpy(), info, gb.cpu().numpy(), gv.cpu().numpy(), ai


def _check_vs_oracle(name, rp, c, v, b, g, tol, maxit, variant="auto"):
    n = len(rp) - 1
    x, info, gb, gv, ai = _pair(rp, c, v, b, g, tol, maxit, variant)
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    xo, io = oracle.pcg_jacobi(A, b, tol, maxit)
    gbo, gvo, aio = oracle.adjoint_jacobi(A, xo, g, tol, maxit)
    say(f"{name}: jacobi iterations {info.iterations}/{io.iterations} adj "
        f"{ai.iterations}/{aio.iterations}; x {rel(x, xo):.1e} lam {rel(gb, gbo):.1e} "
        f"gv {rel(gv, gvo):.1e}")
    assert io.status == oracle.OK and aio.status == oracle.OK
    assert iters_close(info.iterations, io.iterations)
    assert iters_close(ai.iterations, aio.iterations)
    assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD
    return x, info


@pytest.mark.parametrize("N,one_group", [(40, "off"), (40, "auto"), (1000, "off")])
def test_uniform_diagonal_is_cg_bit_for_bit(N, one_group):
    """Diagonal 4: z = r/4 rescales everything by powers of two, so the
    preconditioned iterates, beta and r.r are CG's exactly (row-order kernel
    and the one-workgroup loop at 40^2, line walk at 1000^2: the resident
    grid loop, which unpreconditioned 1000^2 would take, has no Jacobi form)."""
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.poisson_csr(N, np.int32)
    b = W.uniform_rhs(N * N, 40)
    P = csr_handle(rp, c, one_group=one_group)
    vt = t(v)
    x1, i1 = K.sla_cg_solve(P, vt, t(b), 1e-10, 3000, history=True)
    h1 = P.history()
    x2, i2 = K.sla_cg_solve(P, vt, t(b), 1e-10, 3000, history=True, jacobi=True)
    h2 = P.history()
    torch.cuda.synchronize()
    assert i1.iterations == i2.iterations
    assert torch.equal(x1, x2)
    assert np.array_equal(h1[1], h2[1]) and np.array_equal(h1[2], h2[2])
    assert np.array_equal(4.0 * h1[0], h2[0])


@pytest.mark.parametrize("seed", [1, 2])
def test_scaled_spd_against_oracle(seed):
    rp, c, v = _scaled_spd(5000, seed)
    n = len(rp) - 1
    _check_vs_oracle(f"scaled spd {seed}", rp, c, v, W.normal_rhs(n, 41), W.normal_rhs(n, 42),
                     1e-10, 20000)


def test_random_geometric_graph_fewer_iterations():
    import torch
    import krylov_solvers_adjoint_amd as K
    n = 60000
    row, col, val, _ = W.rgg_coo(n, 4, 5)
    rp, c, perm = oracle.csr_from_coo(n, row, col)
    v = oracle.values_from_coo(perm, int(rp[-1]), val)
    b = W.normal_rhs(n, 6)
    g = W.normal_rhs(n, 7)
    rp32 = rp.astype(np.int32)
    x, info = _check_vs_oracle("rgg60k", rp32, c, v, b, g, 1e-8, 20000)
    P = csr_handle(rp32, c)
    _, icg = K.sla_cg_solve(P, t(v), t(b), 1e-8, 20000)
    torch.cuda.synchronize()
    say(f"rgg60k: CG {icg.iterations} iterations, Jacobi {info.iterations}")
    assert info.iterations < icg.iterations


@pytest.mark.parametrize("variant", ["banded", "split", "csr"])
def test_kernel_families(variant):
    """The 3D 7-point Laplacian with a varying diagonal through the banded,
    split and CSR SpMV steps."""
    rp, c, v = W.laplacian3d_csr(24)
    n = len(rp) - 1
    rows = np.repeat(np.arange(n), np.diff(rp))
    v = v.copy()
    v[c == rows] += np.linspace(0.0, 30.0, n)
    _check_vs_oracle(f"3d {variant}", rp, c, v, W.uniform_rhs(n, 43), W.normal_rhs(n, 44),
                     1e-10, 5000, variant)


def test_batched_shifted_poisson():
    import torch
    import krylov_solvers_adjoint_amd as K
    N, B = 64, 6
    rowptr, col, vals, b, shifts = W.batched_poisson(N, B, 2, 3)
    vals = vals.copy()
    # a varying diagonal per system, so that the preconditioner matters
    rows = np.repeat(np.arange(N * N), np.diff(rowptr))
    for s in range(B):
        vals[s, col == rows] += np.linspace(0.0, 5.0 * (s + 1), N * N)
    P = csr_handle(rowptr, col)
    x, infos = K.sla_cg_solve_batched(P, t(vals), t(b), 1e-10, 5000, jacobi=True)
    torch.cuda.synchronize()
    x = x.cpu().numpy()
    for s in range(B):
        A = oracle.CSR(N * N, rowptr.astype(np.int64), col, vals[s])
        xo, io = oracle.pcg_jacobi(A, b[s], 1e-10, 5000)
        assert iters_close(infos[s].iterations, io.iterations), s
        assert rel(x[s], xo) <= TOL_X, s


def test_statuses_and_reproducibility():
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.poisson_csr(30, np.int32)
    n = 900
    b = W.uniform_rhs(n, 45)
    P = csr_handle(rp, c)
    rows = np.repeat(np.arange(n), np.diff(rp))
    bad = v.copy()
    bad[np.flatnonzero(c == rows)[17]] = 0.0
    x, info = K.sla_cg_solve(P, t(bad), t(b), 1e-10, 100, jacobi=True, check=False)
    torch.cuda.synchronize()
    assert info.status == K.ERR_NOT_SPD and info.iterations == 0
    # the flag is cleared: the next solve on good values runs normally
    runs = []
    for _ in range(2):
        x, info = K.sla_cg_solve(P, t(v), t(b), 1e-10, 1000, jacobi=True)
        torch.cuda.synchronize()
        runs.append((x.cpu().numpy(), info.iterations))
        assert info.status == K.OK and info.converged
    assert np.array_equal(runs[0][0], runs[1][0]) and runs[0][1] == runs[1][1]


def test_autograd_jacobi():
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = _scaled_spd(2000, 5, spread=1.0)
    n = len(rp) - 1
    b = W.normal_rhs(n, 46)
    g = W.normal_rhs(n, 47)
    P = csr_handle(rp, c)
    vals = t(v).requires_grad_(True)
    bt = t(b).requires_grad_(True)
    x = K.SparseTensor(P, vals).solve(bt, tol=1e-12, maxit=20000, precond="jacobi")
    (x * t(g)).sum().backward()
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    xo, _ = oracle.pcg_jacobi(A, b, 1e-12, 20000)
    gbo, gvo, _ = oracle.adjoint_jacobi(A, xo, g, 1e-12, 20000)
    assert rel(x.detach().cpu().numpy(), xo) <= TOL_X
    assert rel(bt.grad.cpu().numpy(), gbo) <= TOL_X
    assert rel(vals.grad.cpu().numpy(), gvo) <= TOL_GRAD
