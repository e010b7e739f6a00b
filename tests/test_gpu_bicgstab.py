"""BiCGStab on the GPU (non-symmetric systems) and its adjoint against the
oracle: convection-diffusion grids up to the 10^6-unknown size, random
non-symmetric CSR matrices, fixed iteration counts, warm starts, the batch,
the half-step finish, breakdown and non-finite statuses, and the autograd
node."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_GRAD, TOL_X, csr_handle, rel, say, t

pytestmark = pytest.mark.gpu

# BiCGStab's residual norm is not monotone: near the tolerance it
# oscillates, and which oscillation first dips below tol moves with the
# rounding.  The oracle itself shows it: b changed by one ulp in 5 entries
# moves its count from 747 to 771-907 (300^2 grid, tol 1e-12) and from 1801
# to 1648-2081 (1000^2, tol 1e-8).  So the GPU's count is held to the
# oracle's own spread over such perturbations (widened by 10 %) where the
# oracle is cheap, to 10 % on small and easy systems, and to 25 % at
# 10^6 unknowns; x is held to TOL_X at tol 1e-12.
ITER_FRAC_BICGSTAB = 0.10


def iters_close(a: int, b: int, frac: float = ITER_FRAC_BICGSTAB) -> bool:
    return abs(a - b) <= max(1, frac * max(a, b))


def oracle_spread(A, b, tol, maxit):
    """The oracle's iteration counts for b and three copies with 5 entries
    moved by one ulp."""
    its = []
    for k in range(4):
        bp = b.copy()
        if k:
            idx = np.random.default_rng(k).integers(0, b.shape[0], 5)
            bp[idx] = np.nextafter(bp[idx], np.inf)
        its.append(oracle.bicgstab(A, bp, tol, maxit)[1].iterations)
    return min(its), max(its)


def _nonsym(n, per_row, seed):
    """Random non-symmetric, diagonally dominant CSR (ascending columns) with
    a few rows holding only their diagonal."""
    rng = np.random.default_rng(seed)
    rows, cols, vals = [], [], []
    for i in range(n):
        cs = np.unique(rng.integers(0, n, rng.integers(0, 2 * per_row)))
        cs = cs[cs != i]
        off = rng.uniform(-1, 1, cs.shape[0])
        allc = np.append(cs, i)
        allv = np.append(off, np.abs(off).sum() + rng.uniform(0.5, 1.5))
        o = np.argsort(allc)
        rows.append(np.full(allc.shape[0], i))
        cols.append(allc[o])
        vals.append(allv[o])
    rows, cols, vals = np.concatenate(rows), np.concatenate(cols), np.concatenate(vals)
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    return np.cumsum(rp).astype(np.int32), cols.astype(np.int32), vals


def _solve_both(rp, c, v, b, tol, maxit, x0=None):
    import torch
    import krylov_solvers_adjoint_amd as K
    n = len(rp) - 1
    P = csr_handle(rp, c)
    x, infos = K.sla_bicgstab_solve(P, t(v), t(b), tol, maxit,
                                    x0=t(x0) if x0 is not None else None, history=True)
    torch.cuda.synchronize()
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    xo, io, ho = oracle.bicgstab(A, b, tol, maxit, x0=x0, history=True)
    return P, A, x.cpu().numpy(), infos[0], xo, io, ho


# Converged solutions to a relative residual tol differ by up to about
# cond(A) tol, so parity of x is checked at tol 1e-12 (cond of these
# matrices stays below 1e4).
@pytest.mark.parametrize("N,tol,maxit", [(1, 1e-12, 10), (30, 1e-12, 2000), (97, 1e-12, 3000),
                                         (300, 1e-12, 6000)])
def test_convection_diffusion(N, tol, maxit):
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.convection_diffusion_csr(N)
    b = W.normal_rhs(N * N, 90)
    P, A, x, info, xo, io, ho = _solve_both(rp, c, v, b, tol, maxit)
    rho, alpha, omega, rr = K.sla_bicgstab_history(P)
    k = min(len(rr), len(ho[3]))
    apart = np.nonzero(np.abs(rr[:k] - ho[3][:k]) > 1e-6 * ho[3][:k])[0]
    say(f"N={N}: gpu {info.iterations} it (conv {info.converged}), oracle {io.iterations}; "
        f"rel {rel(x, xo):.2e}; r.r histories within 1e-6 up to iteration "
        f"{apart[0] if apart.size else k}")
    assert info.status == K.OK and info.converged and io.converged
    lo, hi = oracle_spread(A, b, tol, maxit)
    say(f"  oracle spread under 1-ulp perturbations of b: {lo} .. {hi}")
    assert 0.9 * lo - 1 <= info.iterations <= 1.1 * hi + 1
    assert rel(x, xo) <= TOL_X
    # the first iterations' scalars agree closely (rounding differs only in
    # the association of the dot products)
    k = min(10, len(rho), len(ho[0]))
    for g_, o_ in zip((rho, alpha, omega, rr), ho):
        assert np.allclose(g_[:k], o_[:k], rtol=1e-9, atol=0.0)


@pytest.mark.parametrize("n,per_row,seed", [(1, 1, 0), (257, 4, 1), (5000, 6, 2)])
def test_random_nonsymmetric(n, per_row, seed):
    import krylov_solvers_adjoint_amd as K
    rp, c, v = _nonsym(n, per_row, seed)
    b = W.normal_rhs(n, 91)
    _, _, x, info, xo, io, _ = _solve_both(rp, c, v, b, 1e-10, 1000)
    assert info.status == K.OK and info.converged
    assert iters_close(info.iterations, io.iterations)
    assert rel(x, xo) <= TOL_X


def test_fixed_iterations_and_warm_start():
    import krylov_solvers_adjoint_amd as K
    N = 64
    rp, c, v = W.convection_diffusion_csr(N)
    b = W.normal_rhs(N * N, 92)
    # 20 iterations are launched one by one: x against the oracle
    P, _, x, info, xo, io, _ = _solve_both(rp, c, v, b, 0.0, 20)
    assert info.iterations == 20 == io.iterations and not info.converged
    assert rel(x, xo) <= TOL_X
    h20 = K.sla_bicgstab_history(P)
    # 40 and 45 run as graph-captured blocks of 16 iterations, the last block
    # cut short by the limit: the same kernels in the same order, so the
    # first 20 iterations' scalars are the direct launches' bit for bit (past
    # ~30 iterations rounding alone separates BiCGStab trajectories, so the
    # unconverged x is not compared with the oracle there)
    for m in (40, 45):
        P, _, x, info, xo, io, _ = _solve_both(rp, c, v, b, 0.0, m)
        assert info.iterations == m == io.iterations and not info.converged
        h = K.sla_bicgstab_history(P)
        for a_, b_ in zip(h, h20):
            assert len(a_) == m and np.array_equal(a_[:20], b_)
    x0 = W.uniform_rhs(N * N, 93)
    _, _, x, info, xo, io, _ = _solve_both(rp, c, v, b, 1e-9, 1000, x0=x0)
    assert info.converged and iters_close(info.iterations, io.iterations)
    assert rel(x, xo) <= TOL_X


def test_half_step_finish_and_statuses():
    import torch
    import krylov_solvers_adjoint_amd as K
    # A = 2 I: one iteration, finished on the half step, x = alpha b with
    # alpha = rhat.r / rhat.v = 1/2 up to one rounding: the two dot products
    # are summed by different kernels along different trees, so exact halving
    # holds for some right-hand sides only
    n = 1000
    rp = np.arange(n + 1, dtype=np.int32)
    c = np.arange(n, dtype=np.int32)
    b = W.uniform_rhs(n, 94)
    P = csr_handle(rp, c)
    x, infos = K.sla_bicgstab_solve(P, t(np.full(n, 2.0)), t(b), 1e-10, 10)
    torch.cuda.synchronize()
    assert infos[0].iterations == 1 and infos[0].converged
    xh = x.cpu().numpy()
    assert np.all(np.abs(xh - 0.5 * b) <= 2.0 ** -51 * np.abs(0.5 * b))
    # b = 0: converged before the first iteration, x = 0
    rp, c, v = W.convection_diffusion_csr(12)
    P = csr_handle(rp, c)
    x, infos = K.sla_bicgstab_solve(P, t(v), t(np.zeros(144)), 1e-8, 10)
    torch.cuda.synchronize()
    assert infos[0].iterations == 0 and infos[0].converged and not torch.any(x)
    # a rotation: rhat.v = 0 at once
    R = csr_handle(np.array([0, 1, 2], np.int32), np.array([1, 0], np.int32))
    _, infos = K.sla_bicgstab_solve(R, t(np.array([1.0, -1.0])), t(np.array([1.0, 0.0])),
                                    1e-8, 10, check=False)
    assert infos[0].status == K.ERR_BREAKDOWN and infos[0].iterations == 0
    with pytest.raises(K.SlaError) as e:
        K.sla_bicgstab_solve(R, t(np.array([1.0, -1.0])), t(np.array([1.0, 0.0])), 1e-8, 10)
    assert e.value.status == K.ERR_BREAKDOWN
    # a NaN value
    vb = v.copy()
    vb[7] = np.nan
    _, infos = K.sla_bicgstab_solve(P, t(vb), t(W.uniform_rhs(144, 95)), 1e-8, 10, check=False)
    assert infos[0].status == K.ERR_NONFINITE
    # maxit = 0
    _, infos = K.sla_bicgstab_solve(P, t(v), t(W.uniform_rhs(144, 95)), 1e-8, 0)
    assert infos[0].iterations == 0 and not infos[0].converged


def test_batch():
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 40
    rp, c, v = W.convection_diffusion_csr(N)
    rows = np.repeat(np.arange(N * N), np.diff(rp))
    vb = np.stack([v, v + np.where(rows == c, 50.0, 0.0), 2.0 * v])
    b = np.stack([W.normal_rhs(N * N, 96 + s) for s in range(3)])
    P = csr_handle(rp, c)
    x, infos = K.sla_bicgstab_solve(P, t(vb), t(b), 1e-10, 2000)
    torch.cuda.synchronize()
    x = x.cpu().numpy()
    for s in range(3):
        A = oracle.CSR(N * N, rp.astype(np.int64), c, vb[s])
        xo, io = oracle.bicgstab(A, b[s], 1e-10, 2000)
        assert infos[s].converged and iters_close(infos[s].iterations, io.iterations)
        assert rel(x[s], xo) <= TOL_X


def test_adjoint_against_oracle():
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 50
    rp, c, v = W.convection_diffusion_csr(N)
    n = N * N
    b = W.normal_rhs(n, 97)
    g = W.normal_rhs(n, 98)
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    xo, _ = oracle.bicgstab(A, b, 1e-12, 3000)
    lo, gvo, io = oracle.adjoint_bicgstab(A, xo, g, 1e-12, 3000)
    P = csr_handle(rp, c)
    lam, gv, infos = K.sla_bicgstab_adjoint(P, t(v), t(xo), t(g), 1e-12, 3000)
    torch.cuda.synchronize()
    assert infos[0].converged and iters_close(infos[0].iterations, io.iterations)
    assert rel(lam.cpu().numpy(), lo) <= TOL_X
    assert rel(gv.cpu().numpy(), gvo) <= TOL_GRAD


def test_autograd_node():
    """L = g.x through SparseTensor.solve(method="bicgstab"): the gradients
    in b and in the values against the oracle's adjoint."""
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = _nonsym(3000, 5, 7)
    n = 3000
    b = W.normal_rhs(n, 99)
    g = W.normal_rhs(n, 100)
    P = csr_handle(rp, c)
    vals = t(v).requires_grad_(True)
    bt = t(b).requires_grad_(True)
    x = K.SparseTensor(P, vals).solve(bt, tol=1e-12, maxit=2000, method="bicgstab")
    (x * t(g)).sum().backward()
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    xo, _ = oracle.bicgstab(A, b, 1e-12, 2000)
    lo, gvo, _ = oracle.adjoint_bicgstab(A, xo, g, 1e-12, 2000)
    assert rel(x.detach().cpu().numpy(), xo) <= TOL_X
    assert rel(bt.grad.cpu().numpy(), lo) <= TOL_X
    assert rel(vals.grad.cpu().numpy(), gvo) <= TOL_GRAD


def test_symmetric_matches_cg():
    """On the SPD Poisson matrix BiCGStab and CG reach the same solution."""
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 60
    rp, c, v = W.poisson_csr(N)
    b = W.uniform_rhs(N * N, 0)
    P = csr_handle(rp, c)
    xb, ib = K.sla_bicgstab_solve(P, t(v), t(b), 1e-12, 2000)
    xc, ic = K.sla_cg_solve(P, t(v), t(b), 1e-12, 2000)
    torch.cuda.synchronize()
    assert ib[0].converged and ic.converged
    assert rel(xb.cpu().numpy(), xc.cpu().numpy()) <= 1e-9


def test_fullsize_convection_diffusion():
    """The 1000 x 1000 grid (10^6 unknowns) to tol 1e-8, as the bench runs
    it, with the oracle beside it (about 1800 iterations): iteration counts
    within 25 % (the oracle's own spread there is -8 % .. +16 %), the true
    residual of the GPU's x within the tolerance, and x as close to the
    oracle's as two solutions of that residual can be."""
    N = 1000
    rp, c, v = W.convection_diffusion_csr(N)
    b = W.normal_rhs(N * N, 90)
    oracle.set_threads(16)
    _, A, x, info, xo, io, _ = _solve_both(rp, c, v, b, 1e-8, 5000)
    true = np.linalg.norm(b - oracle.spmv(A, x)) / np.linalg.norm(b)
    say(f"1000^2: gpu {info.iterations} it, oracle {io.iterations}, rel {rel(x, xo):.2e}, "
        f"true residual {true:.2e}")
    assert info.converged and iters_close(info.iterations, io.iterations, 0.25)
    assert true <= 1.5e-8
    assert rel(x, xo) <= 1e-4


@pytest.mark.parametrize("N", [1000, 2000])
def test_fullsize_convection_diffusion_first_iterations(N):
    """The same 10^6-unknown grid (and 2000^2, whose SpMVs take the 8-wave
    form with the fused dot partials), 20 fixed iterations (tol 0): x within
    1e-8 of the oracle's and rho, alpha, omega, r.r of every iteration within
    1e-7.  BiCGStab on this matrix is chaotic under rounding (one-ulp changes
    of five entries of b move the oracle's own x by 1e-11 after 20
    iterations and by 4e-2 after 50), so element-wise parity is checked where
    it is defined, and the converged solve above by its residual."""
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.convection_diffusion_csr(N)
    b = W.normal_rhs(N * N, 90)
    oracle.set_threads(oracle.host_threads())
    P, A, x, info, xo, io, ho = _solve_both(rp, c, v, b, 0.0, 20)
    rho, alpha, omega, rr = K.sla_bicgstab_history(P)
    assert info.iterations == io.iterations == 20 and len(rr) == 20
    d = [float(np.max(np.abs(g - o) / np.abs(o))) for g, o in zip((rho, alpha, omega, rr), ho)]
    say(f"{N}^2, 20 iterations: x {rel(x, xo):.1e}; rho/alpha/omega/rr {max(d):.1e}")
    assert rel(x, xo) <= TOL_X and max(d) <= 1e-7
