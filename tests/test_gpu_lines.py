"""The line-walk CG iteration (a band whose far offsets are +-L): the
automatic choice of the two-kernel loop for 2D stencils on grids with lines
of 961 points or more (the handles here keep that loop: single systems of up
to about a million unknowns would otherwise take the resident grid loop);
CG and the adjoint match the oracle, two runs give the same bits, and the
walk handles short last lines, lines that are not a multiple of 64 points,
a matrix whose length is not a multiple of L, and batches."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_GRAD, TOL_X, csr_handle, iters_close, rel, say, t

pytestmark = pytest.mark.gpu


def _solve(rp, c, v, b, g, tol, maxit, variant="auto", wg=2):
    import torch
    import krylov_solvers_adjoint_amd as K
    P = csr_handle(rp, c, one_group="off")
    P.set_workgroups_per_cu(wg)
    P.set_spmv_variant(variant)
    lines = P.lines
    vt = t(v)
    x, info = K.sla_cg_solve(P, vt, t(b), tol, maxit)
    gb, gv, ai = K.sla_cg_adjoint(P, vt, x, t(g), tol, maxit)
    torch.cuda.synchronize()
    return lines, x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy(), info, ai


def _check(name, rp, c, v, b, g, tol, maxit, wg=2):
    n = len(rp) - 1
    lines, x, gb, gv, info, ai = _solve(rp, c, v, b, g, tol, maxit, wg=wg)
    assert lines, "the line walk should apply"
    again = _solve(rp, c, v, b, g, tol, maxit, wg=wg)
    assert np.array_equal(x, again[1]) and np.array_equal(gb, again[2])
    assert np.array_equal(gv, again[3]) and info.iterations == again[4].iterations
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    xo, io = oracle.cg(A, b, tol, maxit)
    gbo, gvo, aio = oracle.adjoint(A, xo, g, tol, maxit)
    say(f"{name}: iterations {info.iterations}/{io.iterations} adj {ai.iterations}/"
        f"{aio.iterations}; x {rel(x, xo):.1e} lam {rel(gb, gbo):.1e} gv {rel(gv, gvo):.1e}")
    assert iters_close(info.iterations, io.iterations)
    assert iters_close(ai.iterations, aio.iterations)
    assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD


@pytest.mark.parametrize("N", [961, 1000, 1024])
def test_poisson_line_walk(N):
    """Grid lines of 961 (15 full tiles + 1 point), 1000 and 1024 points."""
    rp, c, v = W.poisson_csr(N, np.int32)
    b = W.uniform_rhs(N * N, 21)
    g = W.normal_rhs(N * N, 22)
    _check(f"poisson{N}", rp, c, v, b, g, 0.0, 60)


@pytest.mark.parametrize("n,L", [(1000 * 37 + 500, 1000), (5000 * 6 + 123, 5000),
                                 (1100 * 3 + 1, 1100)])
def test_band_short_last_line(n, L):
    """Couplings +-1 and +-L across line ends; n not a multiple of L."""
    rp, c, v = W.band_csr(n, [-L, -1, 1, L], 4.5)
    b = W.uniform_rhs(n, 23)
    g = W.normal_rhs(n, 24)
    _check(f"band n={n} L={L}", rp, c, v, b, g, 1e-10, 5000)


def test_line_walk_one_workgroup_per_cu():
    rp, c, v = W.poisson_csr(1200, np.int32)
    b = W.uniform_rhs(1200 * 1200, 25)
    g = W.normal_rhs(1200 * 1200, 26)
    _check("poisson1200 wg1", rp, c, v, b, g, 0.0, 40, wg=1)


def test_line_walk_int64_rowptr_and_fallback():
    """int64 row pointers take the walk too; a band with two far offset
    magnitudes (L and L + 1) keeps the row-order banded kernel."""
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.poisson_csr(1000, np.int64)
    b = W.uniform_rhs(1000 * 1000, 27)
    g = W.normal_rhs(1000 * 1000, 28)
    _check("poisson1000 i64", rp, c, v, b, g, 0.0, 30)
    rp7, c7, v7 = W.band_csr(100000, [-1001, -1000, -1, 1, 1000, 1001], 6.5)
    P = csr_handle(rp7, c7)
    assert P.banded and not P.lines


def test_line_walk_vs_banded_same_iterates():
    """The walk and the row-order banded kernel compute the same iteration;
    only the order of the p.Ap partial sums differs."""
    N = 1000
    rp, c, v = W.poisson_csr(N, np.int32)
    b = W.uniform_rhs(N * N, 29)
    g = W.normal_rhs(N * N, 30)
    la = _solve(rp, c, v, b, g, 0.0, 200, variant="lines")
    ba = _solve(rp, c, v, b, g, 0.0, 200, variant="banded")
    assert la[0] and not ba[0]
    assert rel(la[1], ba[1]) <= 1e-11 and rel(la[2], ba[2]) <= 1e-11


@pytest.mark.parametrize("n,L,wg", [(1000 * 1599 + 371, 1000, 1), (961 * 3200 + 5, 961, 2)])
def test_long_chunks_short_last_line(n, L, wg):
    """Walks of a dozen lines or more per chunk (1600 lines over 8 XCDs x 16
    chunks; 3201 lines over 8 x 32), which keep two tiles of loads in flight,
    with a short last line and couplings across line ends."""
    rp, c, v = W.band_csr(n, [-L, -1, 1, L], 4.5)
    b = W.uniform_rhs(n, 27)
    g = W.normal_rhs(n, 28)
    _check(f"band n={n} L={L} wg={wg}", rp, c, v, b, g, 1e-10, 5000, wg=wg)


def test_poisson_long_chunks():
    """Poisson 1700^2 with one workgroup per CU: 26 lines per chunk."""
    rp, c, v = W.poisson_csr(1700, np.int32)
    b = W.uniform_rhs(1700 * 1700, 29)
    g = W.normal_rhs(1700 * 1700, 30)
    _check("poisson1700 wg1", rp, c, v, b, g, 0.0, 40, wg=1)


@pytest.mark.parametrize("N", [1000, 1700])
@pytest.mark.parametrize("maxit", [1, 2, 3, 4, 7, 8])
def test_paired_x_updates_fixed_stops(maxit, N):
    """The walk applies x's deferred updates two steps at a time: solves cut
    off after an odd or an even number of iterations (the last pass adding
    one or two pending updates) and their adjoints against the oracle.  At
    one workgroup per CU, 1000^2 gives ~7 lines per chunk (the one-tile
    look-ahead walk) and 1700^2 gives 26 (the two-deep pipelined walk, the
    one the 16M grid takes)."""
    rp, c, v = W.poisson_csr(N)
    A = oracle.CSR(N * N, rp.astype(np.int64), c, v)
    b = W.uniform_rhs(N * N, 31)
    g = W.normal_rhs(N * N, 32)
    lines, x, gb, gv, info, ai = _solve(rp, c, v, b, g, 0.0, maxit, wg=1)
    assert lines and info.iterations == maxit == ai.iterations
    xo, _ = oracle.cg(A, b, 0.0, maxit)
    gbo, gvo, _ = oracle.adjoint(A, xo, g, 0.0, maxit)
    say(f"maxit {maxit}: x {rel(x, xo):.1e} grad_b {rel(gb, gbo):.1e}")
    assert rel(x, xo) <= 1e-12 and rel(gb, gbo) <= 1e-12 and rel(gv, gvo) <= 1e-12


def test_paired_x_updates_breakdown_at_odd_step():
    """An indefinite shift of the 1000^2 Laplacian breaks down (p.Ap <= 0)
    at an odd step, found by the residual step, which then adds the update
    the walk left pending: status, iteration and x against the oracle."""
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 1000
    rp, c, v = W.poisson_csr(N)
    rows = np.repeat(np.arange(N * N), np.diff(rp))
    vs = v - np.where(rows == c, 0.05, 0.0)
    b = W.uniform_rhs(N * N, 0)
    P = csr_handle(rp, c, one_group="off")
    assert P.lines
    x, info = K.sla_cg_solve(P, t(vs), t(b), 1e-8, 5000, check=False)
    torch.cuda.synchronize()
    A = oracle.CSR(N * N, rp.astype(np.int64), c, vs)
    xo, io = oracle.cg(A, b, 1e-8, 5000)
    say(f"shift -0.05: status {info.status} it {info.iterations} (oracle {io.status} "
        f"{io.iterations}) x {rel(x.cpu().numpy(), xo):.1e}")
    assert info.status == K.ERR_NOT_SPD == io.status
    assert info.iterations == io.iterations and info.iterations % 2 == 1
    assert rel(x.cpu().numpy(), xo) <= 1e-10
