"""The resident grid CG loop (single banded systems of 2049 to about a
million unknowns held in registers and LDS, one cooperative launch per
solve): Poisson grids from 46^2 (46 workgroups of one grid line) and 100^2
to the 1000^2 workload (eight rows per thread), a band whose length is not a
multiple of the workgroups' rows, fixed and converged stops, warm starts,
history, statuses and the adjoint's refusal, rough coefficients (thousands
of iterations), against the oracle; two runs
give the same bits; the two-kernel loop agrees within rounding."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_GRAD, TOL_X, csr_handle, iters_close, rel, say, t

pytestmark = pytest.mark.gpu


def _A(rp, c, v):
    return oracle.CSR(len(rp) - 1, np.asarray(rp, np.int64), np.asarray(c, np.int32),
                      np.asarray(v, np.float64))


def _resident(P) -> bool:
    """Whether the last solve on P ran the resident grid loop."""
    import krylov_solvers_adjoint_amd as K
    try:
        return K.sla_resident_loop_ms(P) > 0.0
    except K.SlaError:
        return False


def _solve_adjoint(P, v, b, g, tol, maxit):
    import torch
    import krylov_solvers_adjoint_amd as K
    vt = t(v)
    x, info = K.sla_cg_solve(P, vt, t(b), tol, maxit)
    gb, gv, ai = K.sla_cg_adjoint(P, vt, x, t(g), tol, maxit)
    torch.cuda.synchronize()
    return x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy(), info, ai


@pytest.mark.parametrize("N", [46, 100, 512, 600, 700, 1000])
def test_poisson_against_oracle(N):
    """Poisson N^2 to tol 1e-10, forward and adjoint, against the oracle; the
    same call twice gives the same bits."""
    import oracle as O
    O.set_threads(O.host_threads())
    n = N * N
    rp, c, v = W.poisson_csr(N)
    b = W.uniform_rhs(n, 0)
    g = W.normal_rhs(n, 1)
    P = csr_handle(rp, c)
    x, gb, gv, info, ai = _solve_adjoint(P, v, b, g, 1e-10, 20000)
    assert _resident(P), "the resident grid loop should apply"
    x2, gb2, gv2, info2, ai2 = _solve_adjoint(P, v, b, g, 1e-10, 20000)
    assert np.array_equal(x, x2) and np.array_equal(gb, gb2) and np.array_equal(gv, gv2)
    assert info.iterations == info2.iterations and ai.iterations == ai2.iterations
    A = _A(rp, c, v)
    xo, io = oracle.cg(A, b, 1e-10, 20000)
    gbo, gvo, aio = oracle.adjoint(A, xo, g, 1e-10, 20000)
    say(f"poisson{N}: it {info.iterations}/{io.iterations} adj {ai.iterations}/"
        f"{aio.iterations}; x {rel(x, xo):.1e} lam {rel(gb, gbo):.1e} gv {rel(gv, gvo):.1e}")
    assert info.converged and ai.converged
    assert iters_close(info.iterations, io.iterations)
    assert iters_close(ai.iterations, aio.iterations)
    assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD


def test_headline_fixed_iterations():
    """Poisson 1000^2, b = A u* (u* = sin(pi x) sin(pi y)), 1000 fixed
    iterations forward and adjoint (the headline step): against the oracle,
    and against the two-kernel loop within rounding."""
    import oracle as O
    O.set_threads(O.host_threads())
    N = 1000
    n = N * N
    rp, c, v = W.poisson_csr(N)
    A = _A(rp, c, v)
    _, b = W.manufactured(N)
    g = W.normal_rhs(n, 1)
    P = csr_handle(rp, c)
    x, gb, gv, info, ai = _solve_adjoint(P, v, b, g, 0.0, 1000)
    assert _resident(P)
    assert info.iterations == 1000 == ai.iterations
    Q = csr_handle(rp, c, one_group="off")
    xq, gbq, gvq, iq, aq = _solve_adjoint(Q, v, b, g, 0.0, 1000)
    assert not _resident(Q)
    xo, _ = oracle.cg(A, b, 0.0, 1000)
    gbo, gvo, _ = oracle.adjoint(A, xo, g, 0.0, 1000)
    say(f"1000 fixed: x {rel(x, xo):.1e} (two-kernel {rel(xq, xo):.1e}) lam {rel(gb, gbo):.1e} "
        f"gv {rel(gv, gvo):.1e}; vs two-kernel x {rel(x, xq):.1e}")
    assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD
    assert rel(x, xq) <= 1e-10 and rel(gb, gbq) <= 1e-10


@pytest.mark.parametrize("n,offs", [(300007, (-321, -1, 1, 321)), (270000, (-3, -2, -1, 1, 2, 3)),
                                    (400001, (-1000, -1, 1, 1000))])
def test_band_ragged_blocks(n, offs):
    """Bands whose length is not a multiple of the workgroups' rows (a short
    last block), three and seven offsets: CG and the adjoint against the
    oracle."""
    import oracle as O
    O.set_threads(O.host_threads())
    rp, c, v = W.band_csr(n, offs, 2.0 * len(offs) + 0.5)
    b = W.normal_rhs(n, 5)
    g = W.normal_rhs(n, 6)
    P = csr_handle(rp, c)
    x, gb, gv, info, ai = _solve_adjoint(P, v, b, g, 1e-11, 5000)
    assert _resident(P)
    A = _A(rp, c, v)
    xo, io = oracle.cg(A, b, 1e-11, 5000)
    gbo, gvo, aio = oracle.adjoint(A, xo, g, 1e-11, 5000)
    say(f"band n={n} offs={offs}: it {info.iterations}/{io.iterations} x {rel(x, xo):.1e}")
    assert iters_close(info.iterations, io.iterations)
    assert iters_close(ai.iterations, aio.iterations)
    assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD


@pytest.mark.parametrize("N,spread", [(300, 3.0), (640, 1.5), (1000, 1.0)])
def test_rough_coefficients_against_oracle(N, spread):
    """Diffusion with log-uniform edge conductances (a contrast of e^(2
    spread), thousands of iterations to 1e-10): the loop's single-reduction
    recurrences stay within the parity bounds of the oracle's two-sum CG on
    one, four and eight rows per thread, forward and adjoint."""
    import oracle as O
    O.set_threads(O.host_threads())
    rp, c, v = W.rough_diffusion_csr(N, 3, spread)
    n = N * N
    b = W.normal_rhs(n, 5)
    g = W.normal_rhs(n, 6)
    P = csr_handle(rp, c)
    x, gb, gv, info, ai = _solve_adjoint(P, v, b, g, 1e-10, 40000)
    assert _resident(P)
    A = _A(rp, c, v)
    xo, io = oracle.cg(A, b, 1e-10, 40000)
    gbo, gvo, aio = oracle.adjoint(A, xo, g, 1e-10, 40000)
    say(f"rough {N}^2 spread {spread}: it {info.iterations}/{io.iterations} adj "
        f"{ai.iterations}/{aio.iterations}; x {rel(x, xo):.1e} lam {rel(gb, gbo):.1e} "
        f"gv {rel(gv, gvo):.1e}")
    assert info.converged and ai.converged
    assert iters_close(info.iterations, io.iterations)
    assert iters_close(ai.iterations, aio.iterations)
    assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD


def test_warm_start_history_and_statuses():
    """Poisson 600^2: history against the oracle's alpha, beta, r.r; a warm
    start; -A (NOT_SPD before any update, x = x0 = 0); NaN in b (NONFINITE);
    b = 0; maxit = 0; tol = 0 (exactly maxit iterations)."""
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 600
    n = N * N
    rp, c, v = W.poisson_csr(N)
    A = _A(rp, c, v)
    b = W.uniform_rhs(n, 0)
    P = csr_handle(rp, c)
    x, info = K.sla_cg_solve(P, t(v), t(b), 1e-10, 5000, history=True)
    torch.cuda.synchronize()
    assert _resident(P)
    al, be, rr = P.history()
    xo, io, (ao, bo, ro) = oracle.cg(A, b, 1e-10, 5000, history=True)
    assert len(al) == info.iterations and iters_close(info.iterations, io.iterations)
    k = min(60, len(ao))
    assert rel(al[:k], ao[:k]) <= 1e-9 and rel(be[:k], bo[:k]) <= 1e-9
    assert rel(rr[:k], ro[:k]) <= 1e-9
    x0 = xo + 1e-3 * W.normal_rhs(n, 9)
    xw, iw = K.sla_cg_solve(P, t(v), t(b), 1e-10, 5000, x0=t(x0))
    torch.cuda.synchronize()
    xwo, iwo = oracle.cg(A, b, 1e-10, 5000, x0=x0)
    assert iters_close(iw.iterations, iwo.iterations)
    assert rel(xw.cpu().numpy(), xwo) <= TOL_X
    xn, inn = K.sla_cg_solve(P, t(-v), t(b), 1e-10, 100, check=False)
    torch.cuda.synchronize()
    assert inn.status == K.ERR_NOT_SPD and inn.iterations == 0
    assert float(xn.abs().max()) == 0.0
    bad = b.copy()
    bad[n // 2] = np.nan
    _, ib = K.sla_cg_solve(P, t(v), t(bad), 1e-10, 100, check=False)
    assert ib.status == K.ERR_NONFINITE
    xz, iz = K.sla_cg_solve(P, t(v), t(np.zeros(n)), 1e-10, 100)
    torch.cuda.synchronize()
    assert iz.iterations == 0 and iz.converged and float(xz.abs().max()) == 0.0
    _, im = K.sla_cg_solve(P, t(v), t(b), 1e-10, 0)
    assert im.iterations == 0 and not im.converged
    xf, itf = K.sla_cg_solve(P, t(v), t(b), 0.0, 37)
    torch.cuda.synchronize()
    xfo, ifo = oracle.cg(A, b, 0.0, 37)
    assert itf.iterations == 37 == ifo.iterations
    assert rel(xf.cpu().numpy(), xfo) <= 1e-12


def test_adjoint_refused_values():
    """Values that are not symmetric: the device-side check gates the
    resident loop and the pattern gradient (SLA_ERR_NOT_SYMMETRIC, grad_b and
    grad_vals untouched); the next call with symmetric values is solved."""
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 600
    n = N * N
    rp, c, v = W.poisson_csr(N)
    vn = v.copy()
    off = np.flatnonzero(vn != 4.0)
    vn[int(off[12345])] = -1.25
    b = W.uniform_rhs(n, 6)
    g = W.normal_rhs(n, 7)
    P = csr_handle(rp, c)
    x1, _ = K.sla_cg_solve(P, t(v), t(b), 1e-10, 5000)
    torch.cuda.synchronize()
    P.bind(t(vn))
    gb = torch.full((n,), 7.0, dtype=torch.float64, device=x1.device)
    gv = torch.full((v.shape[0],), 7.0, dtype=torch.float64, device=x1.device)
    info = K._Info()
    gx = t(g)
    st = K._lib.sla_cg_adjoint(P.handle, x1.data_ptr(), gx.data_ptr(), gb.data_ptr(),
                               gv.data_ptr(), 1e-10, 5000, 0, ctypes_byref(info), None)
    torch.cuda.synchronize()
    assert st == K.ERR_NOT_SYMMETRIC and info.status == K.ERR_NOT_SYMMETRIC
    assert info.iterations == 0
    assert bool((gb == 7.0).all()) and bool((gv == 7.0).all())
    A = _A(rp, c, v)
    xo, _ = oracle.cg(A, b, 1e-10, 5000)
    gbo, gvo, aio = oracle.adjoint(A, xo, g, 1e-10, 5000)
    gb, gv, ai = K.sla_cg_adjoint(P, t(v), x1, gx, 1e-10, 5000)
    torch.cuda.synchronize()
    assert _resident(P)
    assert rel(gb.cpu().numpy(), gbo) <= TOL_X and rel(gv.cpu().numpy(), gvo) <= TOL_GRAD


def test_resident_loop_time_query():
    """sla_resident_loop_ms: SLA_ERR_ARG before any resident loop, the
    launch's duration afterwards; Jacobi and batches keep the two-kernel
    loop."""
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 520
    n = N * N
    rp, c, v = W.poisson_csr(N)
    b = W.uniform_rhs(n, 3)
    P = csr_handle(rp, c)
    with pytest.raises(K.SlaError) as e:
        K.sla_resident_loop_ms(P)
    assert e.value.status == K.ERR_ARG
    K.sla_cg_solve(P, t(v), t(b), 1e-8, 5000, jacobi=True)
    torch.cuda.synchronize()
    assert not _resident(P)
    K.sla_cg_solve_batched(P, t(np.stack([v, v])), t(np.stack([b, b])), 1e-8, 5000)
    torch.cuda.synchronize()
    assert not _resident(P)
    K.sla_cg_solve(P, t(v), t(b), 1e-8, 5000)
    torch.cuda.synchronize()
    ms = K.sla_resident_loop_ms(P)
    say(f"resident loop 520^2 to 1e-8: {ms:.3f} ms")
    assert ms > 0.0


def ctypes_byref(x):
    import ctypes
    return ctypes.byref(x)
