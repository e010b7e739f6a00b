"""The one-workgroup CG loop for small systems (at most 2048 unknowns; a
banded pattern, or plain CSR rows whose 64-row tiles hold at most 336 slots):
ragged sizes, Jacobi, history, warm starts, statuses, batches and rough
coefficients against the oracle, in the default (automatic) mode and with
the two-kernel loop forced;
banded rows against the staged CSR rows bit for bit; systems outside its range
take the resident grid loop (banded) or the two-kernel loop bit for bit."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_GRAD, TOL_X, csr_handle, iters_close, rel, say, t

pytestmark = pytest.mark.gpu


def _A(rp, c, v):
    return oracle.CSR(len(rp) - 1, np.asarray(rp, np.int64), np.asarray(c, np.int32),
                      np.asarray(v, np.float64))


def _banded(n, offsets, seed):
    """Symmetric band with random off-diagonal values, diagonally dominant."""
    rp, c, v = W.band_csr(n, offsets, 1.0)
    rng = np.random.default_rng(seed)
    rows = np.repeat(np.arange(n), np.diff(rp))
    M = {}
    for i, j in zip(rows, c):
        if i < j:
            M[(i, j)] = rng.uniform(-1.0, 1.0)
    vals = np.empty(c.shape[0])
    diag = np.full(n, 0.5)
    for k, (i, j) in enumerate(zip(rows, c)):
        if i != j:
            a = M[(min(i, j), max(i, j))]
            vals[k] = a
            diag[i] += abs(a)
    for k, (i, j) in enumerate(zip(rows, c)):
        if i == j:
            vals[k] = diag[i]
    return rp, c, vals


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 1023, 1024, 1025, 2047, 2048])
def test_ragged_sizes_against_oracle(n):
    """Band matrices (at most 5 slots per row) of ragged sizes: CG and the
    adjoint to tol 1e-11 in both loops against the oracle."""
    import torch
    import krylov_solvers_adjoint_amd as K
    offs = tuple(o for o in (-37, -1, 1, 37) if abs(o) < max(n, 2))
    rp, c, v = _banded(n, offs, n)
    A = _A(rp, c, v)
    b = W.normal_rhs(n, 3)
    g = W.normal_rhs(n, 4)
    xo, io = oracle.cg(A, b, 1e-11, 5000)
    gbo, gvo, aio = oracle.adjoint(A, xo, g, 1e-11, 5000)
    for mode in ("auto", "off"):
        P = csr_handle(rp, c, one_group=mode)
        vt = t(v)
        x, info = K.sla_cg_solve(P, vt, t(b), 1e-11, 5000)
        gb, gv, ai = K.sla_cg_adjoint(P, vt, x, t(g), 1e-11, 5000)
        torch.cuda.synchronize()
        x, gb, gv = x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy()
        say(f"n={n} {mode}: it {info.iterations}/{io.iterations} adj {ai.iterations}/"
            f"{aio.iterations} x {rel(x, xo):.1e}")
        assert info.converged and ai.converged
        assert iters_close(info.iterations, io.iterations)
        assert iters_close(ai.iterations, aio.iterations)
        assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD


def test_mode_argument():
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.poisson_csr(8)
    P = csr_handle(rp, c)
    assert K._lib.sla_csr_set_one_group(P.handle, 7) == K.ERR_ARG
    assert K._lib.sla_csr_set_one_group(P.handle, K.ONE_GROUP_OFF) == K.OK
    assert K._lib.sla_csr_set_one_group(P.handle, K.ONE_GROUP_AUTO) == K.OK


def test_outside_the_range():
    """2049 unknowns on a band: the resident grid loop (one launch over the
    whole GPU), against the oracle; plain CSR tiles of more than 336 slots (9
    per row, more offsets than a band holds): the automatic mode gives the
    two-kernel loop's bits."""
    import torch
    import krylov_solvers_adjoint_amd as K
    n = 2049
    rp, c, v = _banded(n, (-37, -1, 1, 37), 7)
    b = W.normal_rhs(n, 8)
    P = csr_handle(rp, c)
    x, info = K.sla_cg_solve(P, t(v), t(b), 1e-11, 5000)
    torch.cuda.synchronize()
    assert K.sla_resident_loop_ms(P) > 0.0
    xo, io = oracle.cg(_A(rp, c, v), b, 1e-11, 5000)
    assert iters_close(info.iterations, io.iterations) and rel(x.cpu().numpy(), xo) <= TOL_X
    n = 1000
    rp, c, v = _banded(n, (-4, -3, -2, -1, 1, 2, 3, 4), 7)
    b = W.normal_rhs(n, 8)
    xs = []
    for mode in ("auto", "off"):
        P = csr_handle(rp, c, one_group=mode)
        assert not P.banded
        x, info = K.sla_cg_solve(P, t(v), t(b), 1e-11, 5000)
        torch.cuda.synchronize()
        xs.append((x.cpu().numpy(), info.iterations))
    assert np.array_equal(xs[0][0], xs[1][0]) and xs[0][1] == xs[1][1]


@pytest.mark.parametrize("n,offs", [(1024, (-32, -1, 1, 32)), (777, (-29, -2, 2, 29)),
                                    (2048, (-45, -1, 1, 45)), (1500, (-40, -1, 1, 40)),
                                    (400, (-20, -1, 1, 20)), (65, (-1, 1)),
                                    (256, (-16, -1, 1, 16))])
def test_banded_rows_match_staged_csr_rows(n, offs):
    """A banded pattern runs the loop with each row's values held by band
    offset; the same pattern forced onto plain CSR rows (products staged in
    LDS) gives the same bits, forward and adjoint, with and without Jacobi:
    both add a row's products in ascending column order.  Between 257 and
    512 unknowns the two take different workgroup shapes (256 threads with
    two banded rows each, 512 with one staged row), so their dot products
    are summed in different orders: there both are held to the oracle
    only."""
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = _banded(n, offs, n + 1)
    A = _A(rp, c, v)
    b = W.normal_rhs(n, 21)
    g = W.normal_rhs(n, 22)
    P1 = csr_handle(rp, c)
    P2 = csr_handle(rp, c)
    P2.set_spmv_variant("csr")
    assert P1.banded and not P2.banded
    vt = t(v)
    for jac in (False, True):
        out = []
        for P in (P1, P2):
            x, info = K.sla_cg_solve(P, vt, t(b), 1e-11, 5000, jacobi=jac)
            gb, gv, ai = K.sla_cg_adjoint(P, vt, x, t(g), 1e-11, 5000, jacobi=jac)
            torch.cuda.synchronize()
            out.append((x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy(),
                        info.iterations, ai.iterations))
        if not 256 < n <= 512:
            for a1, a2 in zip(out[0], out[1]):
                assert np.array_equal(a1, a2)
        xo, io = (oracle.pcg_jacobi if jac else oracle.cg)(A, b, 1e-11, 5000)
        for o in out:
            say(f"n={n} jacobi={jac}: it {o[3]}/{io.iterations} x {rel(o[0], xo):.1e}")
            assert iters_close(o[3], io.iterations) and rel(o[0], xo) <= TOL_X


def test_wide_band_in_range():
    """Seven offsets (448 slots per 64-row tile, more than the staged CSR
    rows take): the banded loop runs it, against the oracle and against the
    two-kernel loop's iterate."""
    import torch
    import krylov_solvers_adjoint_amd as K
    n = 1000
    rp, c, v = _banded(n, (-3, -2, -1, 1, 2, 3), 31)
    A = _A(rp, c, v)
    b = W.normal_rhs(n, 32)
    g = W.normal_rhs(n, 33)
    xo, io = oracle.cg(A, b, 1e-11, 5000)
    gbo, gvo, aio = oracle.adjoint(A, xo, g, 1e-11, 5000)
    res = []
    for mode in ("auto", "off"):
        P = csr_handle(rp, c, one_group=mode)
        assert P.banded
        x, info = K.sla_cg_solve(P, t(v), t(b), 1e-11, 5000)
        gb, gv, ai = K.sla_cg_adjoint(P, t(v), x, t(g), 1e-11, 5000)
        torch.cuda.synchronize()
        x, gb, gv = x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy()
        assert info.converged and ai.converged
        assert iters_close(info.iterations, io.iterations)
        assert iters_close(ai.iterations, aio.iterations)
        assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD
        res.append(x)
    # the two loops sum their dot products in different orders
    assert not np.array_equal(res[0], res[1])


def test_history_warm_start_and_reproducibility():
    """Poisson 32^2: alpha, beta and r.r of every iteration against the
    oracle's; a warm start; two runs give the same bits."""
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.poisson_csr(32)
    A = _A(rp, c, v)
    b = W.uniform_rhs(1024, 0)
    P = csr_handle(rp, c)
    runs = []
    for _ in range(2):
        x, info = K.sla_cg_solve(P, t(v), t(b), 1e-10, 5000, history=True)
        torch.cuda.synchronize()
        runs.append((x.cpu().numpy(), info.iterations, P.history()))
    assert np.array_equal(runs[0][0], runs[1][0]) and runs[0][1] == runs[1][1]
    for h1, h2 in zip(runs[0][2], runs[1][2]):
        assert np.array_equal(h1, h2)
    xo, io, (ao, bo, ro) = oracle.cg(A, b, 1e-10, 5000, history=True)
    al, be, rr = runs[0][2]
    assert len(al) == runs[0][1] == io.iterations
    k = min(60, len(ao))
    assert rel(al[:k], ao[:k]) <= 1e-9 and rel(be[:k], bo[:k]) <= 1e-9
    assert rel(rr[:k], ro[:k]) <= 1e-9
    x0 = xo + 1e-3 * W.normal_rhs(1024, 9)
    xw, iw = K.sla_cg_solve(P, t(v), t(b), 1e-10, 5000, x0=t(x0))
    torch.cuda.synchronize()
    xwo, iwo = oracle.cg(A, b, 1e-10, 5000, x0=x0)
    assert iters_close(iw.iterations, iwo.iterations)
    assert rel(xw.cpu().numpy(), xwo) <= TOL_X


def test_jacobi_and_statuses():
    """A badly scaled SPD band (Jacobi against the oracle's PCG, forward and
    adjoint); a zero diagonal entry (NOT_SPD before any iteration), -A
    (NOT_SPD at the first iteration, x = 0), NaN in b (NONFINITE), b = 0,
    maxit = 0, tol = 0 (exactly maxit iterations)."""
    import torch
    import krylov_solvers_adjoint_amd as K
    n = 1500
    rp, c, v = _banded(n, (-40, -1, 1, 40), 11)
    rows = np.repeat(np.arange(n), np.diff(rp))
    s = np.exp(np.random.default_rng(12).uniform(-3.0, 3.0, n))
    vs = v * s[rows] * s[c]          # D A D: SPD, badly scaled
    A = _A(rp, c, vs)
    b = W.normal_rhs(n, 13)
    g = W.normal_rhs(n, 14)
    P = csr_handle(rp, c)
    x, info = K.sla_cg_solve(P, t(vs), t(b), 1e-10, 20000, jacobi=True)
    gb, gv, ai = K.sla_cg_adjoint(P, t(vs), x, t(g), 1e-10, 20000, jacobi=True)
    torch.cuda.synchronize()
    xo, io = oracle.pcg_jacobi(A, b, 1e-10, 20000)
    gbo, gvo, aio = oracle.adjoint_jacobi(A, xo, g, 1e-10, 20000)
    assert info.converged and iters_close(info.iterations, io.iterations)
    assert iters_close(ai.iterations, aio.iterations)
    assert rel(x.cpu().numpy(), xo) <= TOL_X and rel(gb.cpu().numpy(), gbo) <= TOL_X
    assert rel(gv.cpu().numpy(), gvo) <= TOL_GRAD
    # a zero diagonal entry
    vz = vs.copy()
    vz[np.flatnonzero((rows == 17) & (c == 17))] = 0.0
    _, iz = K.sla_cg_solve(P, t(vz), t(b), 1e-10, 100, jacobi=True, check=False)
    assert iz.status == K.ERR_NOT_SPD and iz.iterations == 0
    # -A, NaN, b = 0, maxit = 0, tol = 0
    xn, inn = K.sla_cg_solve(P, t(-vs), t(b), 1e-10, 100, check=False)
    torch.cuda.synchronize()
    assert inn.status == K.ERR_NOT_SPD and inn.iterations == 0 and float(xn.abs().max()) == 0.0
    bad = b.copy()
    bad[5] = np.nan
    _, ib = K.sla_cg_solve(P, t(vs), t(bad), 1e-10, 100, check=False)
    assert ib.status == K.ERR_NONFINITE
    x0, i0 = K.sla_cg_solve(P, t(vs), t(np.zeros(n)), 1e-10, 100)
    torch.cuda.synchronize()
    assert i0.iterations == 0 and i0.converged and float(x0.abs().max()) == 0.0
    _, im = K.sla_cg_solve(P, t(vs), t(b), 1e-10, 0)
    assert im.iterations == 0 and not im.converged
    xf, itf = K.sla_cg_solve(P, t(vs), t(b), 0.0, 37)
    torch.cuda.synchronize()
    xfo, ifo = oracle.cg(A, b, 0.0, 37)
    assert itf.iterations == 37 == ifo.iterations
    assert rel(xf.cpu().numpy(), xfo) <= 1e-10


def test_batch_of_small_systems():
    """256 shifted Poisson 32^2 systems (one workgroup each) forward and
    adjoint against the oracle; a batch whose second system is negative
    definite reports it while the others converge."""
    import torch
    import krylov_solvers_adjoint_amd as K
    B = 256
    rp, c, vals_b, b_b, _ = W.batched_poisson(32, B, 2, 3)
    n = 1024
    g_b = W.normal_rhs(n, 9, shape=(B, n))
    P = csr_handle(rp, c)
    vt = t(vals_b)
    x, infos = K.sla_cg_solve_batched(P, vt, t(b_b), 1e-10, 5000)
    gb, gv, ainf = K.sla_cg_adjoint_batched(P, vt, x, t(g_b), 1e-10, 5000)
    torch.cuda.synchronize()
    xo, io = oracle.cg_batched(rp, c, vals_b, b_b, 1e-10, 5000)
    gbo, gvo, aio = oracle.adjoint_batched(rp, c, vals_b, xo, g_b, 1e-10, 5000)
    x, gb, gv = x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy()
    for s in range(B):
        assert infos[s].converged and iters_close(infos[s].iterations, io[s].iterations)
        assert iters_close(ainf[s].iterations, aio[s].iterations)
        assert rel(x[s], xo[s]) <= TOL_X and rel(gb[s], gbo[s]) <= TOL_X
        assert rel(gv[s], gvo[s]) <= TOL_GRAD
    v4 = vals_b[:4].copy()
    v4[1] = -v4[1]
    Q = csr_handle(rp, c)
    x4, i4 = K.sla_cg_solve_batched(Q, t(v4), t(b_b[:4]), 1e-10, 5000, check=False)
    torch.cuda.synchronize()
    assert [i.status for i in i4] == [0, K.ERR_NOT_SPD, 0, 0]
    for s in (0, 2, 3):
        assert rel(x4[s].cpu().numpy(), xo[s]) <= TOL_X


def test_adjoint_refused_on_the_device():
    """Values that are not symmetric on the one-workgroup loop: the check runs
    on the device and gates the solve and the pattern gradient there, so every
    system of the batch is refused (SLA_ERR_NOT_SYMMETRIC, no iteration, the
    message) and grad_b and grad_vals keep what they held; with and without
    Jacobi.  The next call, with symmetric values, is solved (against the
    oracle): the flag is cleared by every check."""
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 32
    n = N * N
    rp, c, v = W.poisson_csr(N)
    vn = v.copy()
    off = np.flatnonzero(vn != 4.0)
    vn[int(off[17])] = -1.25  # a_ij changed, a_ji not
    b = W.uniform_rhs(n, 6)
    g = W.normal_rhs(n, 7)
    P = csr_handle(rp, c)
    x1, _ = K.sla_cg_solve(P, t(v), t(b), 1e-10, 5000)
    torch.cuda.synchronize()
    nnz = v.shape[0]
    for jac in (False, True):
        for vals in (vn[None, :], np.stack([v, vn, v])):
            batch = vals.shape[0]
            P.bind(t(vals))
            xb = x1.repeat(batch, 1).contiguous()
            gx = t(np.tile(g, (batch, 1)))
            gb = torch.full((batch, n), 7.0, dtype=torch.float64, device=xb.device)
            gv = torch.full((batch, nnz), 7.0, dtype=torch.float64, device=xb.device)
            infos = (K._Info * batch)()
            st = K._lib.sla_cg_adjoint_batched(P.handle, xb.data_ptr(), gx.data_ptr(),
                                               gb.data_ptr(), gv.data_ptr(), 1e-10, 5000,
                                               K.FLAG_JACOBI if jac else 0, infos, None)
            torch.cuda.synchronize()
            assert st == K.ERR_NOT_SYMMETRIC
            for i in infos:
                assert i.status == K.ERR_NOT_SYMMETRIC and i.iterations == 0 and not i.converged
            assert b"values are not symmetric" in K._lib.sla_last_error()
            assert bool((gb == 7.0).all()) and bool((gv == 7.0).all())
    A = _A(rp, c, v)
    xo, _ = oracle.cg(A, b, 1e-10, 5000)
    gbo, gvo, aio = oracle.adjoint(A, xo, g, 1e-10, 5000)
    gb, gv, ai = K.sla_cg_adjoint(P, t(v), x1, t(g), 1e-10, 5000)
    torch.cuda.synchronize()
    assert ai.converged and iters_close(ai.iterations, aio.iterations)
    assert rel(gb.cpu().numpy(), gbo) <= TOL_X and rel(gv.cpu().numpy(), gvo) <= TOL_GRAD


@pytest.mark.parametrize("jac", [False, True])
def test_rough_coefficients_single_reduction(jac):
    """Rough-coefficient diffusion on 45^2 = 2025 unknowns (four rows per
    thread), plain and Jacobi-preconditioned, forward and adjoint to 1e-10
    (hundreds of iterations at a conductance contrast of e^6): the loop's
    single-reduction recurrences within the parity bounds of the oracle's
    two-sum CG and PCG."""
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.rough_diffusion_csr(45, 4, 3.0)
    n = len(rp) - 1
    b = W.normal_rhs(n, 15)
    g = W.normal_rhs(n, 16)
    P = csr_handle(rp, c)
    vt = t(v)
    x, info = K.sla_cg_solve(P, vt, t(b), 1e-10, 20000, jacobi=jac)
    gb, gv, ai = K.sla_cg_adjoint(P, vt, x, t(g), 1e-10, 20000, jacobi=jac)
    torch.cuda.synchronize()
    A = _A(rp, c, v)
    if jac:
        xo, io = oracle.pcg_jacobi(A, b, 1e-10, 20000)
        gbo, gvo, aio = oracle.adjoint_jacobi(A, xo, g, 1e-10, 20000)
    else:
        xo, io = oracle.cg(A, b, 1e-10, 20000)
        gbo, gvo, aio = oracle.adjoint(A, xo, g, 1e-10, 20000)
    x, gb, gv = x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy()
    say(f"rough 45^2 jacobi={jac}: it {info.iterations}/{io.iterations} adj "
        f"{ai.iterations}/{aio.iterations}; x {rel(x, xo):.1e} lam {rel(gb, gbo):.1e} "
        f"gv {rel(gv, gvo):.1e}")
    assert info.converged and ai.converged
    assert iters_close(info.iterations, io.iterations)
    assert iters_close(ai.iterations, aio.iterations)
    assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD
