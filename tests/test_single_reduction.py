"""The single-reduction rearrangement of CG (Chronopoulos and Gear) that the
resident grid loop and the one-workgroup loop run (the latter also with
Jacobi preconditioning), written out in numpy from its recurrences, against
the oracle's two-sum CG ([torch-sla · Methodology 1], the CG iteration): the
same alpha, beta and r.r history and the same x, to rounding, on a Poisson
grid and on rough-coefficient diffusion; and, step by step, the identity it
rests on, p_k.A p_k = delta_k - beta_k gamma_k / alpha_{k-1}, against the
product formed directly.  A wrong sign or index in those recurrences (the
kernel's, restated here) fails these."""
import numpy as np
import pytest
import scipy.sparse as sp

import oracle
import workloads as W


def _single_reduction(A, b, iters, stop=-1.0):
    """x, alpha, beta, gamma histories and the largest relative gap between
    p.Ap formed directly and by the identity, over `iters` iterations or
    until r.r <= stop."""
    n = b.shape[0]
    x = np.zeros(n)
    r = b.copy()
    p = np.zeros(n)
    s = np.zeros(n)
    alpha = 0.0
    gamma_prev = 0.0
    al, be, gm = [], [], []
    gap = 0.0
    for k in range(iters + 1):
        u = A @ r
        gamma, delta = r @ r, r @ u
        beta = gamma / gamma_prev if k > 0 else 0.0
        if k > 0:
            be.append(beta)
            gm.append(gamma)
        if k == iters or gamma <= stop:
            break
        pap = delta - beta * (gamma / alpha) if k > 0 else delta
        p = r + beta * p
        s = u + beta * s
        direct = p @ (A @ p)
        gap = max(gap, abs(pap - direct) / abs(direct))
        alpha = gamma / pap
        al.append(alpha)
        x = x + alpha * p
        r = r - alpha * s
        gamma_prev = gamma
    return x, np.array(al), np.array(be), np.array(gm), gap


@pytest.mark.parametrize("case", ["poisson", "rough"])
def test_single_reduction_matches_oracle_cg(case):
    if case == "poisson":
        rp, c, v = W.poisson_csr(24)
        b = W.uniform_rhs(576, 0)
        iters = 60
    else:
        # (past about 35 iterations the two forms' histories part by more than
        # rounding on this system, as any two CG forms do once orthogonality
        # is lost; their converged solutions agree: the test below)
        rp, c, v = W.rough_diffusion_csr(20, 3, 2.0)
        b = W.normal_rhs(400, 5)
        iters = 30
    n = len(rp) - 1
    A = sp.csr_matrix((v, c, rp), shape=(n, n))
    Ao = oracle.CSR(n, np.asarray(rp, np.int64), np.asarray(c, np.int32), v)
    xo, io, (ao, bo, ro) = oracle.cg(Ao, b, 0.0, iters, history=True)
    assert io.iterations == iters
    x, al, be, gm, gap = _single_reduction(A, b, iters)
    assert gap <= 1e-10
    # the oracle's history entry k: alpha_k, beta_{k+1}, r_{k+1}.r_{k+1}
    assert np.allclose(al, ao[:iters], rtol=1e-9, atol=0)
    assert np.allclose(be, bo[:iters], rtol=1e-9, atol=0)
    assert np.allclose(gm, ro[:iters], rtol=1e-8, atol=0)
    assert np.linalg.norm(x - xo) <= 1e-10 * np.linalg.norm(xo)


def test_single_reduction_converged_solution():
    """Run to r.r <= 1e-24 b.b on rough-coefficient diffusion: the iteration
    counts within 2 % and x within 1e-9 of the oracle's."""
    rp, c, v = W.rough_diffusion_csr(20, 3, 2.0)
    n = len(rp) - 1
    A = sp.csr_matrix((v, c, rp), shape=(n, n))
    b = W.normal_rhs(n, 5)
    Ao = oracle.CSR(n, np.asarray(rp, np.int64), np.asarray(c, np.int32), v)
    xo, io = oracle.cg(Ao, b, 1e-12, 5000)
    assert io.converged
    stop = 1e-24 * (b @ b)
    x, al, be, gm, _ = _single_reduction(A, b, 5000, stop)
    k = len(al)  # iterations when r.r first met the rule
    assert gm[-1] <= stop and np.all(gm[:-1] > stop)
    assert abs(k - io.iterations) <= max(1, 0.02 * io.iterations)
    assert np.linalg.norm(x - xo) <= 1e-9 * np.linalg.norm(xo)


def test_single_reduction_jacobi_matches_oracle_pcg():
    """The preconditioned form (z = r / d, w = A z; one sum of r.r, z.w and
    r.z; p.Ap = z.w - beta r.z / alpha) against the oracle's Jacobi PCG:
    alpha, beta, r.r and r.z histories and x."""
    rp, c, v = W.rough_diffusion_csr(16, 7, 2.0)
    n = len(rp) - 1
    A = sp.csr_matrix((v, c, rp), shape=(n, n))
    d = A.diagonal()
    b = W.normal_rhs(n, 8)
    iters = 25
    Ao = oracle.CSR(n, np.asarray(rp, np.int64), np.asarray(c, np.int32), v)
    xo, io, (ao, bo, ro, zo) = oracle.pcg_jacobi(Ao, b, 0.0, iters, history=True)
    assert io.iterations == iters
    x = np.zeros(n)
    r = b.copy()
    p = np.zeros(n)
    s = np.zeros(n)
    alpha = rz_prev = 0.0
    al, be, rrs, rzs = [], [], [], []
    for k in range(iters + 1):
        z = r / d
        w = A @ z
        rr, zw, rz = r @ r, z @ w, r @ z
        beta = rz / rz_prev if k > 0 else 0.0
        if k > 0:
            be.append(beta)
            rrs.append(rr)
            rzs.append(rz)
        if k == iters:
            break
        pap = zw - beta * (rz / alpha) if k > 0 else zw
        p = z + beta * p
        s = w + beta * s
        assert abs(pap - p @ (A @ p)) <= 1e-10 * abs(pap)
        alpha = rz / pap
        al.append(alpha)
        x = x + alpha * p
        r = r - alpha * s
        rz_prev = rz
    assert np.allclose(al, ao, rtol=1e-9, atol=0)
    assert np.allclose(be, bo, rtol=1e-9, atol=0)
    assert np.allclose(rrs, ro, rtol=1e-8, atol=0)
    assert np.allclose(rzs, zo, rtol=1e-8, atol=0)
    assert np.linalg.norm(x - xo) <= 1e-10 * np.linalg.norm(xo)


def test_planted_sign_error_is_caught():
    """The same recurrences with the identity's sign flipped drift from the
    oracle at once: the checks above are not vacuous."""
    rp, c, v = W.poisson_csr(12)
    n = len(rp) - 1
    A = sp.csr_matrix((v, c, rp), shape=(n, n))
    b = W.uniform_rhs(n, 0)
    Ao = oracle.CSR(n, np.asarray(rp, np.int64), np.asarray(c, np.int32), v)
    xo, _ = oracle.cg(Ao, b, 0.0, 10)
    x = np.zeros(n)
    r = b.copy()
    p = np.zeros(n)
    s = np.zeros(n)
    alpha = gamma_prev = 0.0
    for k in range(10):
        u = A @ r
        gamma, delta = r @ r, r @ u
        beta = gamma / gamma_prev if k > 0 else 0.0
        pap = delta + beta * (gamma / alpha) if k > 0 else delta
        p = r + beta * p
        s = u + beta * s
        alpha = gamma / pap
        x = x + alpha * p
        r = r - alpha * s
        gamma_prev = gamma
    assert np.linalg.norm(x - xo) > 1e-3 * np.linalg.norm(xo)
