"""Pins of the CPU oracle against what the mathematics fixes.

Each ``pin_*`` function raises ``AssertionError`` when the oracle (or a
deliberately broken build of it, passed as ``lib``) disagrees with a closed
form, a textbook identity, brute force or a hand-derived value.  None of
them re-types the oracle's own formulas: they check properties the correct
result must have.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle
import workloads as W
from closed_forms import eigval, eigvec, spectrum_bounds

EPS = np.finfo(np.float64).eps
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _poisson(N):
    rp, c, v = W.poisson_csr(N, np.int64)
    return oracle.CSR(N * N, rp, c, v)


def _random_spd_csr(n, density, seed):
    """A random sparse SPD matrix (diagonally dominant), CSR built by numpy."""
    rng = np.random.default_rng(seed)
    M = np.where(rng.random((n, n)) < density, rng.uniform(-1, 1, (n, n)), 0.0)
    M = np.triu(M, 1)
    M = M + M.T
    M += np.diag(np.abs(M).sum(axis=1) + rng.uniform(0.5, 1.5, n))
    rows, cols = np.nonzero(M)
    rowptr = np.zeros(n + 1, np.int64)
    np.add.at(rowptr, rows + 1, 1)
    rowptr = np.cumsum(rowptr)
    return oracle.CSR(n, rowptr, cols.astype(np.int32), M[rows, cols].copy()), M


# --------------------------------------------------------------------------
# CSR construction
# --------------------------------------------------------------------------

def pin_csr_poisson_closed_form(lib=None):
    """P0: the merged CSR of a shuffled Poisson COO is the closed-form CSR."""
    for N in (1, 2, 7, 16):
        row, col, val = W.poisson_coo(N)
        r2, c2, v2 = W.shuffled_coo(row, col, val, seed=N)
        rp, cc, perm = oracle.csr_from_coo(N * N, r2, c2, lib=lib)
        vals = oracle.values_from_coo(perm, int(rp[-1]), v2, lib=lib)
        rp_ref, c_ref, v_ref = W.poisson_csr(N, np.int64)
        assert np.array_equal(rp, rp_ref), "rowptr"
        assert np.array_equal(cc, c_ref), "col"
        assert np.array_equal(vals.view(np.int64), v_ref.view(np.int64)), "vals"
        # every COO entry points at a slot with its own row and column
        rows_of_slot = np.repeat(np.arange(N * N), np.diff(rp))
        assert np.array_equal(rows_of_slot[perm], r2) and np.array_equal(cc[perm], c2)


def brute_force_csr(n, row, col, val):
    """Python sorted() over (row, col, input position) and a left fold."""
    order = sorted(range(len(row)), key=lambda k: (row[k], col[k], k))
    rowptr = [0] * (n + 1)
    cols, vals, perm = [], [], [0] * len(row)
    prev = None
    for k in order:
        key = (row[k], col[k])
        if key != prev:
            cols.append(col[k])
            vals.append(val[k])
            rowptr[row[k] + 1] += 1
            prev = key
        else:
            vals[-1] = vals[-1] + val[k]
        perm[k] = len(cols) - 1
    for i in range(n):
        rowptr[i + 1] += rowptr[i]
    return (np.array(rowptr, np.int64), np.array(cols, np.int32),
            np.array(vals, np.float64), np.array(perm, np.int64))


def tiny_coo_cases():
    rng = np.random.default_rng(123)
    cases = [
        (1, [0], [0], [-0.0]),             # a lone negative zero keeps its sign
        (3, [], [], []),                   # no entries at all: three empty rows
        (4, [3, 3, 3], [1, 1, 1], [0.1, 0.2, 0.3]),  # triple duplicate
        (5, [4, 0, 4, 0], [0, 4, 0, 4], [1.0, 2.0, -1.0, -2.0]),  # cancels to 0
    ]
    for t in range(24):
        n = int(rng.integers(1, 65))
        m = int(rng.integers(0, 4 * n))
        row = rng.integers(0, n, m)
        col = rng.integers(0, n, m)
        # force duplicates
        if m > 4:
            k = rng.integers(0, m, m // 4)
            row = np.concatenate([row, row[k]])
            col = np.concatenate([col, col[k]])
        val = rng.standard_normal(row.shape[0])
        val[rng.random(val.shape[0]) < 0.1] = 0.0  # explicit zeros stay stored
        cases.append((n, row.tolist(), col.tolist(), val.tolist()))
    return cases


def pin_csr_brute_force(lib=None):
    """P0b: bit-exact agreement with brute force on tiny COO with duplicates."""
    for n, row, col, val in tiny_coo_cases():
        rp_b, c_b, v_b, p_b = brute_force_csr(n, row, col, val)
        rp, cc, perm = oracle.csr_from_coo(n, np.array(row, np.int64),
                                           np.array(col, np.int64), lib=lib)
        vals = oracle.values_from_coo(perm, int(rp[-1]), np.array(val, np.float64), lib=lib)
        assert np.array_equal(rp, rp_b), (n, "rowptr")
        assert np.array_equal(cc, c_b), (n, "col")
        assert np.array_equal(perm, p_b), (n, "perm")
        assert np.array_equal(vals.view(np.int64), v_b.view(np.int64)), (n, "vals")


def pin_csr_rgg_symmetric(lib=None):
    """P0c: the random-geometric-graph Laplacian is bitwise symmetric and its
    rows sum to the shift (up to rounding)."""
    n = 3000
    row, col, val, _ = W.rgg_coo(n, 4, 5)
    rp, cc, perm = oracle.csr_from_coo(n, row, col, lib=lib)
    vals = oracle.values_from_coo(perm, int(rp[-1]), val, lib=lib)
    A = oracle.CSR(n, rp, cc, vals)
    T = oracle.transpose(A, lib=lib)
    assert np.array_equal(T.rowptr, A.rowptr) and np.array_equal(T.col, A.col)
    assert np.array_equal(T.vals.view(np.int64), A.vals.view(np.int64))
    rowsum = np.add.reduceat(vals, rp[:-1]) if n else vals
    diag = np.abs(vals).max()
    assert np.all(np.abs(rowsum - 1e-2) <= 64 * EPS * diag)
    assert 7.0 < A.nnz / n < 10.0


# --------------------------------------------------------------------------
# SpMV and dot
# --------------------------------------------------------------------------

def pin_spmv_eigenpairs(lib=None):
    """P1: A v = lambda v for the closed-form Laplacian eigenpairs."""
    for N, modes in ((16, [(1, 1), (3, 7), (16, 16)]), (100, [(1, 1), (50, 2), (99, 100)])):
        A = _poisson(N)
        for p, q in modes:
            v = eigvec(N, p, q)
            lam = eigval(N, p, q)
            Av = oracle.spmv(A, v, lib=lib)
            rel = np.linalg.norm(Av - lam * v) / np.linalg.norm(lam * v)
            assert rel <= 64 * EPS * 8.0 / lam, (N, p, q, rel)
            rq = oracle.dot(v, Av, lib=lib) / oracle.dot(v, v, lib=lib)
            assert abs(rq - lam) <= 64 * EPS * 8.0, (N, p, q, rq, lam)


def pin_spmv_dense(lib=None):
    """P1b: matches dense A @ x within the summation error bound."""
    for seed, n in ((0, 1), (1, 17), (2, 64), (3, 200)):
        A, M = _random_spd_csr(n, 0.1, seed)
        x = np.random.default_rng(seed + 100).standard_normal(n)
        y = oracle.spmv(A, x, lib=lib)
        bound = 8 * EPS * (np.abs(M) @ np.abs(x)) + 1e-300
        assert np.all(np.abs(y - M @ x) <= bound), seed


def pin_dot(lib=None):
    """dot agrees with the exactly rounded sum (math.fsum) within n*eps*sum|uv|."""
    rng = np.random.default_rng(9)
    for n in (0, 1, 4095, 4096, 4097, 20000):
        u = rng.standard_normal(n)
        v = rng.standard_normal(n)
        d = oracle.dot(u, v, lib=lib)
        exact = math.fsum((u * v).tolist()) if n else 0.0
        # products are exact-ish: the bound covers their rounding too
        assert abs(d - exact) <= (n + 2) * EPS * float(np.abs(u * v).sum()) + 1e-300, n


# --------------------------------------------------------------------------
# CG
# --------------------------------------------------------------------------

def pin_cg_one_step(lib=None):
    """P2: an eigenvector right-hand side is solved in one iteration."""
    for N, (p, q) in ((8, (2, 3)), (32, (5, 5)), (64, (64, 1))):
        A = _poisson(N)
        v = eigvec(N, p, q)
        lam = eigval(N, p, q)
        x, info = oracle.cg(A, v, 1e-10, 100, lib=lib)
        assert info.status == oracle.OK and info.iterations == 1, (N, info)
        assert np.linalg.norm(x - v / lam) <= 1e-12 * np.linalg.norm(v / lam)


def pin_cg_m_step(lib=None):
    """P3: m eigenvectors with distinct eigenvalues above 4 need exactly m
    iterations (Krylov space of dimension m)."""
    N = 32
    A = _poisson(N)
    for m in range(1, 7):
        modes = [(N, N - k) for k in range(m)]
        lams = [eigval(N, p, q) for p, q in modes]
        assert min(lams) > 4.0 and len(set(np.round(lams, 12))) == m
        b = sum(eigvec(N, p, q) * (1.0 + 0.5 * k) for k, (p, q) in enumerate(modes))
        x, info = oracle.cg(A, b, 1e-12, 100, lib=lib)
        assert info.status == oracle.OK and info.converged and info.iterations == m, (m, info)
        xe = sum(eigvec(N, p, q) * (1.0 + 0.5 * k) / eigval(N, p, q)
                 for k, (p, q) in enumerate(modes))
        assert np.linalg.norm(x - xe) <= 1e-11 * np.linalg.norm(xe)


def pin_cg_dense_lu(lib=None):
    """P4: tiny grids and random SPD matrices agree with a dense LU solve."""
    for N in (1, 2, 5, 16):
        A = _poisson(N)
        b = W.uniform_rhs(N * N, N)
        x, info = oracle.cg(A, b, 1e-13, 1000, lib=lib)
        xl = np.linalg.solve(A.to_dense(), b)
        assert info.converged and np.linalg.norm(x - xl) <= 1e-10 * np.linalg.norm(xl), N
    for seed in range(3):
        A, M = _random_spd_csr(60, 0.15, seed)
        b = np.random.default_rng(seed).standard_normal(60)
        x, info = oracle.cg(A, b, 1e-13, 1000, lib=lib)
        xl = np.linalg.solve(M, b)
        assert info.converged and np.linalg.norm(x - xl) <= 1e-10 * np.linalg.norm(xl), seed


def pin_cg_manufactured(lib=None):
    """P5: b = A u* for u* = sin(pi x) sin(pi y) gives back u*.  n = 10^4 > 4096
    so the blocked dot product uses several blocks."""
    N = 100
    A = _poisson(N)
    u, b = W.manufactured(N)
    x, info = oracle.cg(A, b, 0.0, 600, lib=lib)
    assert info.status == oracle.OK and info.iterations == 600 and not info.converged
    assert np.linalg.norm(x - u) <= 1e-12 * np.linalg.norm(u), np.linalg.norm(x - u)
    # the recursive residual tracks the true one
    r_true = b - A.to_dense() @ x if N <= 40 else b - oracle.spmv(A, x, lib=lib)
    assert np.linalg.norm(r_true) <= 1e-11 * np.linalg.norm(b)


def pin_cg_ritz(lib=None):
    """P10: Ritz values of the Lanczos matrix built from (alpha, beta) lie in
    the closed-form spectrum and reach both ends."""
    N = 32
    A = _poisson(N)
    b = W.uniform_rhs(N * N, 0)
    x, info, (al, be, rr) = oracle.cg(A, b, 1e-10, 10000, history=True, lib=lib)
    k = info.iterations
    lo, hi = spectrum_bounds(N)
    for kk in (10, 50, k):
        d = np.array([1.0 / al[j] + (be[j - 1] / al[j - 1] if j else 0.0) for j in range(kk)])
        e = np.array([np.sqrt(be[j]) / al[j] for j in range(kk - 1)])
        T = np.diag(d) + np.diag(e, 1) + np.diag(e, -1)
        ritz = np.linalg.eigvalsh(T)
        assert ritz.min() >= lo * (1 - 1e-9) and ritz.max() <= hi * (1 + 1e-12), kk
    assert abs(ritz.max() - hi) <= 1e-8 * hi and abs(ritz.min() - lo) <= 1e-6 * lo


def pin_cg_energy(lib=None):
    """P13: with x0 = 0, b.x_k = sum_j alpha_j r_j.r_j (exact arithmetic), and
    the recursive residual matches b - A x_k."""
    for N, tol, maxit in ((32, 1e-10, 10000), (60, 0.0, 150)):
        A = _poisson(N)
        b = W.uniform_rhs(N * N, 0)
        x, info, (al, be, rr) = oracle.cg(A, b, tol, maxit, history=True, lib=lib)
        rrs = np.concatenate([[info.bb], rr[:-1]])
        lhs = float(b @ x)
        rhs = math.fsum((al * rrs).tolist())
        assert abs(lhs - rhs) <= 1e-13 * abs(rhs), (N, lhs, rhs)
        r_true = b - A.to_dense() @ x
        assert abs(np.linalg.norm(r_true) ** 2 - info.rr) <= 1e-6 * info.rr + 1e-28 * info.bb


def pin_cg_statuses(lib=None):
    """Degenerate inputs: b = 0, NaN, an indefinite matrix, maxit, tol = 0, n = 1."""
    A = _poisson(8)
    n = 64
    x, info = oracle.cg(A, np.zeros(n), 1e-10, 100, lib=lib)
    assert info.status == oracle.OK and info.iterations == 0 and info.converged
    assert np.all(x == 0)
    bad = W.uniform_rhs(n, 1)
    bad[5] = np.nan
    _, info = oracle.cg(A, bad, 1e-10, 100, lib=lib)
    assert info.status == oracle.ERR_NONFINITE
    neg = oracle.CSR(A.n, A.rowptr, A.col, -A.vals)
    _, info = oracle.cg(neg, W.uniform_rhs(n, 2), 1e-10, 100, lib=lib)
    assert info.status == oracle.ERR_NOT_SPD and info.iterations == 0
    _, info = oracle.cg(A, W.uniform_rhs(n, 3), 1e-10, 1, lib=lib)
    assert info.status == oracle.OK and info.iterations == 1 and not info.converged
    _, info = oracle.cg(A, W.uniform_rhs(n, 3), 0.0, 7, lib=lib)
    assert info.iterations == 7 and not info.converged
    A1 = oracle.CSR(1, np.array([0, 1], np.int64), np.array([0], np.int32), np.array([2.5]))
    x, info = oracle.cg(A1, np.array([3.0]), 1e-12, 10, lib=lib)
    assert info.iterations == 1 and abs(x[0] - 1.2) <= 2 * EPS * 1.2
    # a warm start at the solution needs no iteration
    b = W.uniform_rhs(n, 4)
    xl = np.linalg.solve(A.to_dense(), b)
    x, info = oracle.cg(A, b, 1e-8, 100, x0=xl, lib=lib)
    assert info.iterations == 0 and np.array_equal(x, xl)


def pin_cg_warm_start(lib=None):
    """A start vector away from the solution still converges to the dense LU
    solution, and from x0 the run equals plain CG on A e = b - A x0."""
    N = 12
    A = _poisson(N)
    n = N * N
    b = W.uniform_rhs(n, 5)
    x0 = W.normal_rhs(n, 6)
    x, info = oracle.cg(A, b, 1e-13, 1000, x0=x0, lib=lib)
    xl = np.linalg.solve(A.to_dense(), b)
    assert info.converged and np.linalg.norm(x - xl) <= 1e-10 * np.linalg.norm(xl)
    e, info_e = oracle.cg(A, b - A.to_dense() @ x0, 1e-13 * np.linalg.norm(b) /
                          np.linalg.norm(b - A.to_dense() @ x0), 1000, lib=lib)
    assert abs(info_e.iterations - info.iterations) <= 1
    assert np.linalg.norm(x0 + e - xl) <= 1e-10 * np.linalg.norm(xl)


# --------------------------------------------------------------------------
# Adjoint
# --------------------------------------------------------------------------

def pin_adjoint_identities(lib=None):
    """P6: g.x = lambda.b;  P6b: sum_k vals_k grad_k = -lambda.(A x) = -lambda.b."""
    N = 32
    A = _poisson(N)
    b = W.uniform_rhs(N * N, 0)
    g = W.normal_rhs(N * N, 1)
    x, _ = oracle.cg(A, b, 1e-12, 10000, lib=lib)
    gb, gv, info = oracle.adjoint(A, x, g, 1e-12, 10000, lib=lib)
    assert info.status == oracle.OK and info.converged
    assert abs(g @ x - gb @ b) <= 1e-10 * abs(g @ x)
    assert abs(A.vals @ gv + gb @ b) <= 1e-10 * abs(gb @ b)


def _dense_loss(M, b, g):
    return float(g @ np.linalg.solve(M, b))


def pin_adjoint_fd(lib=None):
    """P7: central finite differences of L = g.x over every stored slot (the
    perturbed matrix is not symmetric, so it is solved by dense LU) and over b."""
    for N in (3, 4):
        A = _poisson(N)
        n = N * N
        rng = np.random.default_rng(N)
        vals = A.vals + rng.uniform(-0.2, 0.2, A.nnz) * (A.vals == 4.0)  # vary the diagonal
        A = oracle.CSR(n, A.rowptr, A.col, vals)
        b = rng.uniform(-1, 1, n)
        g = rng.standard_normal(n)
        x, _ = oracle.cg(A, b, 1e-14, 1000, lib=lib)
        gb, gv, _ = oracle.adjoint(A, x, g, 1e-14, 1000, lib=lib)
        M = A.to_dense()
        rows = np.repeat(np.arange(n), np.diff(A.rowptr))
        fd = np.zeros(A.nnz)
        for k in range(A.nnz):
            d = 1e-5 * max(1.0, abs(vals[k]))
            Mp = M.copy()
            Mp[rows[k], A.col[k]] += d
            Mm = M.copy()
            Mm[rows[k], A.col[k]] -= d
            fd[k] = (_dense_loss(Mp, b, g) - _dense_loss(Mm, b, g)) / (2 * d)
        assert np.max(np.abs(fd - gv)) <= 1e-6 * np.max(np.abs(gv)), N
        fdb = np.zeros(n)
        for i in range(n):
            e = np.zeros(n)
            e[i] = 1e-5
            fdb[i] = (_dense_loss(M, b + e, g) - _dense_loss(M, b - e, g)) / 2e-5
        assert np.max(np.abs(fdb - gb)) <= 1e-6 * np.max(np.abs(gb)), N


def pin_adjoint_support(lib=None):
    """P8: one gradient per stored slot, in slot order; a stored explicit zero
    still gets -lambda_i x_j; nothing is written for absent entries."""
    n = 6
    # tridiagonal SPD with explicit zeros stored at (0, 5) and (5, 0)
    entries = {}
    for i in range(n):
        entries[(i, i)] = 3.0
        if i + 1 < n:
            entries[(i, i + 1)] = -1.0
            entries[(i + 1, i)] = -1.0
    entries[(0, 5)] = 0.0
    entries[(5, 0)] = 0.0
    keys = sorted(entries)
    rows = [k[0] for k in keys]
    cols = [k[1] for k in keys]
    vals = [entries[k] for k in keys]
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, np.array(rows) + 1, 1)
    A = oracle.CSR(n, np.cumsum(rp), np.array(cols, np.int32), np.array(vals))
    b = np.arange(1.0, n + 1)
    g = np.ones(n)
    x, _ = oracle.cg(A, b, 1e-14, 100, lib=lib)
    gb, gv, _ = oracle.adjoint(A, x, g, 1e-14, 100, lib=lib)
    assert gv.shape == (A.nnz,)
    k05 = [k for k in range(A.nnz) if rows[k] == 0 and cols[k] == 5][0]
    assert vals[k05] == 0.0 and gv[k05] != 0.0
    M = A.to_dense()
    xl = np.linalg.solve(M, b)
    ll = np.linalg.solve(M.T, g)
    full = -np.outer(ll, xl)
    assert np.allclose(gv, full[rows, cols], rtol=1e-10, atol=0)


def pin_adjoint_golden(lib=None):
    """P11: hand-derived exact values (tests/golden/adjoint_small.json) and the
    1 x 1 closed form x = b/a, lambda = g/a, grad = -g b / a^2."""
    with open(os.path.join(GOLDEN, "adjoint_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        fr = lambda xs: np.array([float(Fraction(s)) for s in xs])
        A = oracle.CSR(c["n"], np.array(c["rowptr"], np.int64),
                       np.array(c["col"], np.int32), fr(c["vals"]))
        b, g = fr(c["b"]), fr(c["g"])
        x, info = oracle.cg(A, b, 1e-15, 100, lib=lib)
        assert np.allclose(x, fr(c["x"]), rtol=0, atol=1e-14), c["name"]
        gb, gv, _ = oracle.adjoint(A, x, g, 1e-15, 100, lib=lib)
        assert np.allclose(gb, fr(c["lambda"]), rtol=0, atol=1e-14), c["name"]
        assert np.allclose(gv, fr(c["grad_vals"]), rtol=0, atol=1e-14), c["name"]
        assert abs(g @ x - float(Fraction(c["loss"]))) <= 1e-14
    for a, bb, gg in ((2.5, 3.0, -1.5), (7.0, 0.5, 2.0)):
        A1 = oracle.CSR(1, np.array([0, 1], np.int64), np.array([0], np.int32), np.array([a]))
        x, _ = oracle.cg(A1, np.array([bb]), 1e-15, 10, lib=lib)
        gb, gv, _ = oracle.adjoint(A1, x, np.array([gg]), 1e-15, 10, lib=lib)
        assert abs(gb[0] - gg / a) <= 4 * EPS * abs(gg / a)
        assert abs(gv[0] + gg * bb / a**2) <= 8 * EPS * abs(gg * bb / a**2)


def pin_adjoint_nonsymmetric_flag(lib=None):
    """The adjoint solves with the explicit transpose and reports a matrix that
    is not symmetric."""
    A = oracle.CSR(2, np.array([0, 2, 4], np.int64), np.array([0, 1, 0, 1], np.int32),
                   np.array([4.0, 1.0, 0.5, 3.0]))
    x = np.array([1.0, 2.0])
    g = np.array([1.0, -1.0])
    gb, gv, info = oracle.adjoint(A, x, g, 1e-15, 10, lib=lib)
    assert info.status == oracle.ERR_NOT_SYMMETRIC
    # the gradient is still -lambda_i x_j on the four stored slots
    assert np.array_equal(gv, -(np.repeat(gb, 2) * x[[0, 1, 0, 1]]))
    # D A D of a symmetric A: mirror entries (a s_i) s_j and (a s_j) s_i round
    # apart by a few ulps and still count as symmetric; a relative change of
    # 1e-9 in one entry does not
    N = 12
    rp, c, v = W.poisson_csr(N, np.int64)
    rows = np.repeat(np.arange(N * N), np.diff(rp))
    s = np.exp(np.random.default_rng(40).uniform(-3.0, 3.0, N * N))
    vs = (1.1 * v) * s[rows] * s[c]
    mirror = {(int(i), int(j)): k for k, (i, j) in enumerate(zip(rows, c))}
    assert any(vs[k] != vs[mirror[(int(j), int(i))]] for k, (i, j) in enumerate(zip(rows, c)))
    A = oracle.CSR(N * N, rp, c, vs)
    b = W.normal_rhs(N * N, 41)
    xd, _ = oracle.cg(A, b, 1e-12, 1000, lib=lib)
    _, _, info = oracle.adjoint(A, xd, b, 1e-12, 1000, lib=lib)
    assert info.status == oracle.OK
    _, _, info = oracle.adjoint_jacobi(A, xd, b, 1e-12, 1000, lib=lib)
    assert info.status == oracle.OK
    off = int(np.flatnonzero(rows != c)[7])
    vb = vs.copy()
    vb[off] = vb[off] * (1.0 + 1e-9)
    _, _, info = oracle.adjoint(oracle.CSR(N * N, rp, c, vb), xd, b, 1e-12, 1000, lib=lib)
    assert info.status == oracle.ERR_NOT_SYMMETRIC


# --------------------------------------------------------------------------
# Batched
# --------------------------------------------------------------------------

def pin_batched_shift_spectrum(lib=None):
    """P9: system s of the shifted batch has spectrum lambda_pq + c_s, so an
    eigenvector right-hand side is solved in one iteration with x = v/(lambda+c_s)."""
    N, B = 16, 5
    rowptr, col, vals, _, shifts = W.batched_poisson(N, B, 2, 3)
    v = eigvec(N, 3, 4)
    lam = eigval(N, 3, 4)
    xs, infos = oracle.cg_batched(rowptr.astype(np.int64), col, vals,
                                  np.repeat(v[None], B, 0), 1e-10, 100, lib=lib)
    for s in range(B):
        assert infos[s].iterations == 1
        assert np.linalg.norm(xs[s] - v / (lam + shifts[s])) <= 1e-12 * np.linalg.norm(v)


# --------------------------------------------------------------------------
# Jacobi-preconditioned CG
# --------------------------------------------------------------------------

def _scaled_spd(n, seed, spread=2.0):
    """S M S for a random diagonally dominant SPD M and S = diag(10^U(-spread, spread)):
    SPD, with a diagonal spanning many orders of magnitude."""
    A0, M = _random_spd_csr(n, 0.15, seed)
    rng = np.random.default_rng(seed + 100)
    sd = 10.0 ** rng.uniform(-spread, spread, n)
    rows = np.repeat(np.arange(n), np.diff(A0.rowptr))
    # s_i s_j first: the product commutes exactly, so A stays bitwise symmetric
    vals = A0.vals * (sd[rows] * sd[A0.col])
    return oracle.CSR(n, A0.rowptr, A0.col, vals), M * np.outer(sd, sd)


def pin_pcg_uniform_diagonal(lib=None):
    """With M = 4 I (the Poisson diagonal) the preconditioner only rescales
    z, p and q by powers of two: the iterates, beta and r.r are CG's bit for
    bit, and alpha is exactly 4 times CG's."""
    for N in (16, 40):
        A = _poisson(N)
        b = W.uniform_rhs(N * N, 3)
        x1, i1, (a1, b1, r1) = oracle.cg(A, b, 1e-12, 5000, history=True, lib=lib)
        x2, i2, (a2, b2, r2, z2) = oracle.pcg_jacobi(A, b, 1e-12, 5000, history=True, lib=lib)
        assert i1.iterations == i2.iterations and i2.converged
        assert np.array_equal(x1, x2) and np.array_equal(b1, b2) and np.array_equal(r1, r2)
        assert np.array_equal(4.0 * a1, a2) and np.array_equal(r1 / 4.0, z2)


def pin_pcg_scaled_equivalence(lib=None):
    """Jacobi PCG on A is CG on D^-1/2 A D^-1/2 (b -> D^-1/2 b): PCG's r.z
    after each iteration equals that CG's r.r, and x = D^-1/2 x_hat."""
    n = 60
    A, M = _scaled_spd(n, 7)
    d = np.diag(M).copy()
    h = 1.0 / np.sqrt(d)
    Ah = M * np.outer(h, h)
    rows, cols = np.nonzero(Ah)
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    Ahc = oracle.CSR(n, np.cumsum(rp), cols.astype(np.int32), Ah[rows, cols].copy())
    b = W.normal_rhs(n, 8)
    x, info, (al, be, rr, rz) = oracle.pcg_jacobi(A, b, 1e-13, 500, history=True, lib=lib)
    xh, ih, (alh, beh, rrh) = oracle.cg(Ahc, h * b, 1e-30, len(rz), history=True, lib=lib)
    k = min(12, len(rz))
    assert np.allclose(rz[:k], rrh[:k], rtol=1e-8, atol=0)
    assert np.allclose(be[:k], beh[:k], rtol=1e-8, atol=0)
    assert np.allclose(al[:k], alh[:k], rtol=1e-8, atol=0)
    assert info.converged and np.linalg.norm(x - h * xh) <= 1e-8 * np.linalg.norm(x)


def pin_pcg_diagonal_one_step(lib=None):
    """A diagonal A: z0 is already the solution, so PCG stops after one step."""
    n = 50
    rng = np.random.default_rng(11)
    d = 10.0 ** rng.uniform(-3, 3, n)
    A = oracle.CSR(n, np.arange(n + 1, dtype=np.int64), np.arange(n, dtype=np.int32), d)
    b = rng.uniform(-1, 1, n)
    x, info = oracle.pcg_jacobi(A, b, 1e-12, 100, lib=lib)
    assert info.iterations == 1 and info.converged
    assert np.max(np.abs(x - b / d) / np.abs(b / d)) <= 8 * EPS


def pin_pcg_dense_lu(lib=None):
    """Against dense LU on a badly scaled SPD matrix, where Jacobi also needs
    fewer iterations than plain CG."""
    n = 80
    A, M = _scaled_spd(n, 12, spread=2.5)
    b = W.normal_rhs(n, 13)
    xl = np.linalg.solve(M, b)
    x, info = oracle.pcg_jacobi(A, b, 1e-13, 5000, lib=lib)
    x_cg, info_cg = oracle.cg(A, b, 1e-13, 5000, lib=lib)
    assert info.converged
    assert np.linalg.norm(x - xl) <= 1e-8 * np.linalg.norm(xl)
    assert info.iterations < info_cg.iterations


def pin_pcg_statuses(lib=None):
    """A missing, zero or negative diagonal entry is NOT_SPD before any step;
    b = 0 converges in 0 steps."""
    n = 4
    rp = np.array([0, 2, 4, 6, 8], np.int64)
    col = np.array([0, 1, 0, 1, 2, 3, 2, 3], np.int32)
    for bad in (0.0, -1.0):
        vals = np.array([2.0, -1.0, -1.0, 2.0, bad, 0.5, 0.5, 2.0])
        x, info = oracle.pcg_jacobi(oracle.CSR(n, rp, col, vals), np.ones(n), 1e-10, 10, lib=lib)
        assert info.status == oracle.ERR_NOT_SPD and info.iterations == 0
    col2 = np.array([0, 1, 0, 1, 3, 3, 2, 3], np.int32)   # row 2 has no diagonal slot
    vals = np.array([2.0, -1.0, -1.0, 2.0, 0.5, 0.0, 0.5, 2.0])
    rp2 = np.array([0, 2, 4, 5, 8], np.int64)
    x, info = oracle.pcg_jacobi(oracle.CSR(n, rp2, np.array([0, 1, 0, 1, 3, 1, 2, 3], np.int32), vals),
                                np.ones(n), 1e-10, 10, lib=lib)
    assert info.status == oracle.ERR_NOT_SPD
    A = _poisson(5)
    x, info = oracle.pcg_jacobi(A, np.zeros(25), 1e-10, 10, lib=lib)
    assert info.status == oracle.OK and info.iterations == 0 and not np.any(x)


def pin_adjoint_jacobi(lib=None):
    """The adjoint of the Jacobi-PCG solve: g.x = lambda.b, the slot identity,
    lambda against dense LU on A^T, and central differences over the slots."""
    n = 40
    A, M = _scaled_spd(n, 21, spread=1.5)
    b = W.normal_rhs(n, 22)
    g = W.normal_rhs(n, 23)
    x, _ = oracle.pcg_jacobi(A, b, 1e-14, 2000, lib=lib)
    gb, gv, info = oracle.adjoint_jacobi(A, x, g, 1e-14, 2000, lib=lib)
    assert info.status == oracle.OK and info.converged
    assert abs(g @ x - gb @ b) <= 1e-9 * abs(g @ x)
    assert abs(A.vals @ gv + gb @ b) <= 1e-9 * abs(gb @ b)
    assert np.linalg.norm(gb - np.linalg.solve(M.T, g)) <= 1e-8 * np.linalg.norm(gb)
    rows = np.repeat(np.arange(n), np.diff(A.rowptr))
    for k in range(0, A.nnz, max(1, A.nnz // 25)):
        dlt = 1e-6 * max(1.0, abs(A.vals[k]))
        Mp, Mm = M.copy(), M.copy()
        Mp[rows[k], A.col[k]] += dlt
        Mm[rows[k], A.col[k]] -= dlt
        fd = (_dense_loss(Mp, b, g) - _dense_loss(Mm, b, g)) / (2 * dlt)
        assert abs(fd - gv[k]) <= 1e-5 * np.max(np.abs(gv)), k


# --------------------------------------------------------------------------
# Backward of the SpMV
# --------------------------------------------------------------------------

def _random_nonsym_csr(n, density, seed):
    rng = np.random.default_rng(seed)
    M = np.where(rng.random((n, n)) < density, rng.uniform(-2, 2, (n, n)), 0.0)
    M[3, 7] = 0.0
    rows, cols = np.nonzero(M)
    rows = np.append(rows, 3)
    cols = np.append(cols, 7)   # a stored explicit zero
    order = np.lexsort((cols, rows))
    rows, cols = rows[order], cols[order]
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    return oracle.CSR(n, np.cumsum(rp), cols.astype(np.int32), M[rows, cols].copy()), M, rows, cols


def pin_matvec_grad(lib=None):
    """y = A x with L = g.y: grad_x = A^T g (dense, within the summation
    bound), g.(A x) = (A^T g).x = sum_k vals_k grad_k, central differences in
    the slots, and a stored zero still gets g_i x_j."""
    n = 50
    A, M, rows, cols = _random_nonsym_csr(n, 0.1, 31)
    x = W.normal_rhs(n, 32)
    g = W.normal_rhs(n, 33)
    gx, gv = oracle.matvec_grad(A, x, g, lib=lib)
    dense = M.T @ g
    bound = 4 * n * EPS * (np.abs(M.T) @ np.abs(g))
    assert np.all(np.abs(gx - dense) <= bound + 1e-300)
    y = oracle.spmv(A, x, lib=lib)
    assert abs(g @ y - gx @ x) <= 1e-12 * (np.abs(g) @ np.abs(y) + 1)
    assert abs(g @ y - A.vals @ gv) <= 1e-12 * (np.abs(g) @ np.abs(y) + 1)
    k37 = [k for k in range(A.nnz) if rows[k] == 3 and cols[k] == 7][0]
    assert A.vals[k37] == 0.0 and gv[k37] == g[3] * x[7] != 0.0
    for k in range(0, A.nnz, 17):
        dlt = 1e-3
        Mp, Mm = M.copy(), M.copy()
        Mp[rows[k], cols[k]] += dlt
        Mm[rows[k], cols[k]] -= dlt
        fd = (g @ (Mp @ x) - g @ (Mm @ x)) / (2 * dlt)
        assert abs(fd - gv[k]) <= 1e-9 * max(1.0, abs(gv[k])), k


# --------------------------------------------------------------------------
# Lanczos eigsh and the Hellmann-Feynman gradient
# --------------------------------------------------------------------------

def _poisson_spectrum(N):
    return np.sort([eigval(N, i, j) for i in range(1, N + 1) for j in range(1, N + 1)])


def pin_eigsh_poisson(lib=None):
    """Ritz values of the Poisson matrix against the closed-form spectrum
    (multiple eigenvalues counted with multiplicity): the 4 largest after 300
    steps, the 4 smallest when the Krylov space is exhausted; the Ritz vector
    of the simple top eigenvalue is the closed-form v_NN."""
    N = 24
    A = _poisson(N)
    lam = _poisson_spectrum(N)
    v0 = W.normal_rhs(N * N, 70)
    th, X, res = oracle.eigsh(A, 4, "LA", v0, 150, lib=lib)
    # the residual estimate |beta_m y_m| is the true residual ||A v - theta v||
    for l in range(4):
        true = np.linalg.norm(oracle.spmv(A, X[l], lib=lib) - th[l] * X[l])
        assert abs(res[l] - true) <= 1e-13 + 1e-6 * true, (l, res[l], true)
    th, X, res = oracle.eigsh(A, 4, "LA", v0, 300, lib=lib)
    assert np.allclose(th, lam[-4:], rtol=0, atol=1e-10), (th, lam[-4:])
    assert np.all(res <= 1e-8)
    v = eigvec(N, N, N)
    v = v / np.linalg.norm(v)
    assert abs(abs(X[-1] @ v) - 1.0) <= 1e-10
    th, X, res = oracle.eigsh(A, 4, "SA", v0, N * N, lib=lib)
    assert np.allclose(th, lam[:4], rtol=0, atol=1e-10), (th, lam[:4])


def pin_eigsh_dense(lib=None):
    """A random sparse symmetric matrix with distinct eigenvalues: every Ritz
    value of the full-dimension process against dense eigh, an orthonormal
    basis, and V^T A V = T (tridiagonal)."""
    n = 120
    rng = np.random.default_rng(71)
    M = np.where(rng.random((n, n)) < 0.06, rng.uniform(-1, 1, (n, n)), 0.0)
    M = np.triu(M, 1)
    M = M + M.T + np.diag(rng.uniform(-2, 2, n))
    rows, cols = np.nonzero(M)
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    A = oracle.CSR(n, np.cumsum(rp), cols.astype(np.int32), M[rows, cols].copy())
    alpha, beta, V = oracle.lanczos(A, rng.standard_normal(n), n, lib=lib)
    k = alpha.shape[0]
    Vk = V[:k]
    assert np.max(np.abs(Vk @ Vk.T - np.eye(k))) <= 1e-12
    T = np.diag(alpha) + np.diag(beta[:k - 1], 1) + np.diag(beta[:k - 1], -1)
    assert np.max(np.abs(Vk @ M @ Vk.T - T)) <= 1e-10 * np.abs(M).sum(axis=1).max()
    if k == n:
        from scipy.linalg import eigh_tridiagonal
        th = eigh_tridiagonal(alpha, beta[:k - 1], eigvals_only=True)
        assert np.allclose(np.sort(th), np.linalg.eigvalsh(M), rtol=0, atol=1e-10)
    th, X, res = oracle.eigsh(A, 3, "SA", rng.standard_normal(n), n, lib=lib)
    ev, EV = np.linalg.eigh(M)
    assert np.allclose(th, ev[:3], rtol=0, atol=1e-10)
    for l in range(3):
        assert abs(abs(X[l] @ EV[:, l]) - 1.0) <= 1e-9


def pin_eig_grad(lib=None):
    """d lambda_max / d vals[k] against central differences of the perturbed
    (non-symmetric) matrix's largest eigenvalue; sum_k vals_k grad_k =
    v^T A v = lambda; a stored zero gets v_i v_j."""
    n = 30
    rng = np.random.default_rng(72)
    M = np.where(rng.random((n, n)) < 0.2, rng.uniform(-1, 1, (n, n)), 0.0)
    M = np.triu(M, 1)
    M = M + M.T + np.diag(np.linspace(-3, 3, n))
    M[2, 9] = M[9, 2] = 0.0
    mask = M != 0
    mask[2, 9] = mask[9, 2] = True   # stored zeros
    rows, cols = np.nonzero(mask)
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    A = oracle.CSR(n, np.cumsum(rp), cols.astype(np.int32), M[rows, cols].copy())
    th, X, _ = oracle.eigsh(A, 1, "LA", rng.standard_normal(n), n, lib=lib)
    v = X[0]
    gv = oracle.eig_grad(A, v, lib=lib)
    assert abs(A.vals @ gv - th[0]) <= 1e-12 * max(1.0, abs(th[0]))
    k29 = [k for k in range(A.nnz) if rows[k] == 2 and cols[k] == 9][0]
    assert A.vals[k29] == 0.0 and gv[k29] != 0.0
    for k in range(0, A.nnz, 7):
        d = 1e-6
        Mp, Mm = M.copy(), M.copy()
        Mp[rows[k], cols[k]] += d
        Mm[rows[k], cols[k]] -= d
        fd = (np.max(np.linalg.eigvals(Mp).real) - np.max(np.linalg.eigvals(Mm).real)) / (2 * d)
        assert abs(fd - gv[k]) <= 1e-6, (k, fd, gv[k])


# --------------------------------------------------------------------------
# BiCGStab and its adjoint
# --------------------------------------------------------------------------

def _csr_of(M):
    rows, cols = np.nonzero(M)
    rp = np.zeros(M.shape[0] + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    return oracle.CSR(M.shape[0], np.cumsum(rp), cols.astype(np.int32), M[rows, cols].copy())


def _convection_diffusion(N, eps=0.05):
    """2D upwind convection-diffusion on an N x N grid (flow along the grid
    lines): a non-symmetric M-matrix, dense for the LU check."""
    h = 1.0 / (N + 1)
    n = N * N
    M = np.zeros((n, n))
    for c in range(N):
        for a in range(N):
            i = c * N + a
            M[i, i] = 4 * eps / h ** 2 + 1 / h
            if a > 0:
                M[i, i - 1] = -eps / h ** 2 - 1 / h
            if a + 1 < N:
                M[i, i + 1] = -eps / h ** 2
            if c > 0:
                M[i, i - N] = -eps / h ** 2
            if c + 1 < N:
                M[i, i + N] = -eps / h ** 2
    return M


def pin_bicgstab_dense_lu(lib=None):
    """Converged BiCGStab against dense LU: convection-diffusion, a random
    non-symmetric diagonally dominant matrix, and the SPD Poisson matrix;
    the recursive residual agrees with the true residual b - A x."""
    rng = np.random.default_rng(80)
    R = np.where(rng.random((60, 60)) < 0.1, rng.uniform(-1, 1, (60, 60)), 0.0)
    R += np.diag(np.abs(R).sum(axis=1) + 1.0)
    cases = [_convection_diffusion(12), R, _poisson(10).to_dense()]
    for M in cases:
        A = _csr_of(M)
        b = rng.standard_normal(A.n)
        x, info = oracle.bicgstab(A, b, 1e-12, 2000, lib=lib)
        assert info.status == oracle.OK and info.converged, info
        xe = np.linalg.solve(M, b)
        assert np.linalg.norm(x - xe) <= 1e-9 * np.linalg.norm(xe)
        true = np.linalg.norm(b - M @ x) ** 2
        assert abs(true - info.rr) <= 1e-6 * max(true, info.rr) + 1e-26 * info.bb


def pin_bicgstab_scaling(lib=None):
    """(2A) x = b: rho is unchanged, alpha and omega halve, x halves -- all
    exactly, since every step only rescales by powers of two."""
    M = _convection_diffusion(9)
    A = _csr_of(M)
    A2 = oracle.CSR(A.n, A.rowptr, A.col, 2.0 * A.vals)
    b = W.uniform_rhs(A.n, 4)
    x1, i1, h1 = oracle.bicgstab(A, b, 1e-10, 500, history=True, lib=lib)
    x2, i2, h2 = oracle.bicgstab(A2, b, 1e-10, 500, history=True, lib=lib)
    assert i1.iterations == i2.iterations and i1.iterations > 3
    assert np.array_equal(x2, 0.5 * x1)
    assert np.array_equal(h2[0], h1[0])
    assert np.array_equal(h2[1], 0.5 * h1[1])
    assert np.array_equal(h2[2], 0.5 * h1[2])
    assert np.array_equal(h2[3], h1[3])


def pin_bicgstab_finite_termination(lib=None):
    """BiCG terminates in n steps, so for n = 2 and 3 BiCGStab's s vanishes
    (to rounding) in iteration n and it finishes there, on the half step,
    with the LU solution; for A = 2 I it finishes in iteration 1 with x = b/2
    exactly."""
    rng = np.random.default_rng(81)
    for n in (2, 3):
        for _ in range(5):
            M = rng.uniform(-1, 1, (n, n)) + 3 * np.eye(n)
            A = _csr_of(M)
            b = rng.standard_normal(n)
            x, info, h = oracle.bicgstab(A, b, 1e-10, 10, history=True, lib=lib)
            assert info.converged and info.iterations <= n, (n, info)
            assert h[2][info.iterations - 1] == 0.0   # ended on the half step
            assert np.allclose(x, np.linalg.solve(M, b), rtol=1e-12, atol=1e-14)
    A = _csr_of(2.0 * np.eye(7))
    b = W.uniform_rhs(7, 5)
    x, info = oracle.bicgstab(A, b, 1e-10, 10, lib=lib)
    assert info.iterations == 1 and np.array_equal(x, 0.5 * b)


def pin_bicgstab_statuses(lib=None):
    """b = 0: converged in 0 iterations with x = 0; a skew-symmetric rotation
    gives rhat . v = 0 at once (breakdown); a NaN value is non-finite; tol = 0
    runs exactly maxit iterations."""
    A = _csr_of(_convection_diffusion(5))
    x, info = oracle.bicgstab(A, np.zeros(A.n), 1e-8, 50, lib=lib)
    assert info.status == oracle.OK and info.iterations == 0 and not np.any(x)
    R = _csr_of(np.array([[0.0, 1.0], [-1.0, 0.0]]))
    x, info = oracle.bicgstab(R, np.array([1.0, 0.0]), 1e-8, 50, lib=lib)
    assert info.status == oracle.ERR_BREAKDOWN and info.iterations == 0
    Bad = oracle.CSR(A.n, A.rowptr, A.col, A.vals.copy())
    Bad.vals[4] = np.nan
    _, info = oracle.bicgstab(Bad, W.uniform_rhs(A.n, 6), 1e-8, 50, lib=lib)
    assert info.status == oracle.ERR_NONFINITE
    _, info = oracle.bicgstab(A, W.uniform_rhs(A.n, 6), 0.0, 7, lib=lib)
    assert info.status == oracle.OK and info.iterations == 7


def pin_adjoint_bicgstab(lib=None):
    """A^T lambda = g by BiCGStab on a non-symmetric matrix: lambda against
    LU of A^T; g.x = lambda.b; sum vals.grad = -lambda.b; central
    differences of L = g.x over stored slots (perturbed systems by LU)."""
    M = _convection_diffusion(7)
    A = _csr_of(M)
    rng = np.random.default_rng(82)
    b = rng.standard_normal(A.n)
    g = rng.standard_normal(A.n)
    x, info = oracle.bicgstab(A, b, 1e-13, 2000, lib=lib)
    lam, gv, ainfo = oracle.adjoint_bicgstab(A, x, g, 1e-13, 2000, lib=lib)
    assert ainfo.status == oracle.OK and ainfo.converged
    le = np.linalg.solve(M.T, g)
    assert np.linalg.norm(lam - le) <= 1e-9 * np.linalg.norm(le)
    assert abs(g @ x - lam @ b) <= 1e-9 * abs(g @ x)
    assert abs(A.vals @ gv + lam @ b) <= 1e-9 * abs(lam @ b)
    rows = np.repeat(np.arange(A.n), np.diff(A.rowptr))
    for k in range(0, A.nnz, 11):
        d = 1e-6
        Mp, Mm = M.copy(), M.copy()
        Mp[rows[k], A.col[k]] += d
        Mm[rows[k], A.col[k]] -= d
        fd = (g @ np.linalg.solve(Mp, b) - g @ np.linalg.solve(Mm, b)) / (2 * d)
        assert abs(fd - gv[k]) <= 1e-6 * max(1.0, abs(fd)), (k, fd, gv[k])


# --------------------------------------------------------------------------
# Locality ordering (breadth-first order of the pattern's graph)
# --------------------------------------------------------------------------

def _pattern_csr(n, edges, diag=True):
    """Symmetric pattern of an undirected edge list (values: a Laplacian +
    I, so that the matrix is SPD), rows' columns ascending."""
    M = np.zeros((n, n))
    for i, j in edges:
        M[i, j] = M[j, i] = -1.0
    M += np.diag(np.abs(M).sum(axis=1) + (1.0 if diag else 0.0))
    return _csr_of(M), M


def pin_bfs_order_hand(lib=None):
    """Orders worked out by hand.  A path 3-0-4-1-2: the longest rows (3
    slots) are 0, 4, 1, so the first visit starts at 0; the farthest nodes
    from 0 are {2} (3 edges); the visit from 2 lists 2, 1, 4, 0, 3.  Two
    pieces and an isolated node (edges 0-3, 3-5, 5-1, 2-6; 4 alone): start 3;
    farthest {1}; 1, 5, 3, 0, then the smallest unvisited index 2 (2, 6),
    then 4."""
    A, _ = _pattern_csr(5, [(3, 0), (0, 4), (4, 1), (1, 2)])
    assert oracle.bfs_order(A, lib=lib).tolist() == [2, 1, 4, 0, 3]
    A, _ = _pattern_csr(7, [(0, 3), (3, 5), (5, 1), (2, 6)])
    assert oracle.bfs_order(A, lib=lib).tolist() == [1, 5, 3, 0, 2, 6, 4]
    A, _ = _pattern_csr(1, [])
    assert oracle.bfs_order(A, lib=lib).tolist() == [0]
    # a star: centre 4 has the longest row; every leaf is 1 edge away, the
    # smallest is 0; from 0: 0, 4, then the other leaves ascending
    A, _ = _pattern_csr(6, [(4, 0), (4, 1), (4, 2), (4, 3), (4, 5)])
    assert oracle.bfs_order(A, lib=lib).tolist() == [0, 4, 1, 2, 3, 5]


def _scipy_bfs_order(A):
    """The same order from scipy's graph routines: distances from the start
    by unweighted shortest paths, each piece by breadth_first_order."""
    import scipy.sparse as sp
    from scipy.sparse.csgraph import breadth_first_order, shortest_path
    G = sp.csr_matrix((np.ones(A.nnz), A.col, A.rowptr), shape=(A.n, A.n))
    s0 = int(np.argmax(np.diff(A.rowptr)))
    d = shortest_path(G, directed=True, unweighted=True, indices=s0)
    far = np.max(d[np.isfinite(d)])
    s1 = int(np.flatnonzero(d == far).min())
    out = list(breadth_first_order(G, s1, directed=True, return_predecessors=False))
    seen = np.zeros(A.n, bool)
    seen[out] = True
    for i in range(A.n):
        if not seen[i]:
            piece = breadth_first_order(G, i, directed=True, return_predecessors=False)
            out += list(piece)
            seen[piece] = True
    return np.array(out)


def pin_bfs_order_scipy(lib=None):
    """Symmetric patterns with several pieces (a random geometric graph with
    isolated nodes, a grid, a random sparse matrix): the oracle's order is
    scipy's breadth-first order from the same start, piece by piece, and a
    permutation of 0..n-1."""
    row, col, val, _ = W.rgg_coo(3000, 11, 12, degree=4.0)
    rp, c, perm = oracle.csr_from_coo(3000, row, col)
    A = oracle.CSR(3000, rp, c, oracle.values_from_coo(perm, c.shape[0], val))
    cases = [A, _poisson(17), _random_spd_csr(300, 0.01, 5)[0]]
    for A in cases:
        o = oracle.bfs_order(A, lib=lib)
        assert np.array_equal(np.sort(o), np.arange(A.n))
        assert np.array_equal(o, _scipy_bfs_order(A))


def pin_permute_dense(lib=None):
    """P A P^T against the dense matrix indexed by the order; every row's
    columns ascending; src maps each new slot to the slot of A it holds."""
    A, M = _random_spd_csr(60, 0.08, 9)
    order = np.random.default_rng(3).permutation(60)
    B, src = oracle.permute(A, order, lib=lib)
    assert np.array_equal(B.to_dense(), M[np.ix_(order, order)])
    for t in range(B.n):
        assert np.all(np.diff(B.col[B.rowptr[t]:B.rowptr[t + 1]]) > 0)
    assert np.array_equal(B.vals, A.vals[src])
    assert np.array_equal(np.sort(src), np.arange(A.nnz))


ALL_PINS = [
    pin_csr_poisson_closed_form, pin_csr_brute_force, pin_csr_rgg_symmetric,
    pin_spmv_eigenpairs, pin_spmv_dense, pin_dot,
    pin_cg_one_step, pin_cg_m_step, pin_cg_dense_lu, pin_cg_manufactured,
    pin_cg_ritz, pin_cg_energy, pin_cg_statuses, pin_cg_warm_start,
    pin_adjoint_identities, pin_adjoint_fd, pin_adjoint_support, pin_adjoint_golden,
    pin_adjoint_nonsymmetric_flag, pin_batched_shift_spectrum,
    pin_pcg_uniform_diagonal, pin_pcg_scaled_equivalence, pin_pcg_diagonal_one_step,
    pin_pcg_dense_lu, pin_pcg_statuses, pin_adjoint_jacobi, pin_matvec_grad,
    pin_eigsh_poisson, pin_eigsh_dense, pin_eig_grad,
    pin_bicgstab_dense_lu, pin_bicgstab_scaling, pin_bicgstab_finite_termination,
    pin_bicgstab_statuses, pin_adjoint_bicgstab,
    pin_bfs_order_hand, pin_bfs_order_scipy, pin_permute_dense,
]
