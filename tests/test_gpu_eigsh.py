"""The .eigsh on the GPU (Lanczos with full reorthogonalisation) and the
Hellmann-Feynman gradient: Ritz values and vectors against the oracle's
Lanczos process on the same start vector, the closed-form Poisson spectrum,
the residual estimate against the true residual, finite differences of the
eigenvalue through autograd, the batch, and the degenerate cases."""
import numpy as np
import pytest

import oracle
import workloads as W
from closed_forms import eigval, eigvec, spectrum_bounds
from gpu_util import csr_handle, say, t

pytestmark = pytest.mark.gpu

TOL_THETA = 1e-10   # Ritz values: absolute, relative to the largest |eigenvalue|
TOL_VEC = 1e-9      # Ritz vectors: 1 - |x . x_ref|


def _sym_csr(n, per_row, seed, empty_diag_rows=()):
    """A random sparse symmetric matrix (ascending columns, a few rows
    without a diagonal entry) with well-spread eigenvalues."""
    rng = np.random.default_rng(seed)
    pairs = set()
    for i in range(n):
        for j in rng.integers(0, n, per_row):
            if i != j:
                pairs.add((min(i, int(j)), max(i, int(j))))
    rows, cols, vals = [], [], []
    for (i, j) in sorted(pairs):
        a = rng.uniform(-1, 1)
        rows += [i, j]
        cols += [j, i]
        vals += [a, a]
    for i in range(n):
        if i not in empty_diag_rows:
            rows.append(i)
            cols.append(i)
            vals.append(rng.uniform(-4, 4))
    rows, cols, vals = np.array(rows), np.array(cols), np.array(vals)
    order = np.lexsort((cols, rows))
    rows, cols, vals = rows[order], cols[order], vals[order]
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    return np.cumsum(rp).astype(np.int32), cols.astype(np.int32), vals


def _gpu_eigsh(rp, c, v, k, which, m, v0):
    import torch
    import krylov_solvers_adjoint_amd as K
    P = csr_handle(rp, c)
    th, X, res, infos = K.sla_eigsh(P, t(v), k, which, m, t(v0))
    torch.cuda.synchronize()
    return P, th.cpu().numpy(), X.cpu().numpy(), res.cpu().numpy(), infos


def _compare(rp, c, v, k, which, m, v0, scale):
    n = len(rp) - 1
    P, th, X, res, infos = _gpu_eigsh(rp, c, v, k, which, m, v0)
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    alpha, _, _ = oracle.lanczos(A, v0, m)
    tho, Xo, reso = oracle.eigsh(A, k, which, v0, m)
    say(f"n={n} k={k} {which} m={m}: steps gpu {infos[0].steps} oracle {alpha.shape[0]}, "
        f"max |dtheta| {np.max(np.abs(th - tho)):.2e}")
    assert infos[0].steps == alpha.shape[0]
    assert np.max(np.abs(th - tho)) <= TOL_THETA * scale
    # Ritz vectors: one by one for simple Ritz values; for a cluster of equal
    # ones (a multiple eigenvalue) only the spanned subspace is defined
    l = 0
    while l < k:
        e = l + 1
        while e < k and tho[e] - tho[e - 1] <= 1e-8 * scale:
            e += 1
        G = Xo[l:e] @ X[l:e].T
        off = np.linalg.norm(Xo[l:e] - G @ X[l:e])
        assert off <= np.sqrt(2 * TOL_VEC) * (e - l), (l, e, off)
        l = e
    assert np.allclose(res, reso, rtol=1e-3, atol=1e-10 * scale)
    return P, th, X, res


def _true_residuals(P, v, th, X):
    import torch
    import krylov_solvers_adjoint_amd as K
    Xt = t(X)
    out = []
    for l in range(th.shape[0]):
        y = K.sla_spmv(P, t(v), Xt[l].contiguous())
        torch.cuda.synchronize()
        out.append(np.linalg.norm(y.cpu().numpy() - th[l] * X[l]))
    return np.array(out)


def test_poisson_closed_form():
    """5-point Poisson on a 24 x 24 grid: the 4 largest and 4 smallest
    eigenvalues (counted with multiplicity) against the closed form."""
    N = 24
    rp, c, v = W.poisson_csr(N)
    lam = np.sort([eigval(N, p, q) for p in range(1, N + 1) for q in range(1, N + 1)])
    v0 = W.normal_rhs(N * N, 70)
    P, th, X, res = _compare(rp, c, v, 4, "LA", 300, v0, 8.0)
    assert np.allclose(th, lam[-4:], rtol=0, atol=1e-10)
    assert np.all(res <= 1e-8)
    true = _true_residuals(P, v, th, X)
    assert np.all(np.abs(true - res) <= 1e-12 + 1e-6 * true)
    assert np.max(np.abs(X @ X.T - np.eye(4))) <= 1e-10
    top = eigvec(N, N, N)
    assert 1.0 - abs(X[-1] @ top) / np.linalg.norm(top) <= 1e-10
    P, th, X, res = _compare(rp, c, v, 4, "SA", N * N, v0, 8.0)
    assert np.allclose(th, lam[:4], rtol=0, atol=1e-10)


@pytest.mark.parametrize("n,per_row,k,which,m,seed", [
    (3000, 3, 5, "LA", 120, 1),
    (3000, 3, 5, "SA", 120, 2),
    (700, 4, 3, "LA", 700, 3),     # to the end of the Krylov space
    (97, 2, 1, "SA", 40, 4),       # one partial tile
    (1200, 3, 2, "LA", 1000, 5),   # a tridiagonal too large for LDS
])
def test_random_symmetric(n, per_row, k, which, m, seed):
    rp, c, v = _sym_csr(n, per_row, seed, empty_diag_rows={0, n // 2})
    scale = float(np.max(np.abs(v))) * (2 * per_row + 1)
    _compare(rp, c, v, k, which, m, W.normal_rhs(n, 100 + seed), scale)


def test_four_rows_per_thread():
    """A Poisson grid of 777 x 777 (603729 unknowns, a ragged last
    workgroup) takes the kernels that hold 4 rows per thread."""
    N = 777
    rp, c, v = W.poisson_csr(N)
    _compare(rp, c, v, 3, "LA", 24, W.normal_rhs(N * N, 71), 8.0)


def test_eig_grad_against_oracle():
    """One vector with weight 1: bit for bit v_i v_j; three vectors with
    weights: the weighted sum of the oracle's outer products."""
    import torch
    import krylov_solvers_adjoint_amd as K
    n = 2000
    rp, c, v = _sym_csr(n, 3, 11)
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    P = csr_handle(rp, c)
    X = np.stack([W.normal_rhs(n, 200 + q) for q in range(3)])
    X /= np.linalg.norm(X, axis=1, keepdims=True)
    g1 = K.sla_eig_grad(P, t(v), t(X[:1]), t(np.ones(1)))
    g = np.array([0.5, -2.0, 1.25])
    g3 = K.sla_eig_grad(P, t(v), t(X), t(g))
    torch.cuda.synchronize()
    assert np.array_equal(g1.cpu().numpy(), oracle.eig_grad(A, X[0]))
    ref = sum(g[q] * oracle.eig_grad(A, X[q]) for q in range(3))
    assert np.max(np.abs(g3.cpu().numpy() - ref)) <= 1e-14 * np.max(np.abs(ref))


def test_autograd_finite_differences():
    """d(theta_max + theta_second) / d vals through SparseTensor.eigsh against
    central differences of the GPU eigenvalues under a symmetric perturbation
    of a pair of slots (i, j), (j, i): relative error below 1e-5."""
    import torch
    import krylov_solvers_adjoint_amd as K
    n = 400
    rp, c, v = _sym_csr(n, 3, 21)
    P = csr_handle(rp, c)
    v0 = t(W.normal_rhs(n, 300))
    vals = t(v).requires_grad_(True)
    S = K.SparseTensor(P, vals)
    th, X = S.eigsh(k=2, which="LA", m=n, v0=v0)
    th.sum().backward()
    grad = vals.grad.cpu().numpy()
    rows = np.repeat(np.arange(n), np.diff(rp))
    slot = {(int(rows[q]), int(c[q])): q for q in range(len(c))}
    rng = np.random.default_rng(5)
    picks = [q for q in rng.permutation(len(c)) if rows[q] < c[q]][:6]
    picks += [q for q in range(len(c)) if rows[q] == c[q]][:2]
    d = 1e-5
    for q in picks:
        i, j = int(rows[q]), int(c[q])
        both = [q] if i == j else [q, slot[(j, i)]]
        vp, vm = v.copy(), v.copy()
        vp[both] += d
        vm[both] -= d
        tp, _, _, _ = K.sla_eigsh(P, t(vp), 2, "LA", n, v0)
        tm, _, _, _ = K.sla_eigsh(P, t(vm), 2, "LA", n, v0)
        fd = (tp.sum().item() - tm.sum().item()) / (2 * d)
        an = float(sum(grad[s] for s in both))
        say(f"slot ({i},{j}): fd {fd:.10f} autograd {an:.10f}")
        assert abs(fd - an) <= 1e-5 * max(abs(an), 1e-3)


def test_batch_matches_single_systems():
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 30
    rp, c, v = W.poisson_csr(N)
    rows = np.repeat(np.arange(N * N), np.diff(rp))
    v2 = 0.5 * v + np.where(rows == c, 0.25, 0.0)   # symmetric: a diagonal shift
    vb = np.stack([v, v2])
    v0 = np.stack([W.normal_rhs(N * N, 80), W.normal_rhs(N * N, 81)])
    P = csr_handle(rp, c)
    th, X, res, infos = K.sla_eigsh(P, t(vb), 3, "LA", 200, t(v0))
    for s in range(2):
        th1, X1, res1, inf1 = K.sla_eigsh(P, t(vb[s]), 3, "LA", 200, t(v0[s]))
        torch.cuda.synchronize()
        assert infos[s].steps == inf1[0].steps
        assert np.array_equal(th[s].cpu().numpy(), th1.cpu().numpy())
        assert np.array_equal(X[s].cpu().numpy(), X1.cpu().numpy())
        assert np.array_equal(res[s].cpu().numpy(), res1.cpu().numpy())


def test_degenerate_cases():
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 12
    rp, c, v = W.poisson_csr(N)
    P = csr_handle(rp, c)
    n = N * N
    # zero start vector
    with pytest.raises(K.SlaError) as e:
        K.sla_eigsh(P, t(v), 2, "LA", 10, t(np.zeros(n)))
    assert e.value.status == K.ERR_ARG
    # sizes
    for k, m in ((0, 5), (6, 5), (2, n + 1)):
        with pytest.raises(K.SlaError) as e:
            K.sla_eigsh(P, t(v), k, "LA", m, t(np.ones(n)))
        assert e.value.status == K.ERR_ARG
    # an eigenvector as the start: one step, an invariant subspace
    ev = eigvec(N, 2, 3)
    th, X, res, infos = K.sla_eigsh(P, t(v), 1, "LA", 10, t(ev))
    torch.cuda.synchronize()
    assert infos[0].steps == 1 and infos[0].status == K.OK
    assert abs(th.item() - eigval(N, 2, 3)) <= 1e-13
    _, _, _, infos = K.sla_eigsh(P, t(v), 2, "LA", 10, t(ev), check=False)
    assert infos[0].steps == 1 and infos[0].status == K.ERR_KRYLOV
    # a 1 x 1 matrix
    P1 = csr_handle(np.array([0, 1], np.int32), np.array([0], np.int32))
    th, X, res, infos = K.sla_eigsh(P1, t(np.array([-2.5])), 1, "SA", 1, t(np.array([3.0])))
    torch.cuda.synchronize()
    assert abs(th.item() + 2.5) <= 1e-14 and abs(abs(X.item()) - 1.0) <= 1e-15
    assert infos[0].steps == 1


def test_fullsize_poisson_properties():
    """The 1000 x 1000 Poisson grid (10^6 unknowns) with 60 steps: the
    residual estimates equal the true residuals, the Ritz vectors are
    orthonormal, and every Ritz value lies inside the closed-form spectrum
    (Ritz values of a symmetric matrix interlace its eigenvalues)."""
    N = 1000
    rp, c, v = W.poisson_csr(N)
    P, th, X, res, infos = _gpu_eigsh(rp, c, v, 4, "LA", 60, W.normal_rhs(N * N, 72))
    lo, hi = spectrum_bounds(N)
    say(f"theta {th} resid {res} steps {infos[0].steps}")
    assert infos[0].steps == 60
    assert np.all(th <= hi + 1e-12) and np.all(th >= lo - 1e-12)
    assert np.all(np.diff(th) >= 0)
    true = _true_residuals(P, v, th, X)
    assert np.all(np.abs(true - res) <= 1e-10 + 1e-6 * true), (true, res)
    assert np.max(np.abs(X @ X.T - np.eye(4))) <= 1e-10
