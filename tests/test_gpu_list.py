"""Lists of systems with distinct patterns (SparseTensorList): every system
of a list solve is its single solve bit for bit (the same kernels on its
own handle, run concurrently on worker streams; where the single solve takes
the resident grid loop, whose cooperative launch would serialize the list,
the list takes the two-kernel loop: the bits of a single solve with that
loop) and matches the oracle; the
adjoint list, the autograd node, Jacobi and BiCGStab lists, and the error
reporting of a failing system."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_GRAD, TOL_X, csr_handle, rel, t

pytestmark = pytest.mark.gpu


def _spd(n, per_row, seed):
    """Random sparse symmetric diagonally dominant matrix (SPD), CSR with
    ascending columns."""
    rng = np.random.default_rng(seed)
    pairs = {}
    for i in range(n):
        for j in rng.integers(0, n, per_row):
            if i != j:
                pairs[(min(i, int(j)), max(i, int(j)))] = rng.uniform(-1, 1)
    rows, cols, vals = [], [], []
    diag = np.full(n, 0.1)
    for (i, j), a in pairs.items():
        rows += [i, j]
        cols += [j, i]
        vals += [a, a]
        diag[i] += abs(a)
        diag[j] += abs(a)
    rows += list(range(n))
    cols += list(range(n))
    vals += list(diag)
    rows, cols, vals = np.array(rows), np.array(cols), np.array(vals)
    o = np.lexsort((cols, rows))
    rows, cols, vals = rows[o], cols[o], vals[o]
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    return np.cumsum(rp).astype(np.int32), cols.astype(np.int32), vals


def _cg_systems():
    out = []
    for N in (10, 33, 64):
        out.append(W.poisson_csr(N))
    out.append(_spd(500, 4, 1))
    out.append(_spd(2000, 6, 2))
    out.append(W.band_csr(3001, (-1000, -1, 1, 1000), 5.0))
    return out


def _resident(P) -> bool:
    """Whether the last solve on P ran the resident grid loop."""
    import krylov_solvers_adjoint_amd as K
    try:
        return K.sla_resident_loop_ms(P) > 0.0
    except K.SlaError:
        return False


def _oracle_A(rp, c, v):
    return oracle.CSR(len(rp) - 1, rp.astype(np.int64), c, v)


def test_cg_list_matches_single_solves_and_oracle():
    import torch
    import krylov_solvers_adjoint_amd as K
    systems = _cg_systems()
    Ps = [csr_handle(rp, c) for rp, c, _ in systems]
    vals = [t(v) for _, _, v in systems]
    bs = [t(W.normal_rhs(len(rp) - 1, 10 + i)) for i, (rp, _, _) in enumerate(systems)]
    xs, infos = K.sla_solve_list(Ps, vals, bs, 1e-10, 5000)
    torch.cuda.synchronize()
    single = []  # the handle whose single solves give the list's bits
    for i, (rp, c, v) in enumerate(systems):
        x1, i1 = K.sla_cg_solve(Ps[i], vals[i], bs[i], 1e-10, 5000)
        torch.cuda.synchronize()
        if _resident(Ps[i]):
            Q = csr_handle(rp, c, one_group="off")
            x1, i1 = K.sla_cg_solve(Q, vals[i], bs[i], 1e-10, 5000)
            torch.cuda.synchronize()
            single.append(Q)
        else:
            single.append(Ps[i])
        assert np.array_equal(xs[i].cpu().numpy(), x1.cpu().numpy()), i
        assert infos[i].iterations == i1.iterations and infos[i].converged
        xo, io = oracle.cg(_oracle_A(rp, c, v), bs[i].cpu().numpy(), 1e-10, 5000)
        assert rel(xs[i].cpu().numpy(), xo) <= TOL_X
    # the adjoint list against single adjoints
    gs = [t(W.normal_rhs(len(rp) - 1, 30 + i)) for i, (rp, _, _) in enumerate(systems)]
    gbs, gvs, ainf = K.sla_adjoint_list(Ps, vals, xs, gs, 1e-10, 5000)
    torch.cuda.synchronize()
    assert any(S is not P for S, P in zip(single, Ps))  # a resident-size system is listed
    for i in range(len(systems)):
        gb1, gv1, _ = K.sla_cg_adjoint(single[i], vals[i], xs[i], gs[i], 1e-10, 5000)
        torch.cuda.synchronize()
        assert np.array_equal(gbs[i].cpu().numpy(), gb1.cpu().numpy())
        assert np.array_equal(gvs[i].cpu().numpy(), gv1.cpu().numpy())


def test_jacobi_and_bicgstab_lists():
    import torch
    import krylov_solvers_adjoint_amd as K
    # Jacobi-preconditioned CG on SPD systems of different sizes
    systems = _cg_systems()[3:]
    Ps = [csr_handle(rp, c) for rp, c, _ in systems]
    vals = [t(v) for _, _, v in systems]
    bs = [t(W.normal_rhs(len(rp) - 1, 50 + i)) for i, (rp, _, _) in enumerate(systems)]
    xs, infos = K.sla_solve_list(Ps, vals, bs, 1e-10, 5000, jacobi=True)
    torch.cuda.synchronize()
    for i, (rp, c, v) in enumerate(systems):
        xo, _ = oracle.pcg_jacobi(_oracle_A(rp, c, v), bs[i].cpu().numpy(), 1e-10, 5000)
        assert infos[i].converged and rel(xs[i].cpu().numpy(), xo) <= TOL_X
    # BiCGStab on non-symmetric systems
    systems = [W.convection_diffusion_csr(N) for N in (20, 45, 80)]
    Ps = [csr_handle(rp, c) for rp, c, _ in systems]
    vals = [t(v) for _, _, v in systems]
    bs = [t(W.normal_rhs(len(rp) - 1, 60 + i)) for i, (rp, _, _) in enumerate(systems)]
    xs, infos = K.sla_solve_list(Ps, vals, bs, 1e-12, 5000, method="bicgstab")
    torch.cuda.synchronize()
    for i, (rp, c, v) in enumerate(systems):
        x1, _ = K.sla_bicgstab_solve(Ps[i], vals[i], bs[i], 1e-12, 5000)
        torch.cuda.synchronize()
        assert np.array_equal(xs[i].cpu().numpy(), x1.cpu().numpy())
        xo, _ = oracle.bicgstab(_oracle_A(rp, c, v), bs[i].cpu().numpy(), 1e-12, 5000)
        assert infos[i].converged and rel(xs[i].cpu().numpy(), xo) <= TOL_X
    gs = [t(W.normal_rhs(len(rp) - 1, 70 + i)) for i, (rp, _, _) in enumerate(systems)]
    gbs, gvs, _ = K.sla_adjoint_list(Ps, vals, xs, gs, 1e-12, 5000, method="bicgstab")
    torch.cuda.synchronize()
    for i, (rp, c, v) in enumerate(systems):
        lo, gvo, _ = oracle.adjoint_bicgstab(_oracle_A(rp, c, v), xs[i].cpu().numpy(),
                                             gs[i].cpu().numpy(), 1e-12, 5000)
        assert rel(gbs[i].cpu().numpy(), lo) <= TOL_X
        assert rel(gvs[i].cpu().numpy(), gvo) <= TOL_GRAD


def test_sparse_tensor_list_autograd():
    """L = sum_i g_i . x_i through SparseTensorList.solve: gradients in every
    item's values and right-hand side against the oracle's adjoints."""
    import torch
    import krylov_solvers_adjoint_amd as K
    systems = _cg_systems()
    vals = [t(v).requires_grad_(True) for _, _, v in systems]
    L = K.SparseTensorList([K.SparseTensor(csr_handle(rp, c), vv)
                            for (rp, c, _), vv in zip(systems, vals)])
    bs = [t(W.normal_rhs(len(rp) - 1, 80 + i)).requires_grad_(True)
          for i, (rp, _, _) in enumerate(systems)]
    gs = [W.normal_rhs(len(rp) - 1, 90 + i) for i, (rp, _, _) in enumerate(systems)]
    xs = L.solve(bs, tol=1e-12, maxit=5000)
    loss = sum((x * t(g)).sum() for x, g in zip(xs, gs))
    loss.backward()
    for i, (rp, c, v) in enumerate(systems):
        A = _oracle_A(rp, c, v)
        xo, _ = oracle.cg(A, bs[i].detach().cpu().numpy(), 1e-12, 5000)
        lo, gvo, _ = oracle.adjoint(A, xo, gs[i], 1e-12, 5000)
        assert rel(bs[i].grad.cpu().numpy(), lo) <= TOL_X
        assert rel(vals[i].grad.cpu().numpy(), gvo) <= TOL_GRAD


def test_list_errors():
    import ctypes
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.poisson_csr(12)
    P = csr_handle(rp, c)
    vt = t(v)
    b = t(W.normal_rhs(144, 1))
    with pytest.raises(ValueError):
        K.sla_solve_list([P, P], [vt, vt], [b, b], 1e-8, 100)
    # the C ABI rejects a handle listed twice, too
    P.bind(vt)
    hs = (ctypes.c_void_p * 2)(P.handle, P.handle)
    ptrs = (ctypes.c_void_p * 2)(b.data_ptr(), b.data_ptr())
    x = torch.empty_like(b)
    xp = (ctypes.c_void_p * 2)(x.data_ptr(), x.data_ptr())
    assert K._lib.sla_solve_list(2, hs, ptrs, xp, 1e-8, 100, 0, 0, None, None) == K.ERR_ARG
    # a failing system is named; the others are still solved
    rpi, ci, vi = W.poisson_csr(10)
    vbad = -vi                      # negative definite: CG breaks down at once
    Q = csr_handle(rpi, ci)
    R = csr_handle(rp, c)
    b2 = t(W.normal_rhs(100, 2))
    xs, infos = K.sla_solve_list([R, Q], [vt, t(vbad)], [b, b2], 1e-8, 500, check=False)
    torch.cuda.synchronize()
    assert infos[0].converged and infos[1].status == K.ERR_NOT_SPD
    with pytest.raises(K.SlaError) as e:
        K.sla_solve_list([R, Q], [vt, t(vbad)], [b, b2], 1e-8, 500)
    assert "system 1" in str(e.value)
