"""GPU CG solve and adjoint vs the oracle (x, lambda within 1e-8 relative L2,
grad_vals within 1e-7, iteration counts within 2 %), degenerate cases,
reproducibility and the autograd node."""
import numpy as np
import pytest

import oracle
import workloads as W
from closed_forms import eigval, eigvec
from gpu_util import TOL_GRAD, TOL_X, csr_handle, iters_close, rel, say, t

pytestmark = pytest.mark.gpu


def _poisson(N, rp_dtype=np.int32):
    rp, c, v = W.poisson_csr(N, rp_dtype)
    return rp, c, v, oracle.CSR(N * N, rp.astype(np.int64), c, v)


def _solve_pair(rp, c, v, Ao, b, g, tol, maxit, graph_block=None, one_group="auto"):
    import torch
    import krylov_solvers_adjoint_amd as K
    P = csr_handle(rp, c, one_group=one_group)
    if graph_block is not None:
        P.set_graph_block(graph_block)
    vt = t(v)
    x, info = K.sla_cg_solve(P, vt, t(b), tol, maxit)
    gb, gv, ainfo = K.sla_cg_adjoint(P, vt, x, t(g), tol, maxit)
    torch.cuda.synchronize()
    xo, io = oracle.cg(Ao, b, tol, maxit)
    gbo, gvo, aio = oracle.adjoint(Ao, xo, g, tol, maxit)
    return (x.cpu().numpy(), info, gb.cpu().numpy(), gv.cpu().numpy(), ainfo,
            xo, io, gbo, gvo, aio)


@pytest.mark.parametrize("one_group", ["auto", "off"])
def test_poisson32_forward_and_adjoint(one_group):
    """The 32 x 32 Poisson workload: b ~ U(-1,1) seed 0, g ~ N(0,1) seed 1,
    tol 1e-10 forward and adjoint (the one-workgroup loop and the two-kernel
    loop)."""
    rp, c, v, Ao = _poisson(32)
    b = W.uniform_rhs(1024, 0)
    g = W.normal_rhs(1024, 1)
    x, info, gb, gv, ainfo, xo, io, gbo, gvo, aio = _solve_pair(rp, c, v, Ao, b, g, 1e-10, 10000,
                                                                one_group=one_group)
    say(f"poisson32 {one_group}: iters gpu {info.iterations} oracle {io.iterations}; adjoint gpu "
        f"{ainfo.iterations} oracle {aio.iterations}; x {rel(x, xo):.2e} lam {rel(gb, gbo):.2e} "
        f"gv {rel(gv, gvo):.2e}")
    assert info.converged and ainfo.converged
    assert iters_close(info.iterations, io.iterations)
    assert iters_close(ainfo.iterations, aio.iterations)
    assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD


@pytest.mark.parametrize("graph_block", [0, 1, 7, 32])
def test_graph_blocks_give_identical_bits(graph_block):
    """Graph capture and polling granularity change speed only."""
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v, _ = _poisson(45)
    b = W.uniform_rhs(45 * 45, 3)
    ref = None
    for gbk in (32, graph_block):
        P = csr_handle(rp, c, one_group="off")  # 2025 unknowns: keep the graph loop
        P.set_graph_block(gbk)
        x, info = K.sla_cg_solve(P, t(v), t(b), 1e-9, 5000)
        torch.cuda.synchronize()
        cur = (x.cpu().numpy(), info.iterations)
        if ref is None:
            ref = cur
        else:
            assert np.array_equal(cur[0], ref[0]) and cur[1] == ref[1]


def test_one_workgroup_per_cu():
    """The one-workgroup-per-CU grid: CG and the adjoint still match the
    oracle, two runs give the same bits, and the SpMV is unchanged."""
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 150
    rp, c, v, Ao = _poisson(N)
    b = W.uniform_rhs(N * N, 5)
    g = W.normal_rhs(N * N, 6)
    runs = []
    for _ in range(2):
        P = csr_handle(rp, c)
        P.set_workgroups_per_cu(1)
        vt = t(v)
        x, info = K.sla_cg_solve(P, vt, t(b), 1e-10, 5000)
        gb, gv, ai = K.sla_cg_adjoint(P, vt, x, t(g), 1e-10, 5000)
        y = K.sla_spmv(P, vt, t(b))
        torch.cuda.synchronize()
        runs.append((x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy(), y.cpu().numpy(),
                     info.iterations, ai.iterations))
    for u, w in zip(*runs):
        assert np.array_equal(np.asarray(u), np.asarray(w))
    xo, io = oracle.cg(Ao, b, 1e-10, 5000)
    gbo, gvo, aio = oracle.adjoint(Ao, xo, g, 1e-10, 5000)
    x, gb, gv, y, it, ait = runs[0]
    assert np.array_equal(y, oracle.spmv(Ao, b))
    assert iters_close(it, io.iterations) and iters_close(ait, aio.iterations)
    assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD
    # automatic (the default): one workgroup per CU at this size, so the
    # same bits as the explicit setting
    Q = csr_handle(rp, c)
    Q.set_workgroups_per_cu(0)
    xa, ia = K.sla_cg_solve(Q, t(v), t(b), 1e-10, 5000)
    torch.cuda.synchronize()
    assert np.array_equal(xa.cpu().numpy(), x) and ia.iterations == it
    with pytest.raises(K.SlaError):
        P.set_workgroups_per_cu(3)


def test_reproducible_bits_and_history():
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 64
    rp, c, v, Ao = _poisson(N)
    b = W.uniform_rhs(N * N, 0)
    g = W.normal_rhs(N * N, 1)
    P = csr_handle(rp, c)
    runs = []
    for _ in range(2):
        x, info = K.sla_cg_solve(P, t(v), t(b), 1e-10, 10000, history=True)
        hist = P.history()
        gb, gv, ai = K.sla_cg_adjoint(P, t(v), x, t(g), 1e-10, 10000)
        torch.cuda.synchronize()
        runs.append((x.cpu().numpy(), info.iterations, hist, gb.cpu().numpy(), gv.cpu().numpy()))
    a, bb = runs
    assert np.array_equal(a[0], bb[0]) and a[1] == bb[1]
    for h1, h2 in zip(a[2], bb[2]):
        assert np.array_equal(h1, h2)
    assert np.array_equal(a[3], bb[3]) and np.array_equal(a[4], bb[4])
    # the history matches the oracle's alpha, beta, rr closely
    xo, io, (ao, bo, ro) = oracle.cg(Ao, b, 1e-10, 10000, history=True)
    k = min(len(ao), len(a[2][0]))
    assert np.max(np.abs(a[2][0][:k] - ao[:k]) / np.abs(ao[:k])) < 1e-8
    assert np.max(np.abs(a[2][1][:k] - bo[:k]) / np.abs(bo[:k])) < 1e-6


def test_ragged_sizes_and_int64_rowptr():
    for N, rpd in ((1, np.int32), (2, np.int32), (17, np.int64), (23, np.int32),
                   (130, np.int64)):
        rp, c, v, Ao = _poisson(N, rpd)
        n = N * N
        b = W.uniform_rhs(n, N)
        g = W.normal_rhs(n, N + 1)
        x, info, gb, gv, ainfo, xo, io, gbo, gvo, aio = _solve_pair(rp, c, v, Ao, b, g, 1e-10,
                                                                    10000)
        say(f"N={N}: iters {info.iterations}/{io.iterations} x {rel(x, xo):.1e}")
        assert iters_close(info.iterations, io.iterations)
        assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD


def test_fixed_iterations_tol0():
    """tol = 0 runs exactly maxit iterations; the manufactured solution of the
    1000 x 1000 workload, at 300 x 300 here so the oracle stays quick."""
    N = 300
    rp, c, v, Ao = _poisson(N)
    u, b = W.manufactured(N)
    g = W.normal_rhs(N * N, 1)
    x, info, gb, gv, ainfo, xo, io, gbo, gvo, aio = _solve_pair(rp, c, v, Ao, b, g, 0.0, 1000)
    say(f"fixed: x {rel(x, xo):.2e} lam {rel(gb, gbo):.2e} gv {rel(gv, gvo):.2e} "
        f"|x-u*| {rel(x, u):.2e}")
    assert info.iterations == 1000 and ainfo.iterations == 1000
    assert not info.converged
    assert rel(x, xo) <= TOL_X and rel(gb, gbo) <= TOL_X and rel(gv, gvo) <= TOL_GRAD
    assert rel(x, u) <= 1e-12


def test_eigenvector_rhs_one_iteration():
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 40
    rp, c, v, _ = _poisson(N)
    vec = eigvec(N, 3, 5)
    P = csr_handle(rp, c)
    x, info = K.sla_cg_solve(P, t(v), t(vec), 1e-10, 100)
    torch.cuda.synchronize()
    assert info.iterations == 1
    assert rel(x.cpu().numpy(), vec / eigval(N, 3, 5)) <= 1e-12


@pytest.mark.parametrize("one_group", ["auto", "off"])
def test_degenerate_cases(one_group):
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 10
    rp, c, v, Ao = _poisson(N)
    n = N * N
    P = csr_handle(rp, c, one_group=one_group)
    # b = 0: no iteration, x = 0
    x, info = K.sla_cg_solve(P, t(v), t(np.zeros(n)), 1e-10, 100)
    assert info.iterations == 0 and info.converged and float(x.abs().max()) == 0.0
    # maxit = 0
    x, info = K.sla_cg_solve(P, t(v), t(W.uniform_rhs(n, 1)), 1e-10, 0)
    assert info.iterations == 0 and not info.converged
    # NaN right-hand side
    bad = W.uniform_rhs(n, 1)
    bad[17] = np.nan
    with pytest.raises(K.SlaError) as e:
        K.sla_cg_solve(P, t(v), t(bad), 1e-10, 100)
    assert e.value.status == K.ERR_NONFINITE
    # negative definite: breakdown at the first iteration, x = 0
    x, info = K.sla_cg_solve(P, t(-v), t(W.uniform_rhs(n, 2)), 1e-10, 100, check=False)
    assert info.status == K.ERR_NOT_SPD and info.iterations == 0
    # maxit = 1
    x, info = K.sla_cg_solve(P, t(v), t(W.uniform_rhs(n, 3)), 1e-10, 1)
    xo, io = oracle.cg(Ao, W.uniform_rhs(n, 3), 1e-10, 1)
    assert info.iterations == 1 and rel(x.cpu().numpy(), xo) <= 1e-14
    # warm start
    b = W.uniform_rhs(n, 4)
    x0 = W.normal_rhs(n, 5)
    x, info = K.sla_cg_solve(P, t(v), t(b), 1e-12, 1000, x0=t(x0))
    xo, io = oracle.cg(Ao, b, 1e-12, 1000, x0=x0)
    assert iters_close(info.iterations, io.iterations) and rel(x.cpu().numpy(), xo) <= TOL_X
    # n = 1
    P1 = csr_handle(np.array([0, 1], np.int32), np.array([0], np.int32), one_group=one_group)
    x, info = K.sla_cg_solve(P1, t(np.array([2.5])), t(np.array([3.0])), 1e-12, 10)
    gb, gv, _ = K.sla_cg_adjoint(P1, t(np.array([2.5])), x, t(np.array([-1.5])), 1e-12, 10)
    torch.cuda.synchronize()
    assert info.iterations == 1 and abs(float(x[0]) - 1.2) <= 4e-16
    assert abs(float(gb[0]) + 0.6) <= 4e-16 and abs(float(gv[0]) - 1.5 * 3.0 / 6.25) <= 8e-16
    # argument errors
    with pytest.raises(K.SlaError) as e:
        K.sla_cg_solve(P, t(v), t(b), -1.0, 10)
    assert e.value.status == K.ERR_ARG


def test_pattern_grad_bitexact():
    """One correctly rounded product per slot: bit-identical to the oracle
    given the same lambda and x."""
    import torch
    import krylov_solvers_adjoint_amd as K
    n = 20000
    row, col, val, _ = W.rgg_coo(n, 4, 5)
    rp, c, perm = oracle.csr_from_coo(n, row, col)
    vals = oracle.values_from_coo(perm, int(rp[-1]), val)
    lam = W.normal_rhs(n, 8)
    x = W.normal_rhs(n, 9)
    P = csr_handle(rp.astype(np.int32), c)
    gv = K.sla_pattern_grad(P, t(vals), t(lam), t(x))
    torch.cuda.synchronize()
    go = oracle.pattern_grad(oracle.CSR(n, rp, c, vals), lam, x)
    assert np.array_equal(gv.cpu().numpy(), go)


def test_autograd_one_node():
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 24
    rp, c, v, Ao = _poisson(N)
    n = N * N
    b = W.uniform_rhs(n, 0)
    g = W.normal_rhs(n, 1)
    P = csr_handle(rp, c)
    vt = t(v).requires_grad_(True)
    bt = t(b).requires_grad_(True)
    x = K.SparseTensor(P, vt).solve(bt, tol=1e-12, maxit=5000)
    # one node between the leaves and x: the solve itself
    assert type(x.grad_fn).__name__ == "_CGSolveBackward"
    assert [type(f[0]).__name__ for f in x.grad_fn.next_functions[:2]] == ["AccumulateGrad"] * 2
    (x * t(g)).sum().backward()
    torch.cuda.synchronize()
    xo, _ = oracle.cg(Ao, b, 1e-12, 5000)
    gbo, gvo, _ = oracle.adjoint(Ao, xo, g, 1e-12, 5000)
    assert rel(bt.grad.cpu().numpy(), gbo) <= TOL_X
    assert rel(vt.grad.cpu().numpy(), gvo) <= TOL_GRAD
