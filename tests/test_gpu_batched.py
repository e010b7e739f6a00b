"""Shared-pattern batch vs one oracle solve per system: 64 systems on the
128 x 128 Poisson pattern with diagonal shifts c_s ~ U(0,1) (seed 2),
b ~ N(0,1) (seed 3), tol 1e-8."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_GRAD, TOL_X, csr_handle, iters_close, rel, say, t

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,B", [(128, 64), (33, 5)])
def test_batched_forward_and_adjoint(N, B):
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, vals, b, shifts = W.batched_poisson(N, B, 2, 3)
    g = W.normal_rhs(N * N, 4, shape=(B, N * N))
    P = csr_handle(rp, c)
    vt = t(vals)
    x, infos = K.sla_cg_solve_batched(P, vt, t(b), 1e-8, 10000)
    gb, gv, ainfos = K.sla_cg_adjoint_batched(P, vt, x, t(g), 1e-8, 10000)
    torch.cuda.synchronize()
    xo, io = oracle.cg_batched(rp.astype(np.int64), c, vals, b, 1e-8, 10000)
    gbo, gvo, aio = oracle.adjoint_batched(rp.astype(np.int64), c, vals, xo, g, 1e-8, 10000)
    x, gb, gv = x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy()
    its = [i.iterations for i in infos]
    say(f"batched {B}x{N}^2: iterations {min(its)}..{max(its)} (total {sum(its)})")
    for s in range(B):
        assert infos[s].converged and ainfos[s].converged
        assert iters_close(infos[s].iterations, io[s].iterations), s
        assert iters_close(ainfos[s].iterations, aio[s].iterations), s
        assert rel(x[s], xo[s]) <= TOL_X, s
        assert rel(gb[s], gbo[s]) <= TOL_X, s
        assert rel(gv[s], gvo[s]) <= TOL_GRAD, s


def test_batched_equals_single_solves():
    """Each system of the batch gets the same bits as solving it alone (its
    kernels and partial sums do not depend on the other systems)... up to
    the grid split, so compare within rounding instead."""
    import torch
    import krylov_solvers_adjoint_amd as K
    N, B = 50, 4
    rp, c, vals, b, _ = W.batched_poisson(N, B, 2, 3)
    P = csr_handle(rp, c)
    xb, ib = K.sla_cg_solve_batched(P, t(vals), t(b), 1e-10, 5000)
    for s in range(B):
        Ps = csr_handle(rp, c)
        xs, i_s = K.sla_cg_solve(Ps, t(vals[s]), t(b[s]), 1e-10, 5000)
        torch.cuda.synchronize()
        assert iters_close(ib[s].iterations, i_s.iterations)
        assert rel(xb[s].cpu().numpy(), xs.cpu().numpy()) <= 1e-12


@pytest.mark.parametrize("one_group", ["auto", "off"])
def test_alternating_batch_sizes_on_one_handle(one_group):
    """One handle solving batches of 4, 2, 4, 8, 1 and 4 systems in turn (the
    buffers of a larger batch serve a smaller one; a larger batch
    reallocates; the captured graphs are kept per batch), with and without
    Jacobi: every call gives the bits of a fresh handle solving the same
    batch.  40^2 and 33^2 Poisson: the two-kernel loop ("off") and the
    one-workgroup loop."""
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 40 if one_group == "off" else 33
    n = N * N
    rp, c, vals, b, _ = W.batched_poisson(N, 8, 2, 3)
    g = W.normal_rhs(n, 4, shape=(8, n))
    P = csr_handle(rp, c, one_group=one_group)

    def run(H, B, jac):
        x, infos = K.sla_cg_solve_batched(H, t(vals[:B]), t(b[:B]), 1e-10, 5000, jacobi=jac)
        gb, gv, ai = K.sla_cg_adjoint_batched(H, t(vals[:B]), x, t(g[:B]), 1e-10, 5000,
                                              jacobi=jac)
        torch.cuda.synchronize()
        return ([a.cpu().numpy() for a in (x, gb, gv)],
                [i.iterations for i in infos] + [i.iterations for i in ai])

    for B, jac in ((4, False), (2, False), (4, True), (8, False), (1, True), (4, False)):
        got, its = run(P, B, jac)
        ref, its_ref = run(csr_handle(rp, c, one_group=one_group), B, jac)
        assert its == its_ref, (B, jac)
        for a1, a2 in zip(got, ref):
            assert np.array_equal(a1, a2), (B, jac)
