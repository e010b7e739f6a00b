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
