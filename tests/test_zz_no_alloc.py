"""sla_cg_solve_noalloc (the CG solve for callers that cannot allocate)
against sla_cg_solve, the entry point it is a variant of, through the C ABI:
two calls in a row, the second on a smaller system (and a third on a system
small enough for the one-workgroup loop, with a start vector), each equal to
the existing entry point's result (iterations, x bit for bit, hence within
the 1e-8 bar) and to the oracle's within the bar; the calls allocate no
device memory (the library's accounting and torch's allocator unchanged);
a system beyond the scratch limit is refused with SLA_ERR_ARG."""
import ctypes
import gc

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_X, csr_handle, rel, say, t

pytestmark = pytest.mark.gpu


def _noalloc(P, vt, bt, x, tol, maxit, flags=0):
    import torch
    import krylov_solvers_adjoint_amd as K
    assert P.bind(vt) == 1
    info = K._Info()
    # handles of earlier tests that only the cycle collector frees would
    # change the library's count inside the window
    gc.collect()
    gc.disable()
    try:
        torch.cuda.synchronize()
        live0, _ = K.sla_memory_usage()
        torch0 = torch.cuda.memory_allocated()
        st = K._lib.sla_cg_solve_noalloc(P.handle, bt.data_ptr(), x.data_ptr(), float(tol),
                                         int(maxit), flags, ctypes.byref(info),
                                         torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        live1, _ = K.sla_memory_usage()
    finally:
        gc.enable()
    assert st == 0, K._lib.sla_last_error()
    # nothing allocated: neither by the library nor through torch
    assert live1 == live0 and torch.cuda.memory_allocated() == torch0
    return info


def _case(name, rp, c, v, b, tol, maxit, x0=None, one_group="auto"):
    import torch
    import krylov_solvers_adjoint_amd as K
    n = len(rp) - 1
    vt, bt = t(v), t(b)
    # the existing entry point, on a handle of its own ("off" where it would
    # take the resident grid loop, which the allocation-free variant does not)
    R = csr_handle(rp, c, one_group=one_group)
    x_ref, info_ref = K.sla_cg_solve(R, vt, bt, tol, maxit,
                                     x0=t(x0) if x0 is not None else None)
    torch.cuda.synchronize()
    # the allocation-free one, on a fresh handle (no workspace of its own)
    P = csr_handle(rp, c)
    x = t(x0) if x0 is not None else torch.full_like(bt, float("nan"))
    say(f"{name}: sla_cg_solve_noalloc n={n} tol={tol} maxit={maxit}")
    info = _noalloc(P, vt, bt, x, tol, maxit, K.FLAG_X0 if x0 is not None else 0)
    x, x_ref = x.cpu().numpy(), x_ref.cpu().numpy()
    Ao = oracle.CSR(n, rp.astype(np.int64), c, v)
    xo, io = oracle.cg(Ao, b, tol, maxit, x0=x0)
    say(f"{name}: iterations {info.iterations} (sla_cg_solve {info_ref.iterations}, oracle "
        f"{io.iterations}); x vs sla_cg_solve {rel(x, x_ref):.1e} (bitwise "
        f"{np.array_equal(x, x_ref)}), vs oracle {rel(x, xo):.1e}")
    assert info.status == info_ref.status == 0
    assert info.iterations == info_ref.iterations == io.iterations
    assert info.converged == info_ref.converged
    assert rel(x, x_ref) <= TOL_X and rel(x, xo) <= TOL_X
    assert np.array_equal(x, x_ref)  # the same kernels and grid: the same bits
    return P


def test_noalloc_matches_cg_solve_twice_then_smaller():
    import krylov_solvers_adjoint_amd as K
    oracle.set_threads(oracle.host_threads())
    # the 1000^2 workload: b = A u*, 1000 fixed iterations (the line walk)
    rp, c, v = W.poisson_csr(1000)
    _, b = W.manufactured(1000)
    _case("poisson1000 fixed", rp, c, v, b, 0.0, 1000, one_group="off")
    # a smaller system next (the row-order banded step), to a tolerance
    rp, c, v = W.poisson_csr(300)
    _case("poisson300 tol", rp, c, v, W.uniform_rhs(300 * 300, 3), 1e-10, 5000,
          one_group="off")
    # smaller still: the one-workgroup loop, from a start vector
    rp, c, v = W.poisson_csr(32)
    _case("poisson32 x0", rp, c, v, W.uniform_rhs(1024, 4), 1e-10, 5000,
          x0=W.normal_rhs(1024, 5))
    assert K.sla_cg_solve_noalloc is not None


def test_noalloc_refuses_what_it_cannot_hold():
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.poisson_csr(1500)  # 2.25M unknowns: beyond the 64 MiB scratch
    P = csr_handle(rp, c)
    vt, bt = t(v), t(W.uniform_rhs(1500 * 1500, 6))
    x = torch.zeros_like(bt)
    assert P.bind(vt) == 1
    info = K._Info()
    st = K._lib.sla_cg_solve_noalloc(P.handle, bt.data_ptr(), x.data_ptr(), 1e-8, 100, 0,
                                     ctypes.byref(info), None)
    assert st == K.ERR_ARG and b"limit" in K._lib.sla_last_error()
    # flags it does not take
    st = K._lib.sla_cg_solve_noalloc(P.handle, bt.data_ptr(), x.data_ptr(), 1e-8, 100,
                                     K.FLAG_JACOBI, ctypes.byref(info), None)
    assert st == K.ERR_ARG
    torch.cuda.synchronize()
