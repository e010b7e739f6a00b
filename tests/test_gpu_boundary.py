"""The C ABI's handle views, owned values, memory accounting and symmetry
guard, called through ctypes as a C caller would:

* sla_csr_arrays returns the pattern's device arrays (the same addresses as
  sla_csr_pattern) and the bound values; sla_csr_load_values copies values
  into the handle (from COO triplets, merged as the oracle merges them, or
  in CSR order) and products with them match the oracle bit for bit, also
  after an in-place update through the returned address and after the
  caller's source array is overwritten.
* sla_memory_usage counts what a handle and its workspace allocate and what
  destroying it frees.
* CG needs A^T = A (Methodology 2 of the torch-sla explainer: the backward
  pass solves A^T lambda = dL/dx with A in place of A^T): a pattern that is
  not symmetric is refused by the CG solve, adjoint and list calls; values
  that are not symmetric are refused by the adjoint (the oracle's adjoint
  flags the same inputs); BiCGStab still takes them.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_X, rel, t

pytestmark = pytest.mark.gpu


def _hip():
    import torch  # noqa: F401  (the HIP runtime torch loaded)
    h = ctypes.CDLL("libamdhip64.so.7")
    h.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    h.hipMemcpy.restype = ctypes.c_int
    return h


def _memcpy(dst: int, src: int, nbytes: int):
    assert _hip().hipMemcpy(dst, src, nbytes, 3) == 0  # device to device


def _arrays(lib, h):
    rp, c, v, pm = (ctypes.c_void_p() for _ in range(4))
    assert lib.sla_csr_arrays(h, ctypes.byref(rp), ctypes.byref(c), ctypes.byref(v),
                              ctypes.byref(pm)) == 0
    return rp.value or 0, c.value or 0, v.value or 0, pm.value or 0


def _spmv(lib, h, x):
    import torch
    y = torch.empty_like(x)
    st = lib.sla_spmv(h, x.data_ptr(), y.data_ptr(), None)
    torch.cuda.synchronize()
    assert st == 0, lib.sla_last_error()
    return y.cpu().numpy()


def test_arrays_and_owned_values():
    import torch
    import krylov_solvers_adjoint_amd as K
    lib = K._lib
    N = 40
    n = N * N
    row, col, val = W.poisson_coo(N)
    row, col, val = W.shuffled_coo(row, col, val, 11, dup_frac=0.2)
    rt, ct, vt = t(row.astype(np.int32)), t(col.astype(np.int32)), t(val)
    h = ctypes.c_void_p()
    assert lib.sla_csr_create(n, row.shape[0], K.I32, rt.data_ptr(), ct.data_ptr(), K.I32, None,
                              ctypes.byref(h)) == 0
    try:
        rp, c, pm = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        assert lib.sla_csr_pattern(h, ctypes.byref(rp), ctypes.byref(c), ctypes.byref(pm)) == 0
        a_rp, a_c, a_v, a_pm = _arrays(lib, h)
        assert (a_rp, a_c, a_pm) == (rp.value, c.value, pm.value) and a_v == 0
        rp_o, c_o, perm_o = oracle.csr_from_coo(n, row, col)
        nnz = int(rp_o[-1])
        vals_o = oracle.values_from_coo(perm_o, nnz, val)
        A = oracle.CSR(n, rp_o, c_o, vals_o)
        x = W.normal_rhs(n, 12)
        xt = t(x)
        # COO values merged into a copy the handle owns
        assert lib.sla_csr_load_values(h, vt.data_ptr(), 1, K.VALUES_COO, None) == 0
        owned = _arrays(lib, h)[2]
        assert owned not in (0, vt.data_ptr())
        vt.fill_(7.0)  # the caller's array no longer matters
        assert np.array_equal(_spmv(lib, h, xt), oracle.spmv(A, x))
        # in-place update through the returned address: values = 2 vals_o
        v2 = t(2.0 * vals_o)
        _memcpy(owned, v2.data_ptr(), 8 * nnz)
        assert np.array_equal(_spmv(lib, h, xt), oracle.spmv(oracle.CSR(n, rp_o, c_o, 2.0 * vals_o), x))
        # a caller's array bound in place, then the owned copy again
        v3 = t(3.0 * vals_o)
        assert lib.sla_csr_set_values(h, v3.data_ptr(), 1) == 0
        assert _arrays(lib, h)[2] == v3.data_ptr()
        assert np.array_equal(_spmv(lib, h, xt), oracle.spmv(oracle.CSR(n, rp_o, c_o, 3.0 * vals_o), x))
        assert lib.sla_csr_set_values(h, owned, 1) == 0
        assert np.array_equal(_spmv(lib, h, xt), oracle.spmv(oracle.CSR(n, rp_o, c_o, 2.0 * vals_o), x))
        # CSR-order values of a batch of two: a new owned array
        vb = t(np.stack([vals_o, 4.0 * vals_o]))
        assert lib.sla_csr_load_values(h, vb.data_ptr(), 2, K.VALUES_CSR, None) == 0
        xb = t(np.stack([x, x]))
        yb = _spmv(lib, h, xb)
        assert np.array_equal(yb[0], oracle.spmv(A, x))
        assert np.array_equal(yb[1], oracle.spmv(oracle.CSR(n, rp_o, c_o, 4.0 * vals_o), x))
        # a CG solve on owned values against the oracle: the merged pattern
        # is the Laplacian's (the duplicates above carry arbitrary values,
        # so the Laplacian's own values, in CSR order, are loaded)
        vp = W.poisson_csr(N)[2]
        A = oracle.CSR(n, rp_o, c_o, vp)
        assert lib.sla_csr_load_values(h, t(vp).data_ptr(), 1, K.VALUES_CSR, None) == 0
        b = W.uniform_rhs(n, 13)
        bt = t(b)
        xs = torch.empty_like(bt)
        info = K._Info()
        assert lib.sla_cg_solve(h, bt.data_ptr(), xs.data_ptr(), 1e-10, 5000, 0,
                                ctypes.byref(info), None) == 0
        xo, io = oracle.cg(A, b, 1e-10, 5000)
        assert info.iterations == io.iterations and rel(xs.cpu().numpy(), xo) <= TOL_X
        # COO order needs a COO-built handle; a bad order is an argument error
        assert lib.sla_csr_load_values(h, vt.data_ptr(), 1, 7, None) == K.ERR_ARG
    finally:
        torch.cuda.synchronize()
        lib.sla_csr_destroy(h)
    rp_c, c_c, v_c = W.poisson_csr(8)
    P = K.sla_csr_create_from_csr(t(rp_c), t(c_c))
    assert lib.sla_csr_load_values(P.handle, t(v_c).data_ptr(), 1, K.VALUES_COO,
                                   None) == K.ERR_ARG
    assert K.sla_csr_arrays(P)["perm"] == 0


def test_memory_usage_counts_handles():
    import torch
    import krylov_solvers_adjoint_amd as K
    torch.cuda.synchronize()
    live0, _ = K.sla_memory_usage(reset_peak=True)
    N = 300
    n = N * N
    rp, c, v = W.poisson_csr(N)
    P = K.sla_csr_create_from_csr(t(rp), t(c))
    live1, _ = K.sla_memory_usage()
    # the pattern: row pointers, columns and the band mask at least
    assert live1 - live0 >= 4 * (n + 1) + 4 * len(c)
    x, _ = K.sla_cg_solve(P, t(v), t(W.uniform_rhs(n, 0)), 0.0, 10)
    torch.cuda.synchronize()
    live2, peak2 = K.sla_memory_usage()
    # the workspace: r, two search directions and q, n doubles each
    assert live2 - live1 >= 4 * 8 * n and peak2 >= live2
    P.close()
    torch.cuda.synchronize()
    live3, peak3 = K.sla_memory_usage()
    assert live3 == live0 and peak3 == peak2


def _nonsym_pattern(n, seed):
    """Tridiagonal SPD values plus one extra stored (i, j) without (j, i)."""
    rng = np.random.default_rng(seed)
    rows, cols, vals = [], [], []
    for i in range(n):
        for j in (i - 1, i, i + 1):
            if 0 <= j < n:
                rows.append(i)
                cols.append(j)
                vals.append(4.0 if i == j else -1.0)
    i = int(rng.integers(0, n - 3))
    rows.append(i)
    cols.append(i + 3)
    vals.append(-0.5)
    order = np.lexsort((cols, rows))
    rows, cols, vals = np.array(rows)[order], np.array(cols)[order], np.array(vals)[order]
    rp = np.zeros(n + 1, np.int64)
    np.add.at(rp, rows + 1, 1)
    return np.cumsum(rp).astype(np.int32), cols.astype(np.int32), vals


def test_cg_refuses_a_pattern_that_is_not_symmetric():
    import torch
    import krylov_solvers_adjoint_amd as K
    n = 5000
    rp, c, v = _nonsym_pattern(n, 3)
    P = K.sla_csr_create_from_csr(t(rp), t(c))
    b = t(W.uniform_rhs(n, 4))
    x = torch.full_like(b, 123.0)
    infos = (K._Info * 1)()
    assert P.bind(t(v)) == 1
    st = K._lib.sla_cg_solve(P.handle, b.data_ptr(), x.data_ptr(), 1e-10, 100, 0, infos, None)
    torch.cuda.synchronize()
    assert st == K.ERR_NOT_SYMMETRIC and infos[0].status == K.ERR_NOT_SYMMETRIC
    assert b"not symmetric" in K._lib.sla_last_error()
    assert bool(torch.all(x == 123.0))  # untouched
    with pytest.raises(K.SlaError):
        K.sla_cg_adjoint(P, t(v), b, b, 1e-10, 100)
    with pytest.raises(K.SlaError) as e:
        K.sla_solve_list([P], [t(v)], [b], 1e-10, 100)
    assert e.value.status == K.ERR_NOT_SYMMETRIC and "system 0" in str(e.value)
    # BiCGStab takes general matrices
    xb, ib = K.sla_bicgstab_solve(P, t(v), b, 1e-12, 1000)
    torch.cuda.synchronize()
    xo, io = oracle.bicgstab(oracle.CSR(n, rp.astype(np.int64), c, v), W.uniform_rhs(n, 4),
                             1e-12, 1000)
    assert ib[0].converged and rel(xb.cpu().numpy(), xo) <= TOL_X
    # the oracle's adjoint flags the same input
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    _, _, ai = oracle.adjoint(A, xo, W.uniform_rhs(n, 4), 1e-10, 100)
    assert ai.status == oracle.ERR_NOT_SYMMETRIC


def test_adjoint_refuses_values_that_are_not_symmetric():
    import torch
    import krylov_solvers_adjoint_amd as K
    N = 50
    n = N * N
    rp, c, v = W.poisson_csr(N)
    rng = np.random.default_rng(5)
    vn = v.copy()
    off = np.flatnonzero(vn != 4.0)
    k = int(off[rng.integers(0, off.shape[0])])
    vn[k] = -1.25  # a_ij changed, a_ji not
    A = oracle.CSR(n, rp.astype(np.int64), c, vn)
    b = W.uniform_rhs(n, 6)
    g = W.normal_rhs(n, 7)
    P = K.sla_csr_create_from_csr(t(rp), t(c))
    # the forward solve does not check the values
    x, info = K.sla_cg_solve(P, t(vn), t(b), 1e-10, 5000)
    gb, gv, ai = K.sla_cg_adjoint(P, t(vn), x, t(g), 1e-10, 5000, check=False)
    torch.cuda.synchronize()
    assert ai.status == K.ERR_NOT_SYMMETRIC and ai.iterations == 0
    assert b"values are not symmetric" in K._lib.sla_last_error()
    xo, _ = oracle.cg(A, b, 1e-10, 5000)
    _, _, aio = oracle.adjoint(A, xo, g, 1e-10, 5000)
    assert aio.status == oracle.ERR_NOT_SYMMETRIC
    # symmetric values on the same handle: accepted, against the oracle
    x, _ = K.sla_cg_solve(P, t(v), t(b), 1e-10, 5000)
    gb, gv, ai = K.sla_cg_adjoint(P, t(v), x, t(g), 1e-10, 5000)
    torch.cuda.synchronize()
    Ao = oracle.CSR(n, rp.astype(np.int64), c, v)
    xo, _ = oracle.cg(Ao, b, 1e-10, 5000)
    gbo, _, aio = oracle.adjoint(Ao, xo, g, 1e-10, 5000)
    assert aio.status == oracle.OK and rel(gb.cpu().numpy(), gbo) <= TOL_X
    # a batch with one bad system is refused as a whole; the reordered handle too
    vb = np.stack([v, vn, v])
    bb = np.stack([b, b, b])
    xb, _ = K.sla_cg_solve_batched(P, t(vb), t(bb), 1e-10, 5000)
    _, _, bi = K.sla_cg_adjoint_batched(P, t(vb), xb, t(np.stack([g, g, g])), 1e-10, 5000,
                                        check=False)
    assert all(i.status == K.ERR_NOT_SYMMETRIC for i in bi)
    P.reorder()
    with pytest.raises(K.SlaError) as e:
        K.sla_cg_adjoint(P, t(vn), x, t(g), 1e-10, 5000)
    assert e.value.status == K.ERR_NOT_SYMMETRIC
    torch.cuda.synchronize()
