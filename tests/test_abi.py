"""The C-ABI library loads and exports every symbol include/sla.h declares;
argument errors are reported before anything touches a GPU (runs on CPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sla.h")
LIB = os.path.join(ROOT, "krylov_solvers_adjoint_amd", "libsla.so")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:sla_status|const char\*)\s+(sla_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared()
    for required in ("sla_csr_create", "sla_spmv", "sla_cg_solve", "sla_cg_adjoint",
                     "sla_cg_solve_batched", "sla_cg_adjoint_batched"):
        assert required in names


def test_library_exports_every_declared_symbol():
    assert os.path.exists(LIB), "build the library first (__graft_entry__.build())"
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_covers_every_symbol():
    import krylov_solvers_adjoint_amd as K
    assert sorted(K.EXPORTS) == declared()


def test_argument_errors_need_no_gpu():
    import krylov_solvers_adjoint_amd as K
    lib = K._lib
    h = ctypes.c_void_p()
    # NULL handle / NULL out / bad sizes are rejected before any HIP call
    assert lib.sla_csr_create(10, 0, 4, None, None, 4, None, None) == K.ERR_ARG
    assert b"out is NULL" in lib.sla_last_error()
    assert lib.sla_csr_create(0, 0, 4, None, None, 4, None, ctypes.byref(h)) == K.ERR_ARG
    assert lib.sla_csr_create(10, 5, 3, None, None, 4, None, ctypes.byref(h)) == K.ERR_ARG
    assert lib.sla_csr_create(10, 5, 4, None, None, 4, None, ctypes.byref(h)) == K.ERR_ARG
    assert lib.sla_csr_create_from_csr(10, 1 << 31, 4, 1, 1, None, ctypes.byref(h)) == K.ERR_ARG
    assert lib.sla_spmv(None, None, None, None) == K.ERR_ARG
    assert lib.sla_cg_solve(None, None, None, 1e-8, 10, 0, None, None) == K.ERR_ARG
    assert lib.sla_cg_adjoint(None, None, None, None, None, 1e-8, 10, 0, None, None) == K.ERR_ARG
    assert lib.sla_csr_set_values(None, None, 1) == K.ERR_ARG
    assert lib.sla_csr_set_workgroups_per_cu(None, 1) == K.ERR_ARG
    assert lib.sla_spmv_transpose(None, None, None, None) == K.ERR_ARG
    assert lib.sla_matvec_grad(None, None, None, None, None, None) == K.ERR_ARG
    assert lib.sla_eigsh(None, 1, 1, 4, None, None, None, None, None, None) == K.ERR_ARG
    assert lib.sla_eig_grad(None, 1, None, None, None, None) == K.ERR_ARG
    assert lib.sla_status_string(K.ERR_KRYLOV) == b"SLA_ERR_KRYLOV"
    assert lib.sla_bicgstab_solve(None, None, None, 1e-8, 10, 0, None, None) == K.ERR_ARG
    assert lib.sla_bicgstab_adjoint(None, None, None, None, None, 1e-8, 10, 0, None,
                                    None) == K.ERR_ARG
    assert lib.sla_bicgstab_history(None, 0, None, None, None, None, 0, None) == K.ERR_ARG
    assert lib.sla_status_string(K.ERR_BREAKDOWN) == b"SLA_ERR_BREAKDOWN"
    assert lib.sla_solve_list(0, None, None, None, 1e-8, 10, 0, 0, None, None) == K.ERR_ARG
    assert lib.sla_adjoint_list(0, None, None, None, None, None, 1e-8, 10, 0, 0, None,
                                None) == K.ERR_ARG
    assert lib.sla_csr_set_graph_block(None, 32) == K.ERR_ARG
    assert lib.sla_csr_reorder(None, K.ORDER_BFS, None) == K.ERR_ARG
    assert lib.sla_csr_ordering(None, None, None) == K.ERR_ARG
    assert lib.sla_csr_set_one_group(None, K.ONE_GROUP_AUTO) == K.ERR_ARG
    assert lib.sla_status_string(K.ERR_NOT_SPD) == b"SLA_ERR_NOT_SPD"
    assert lib.sla_status_string(K.ERR_NOT_SYMMETRIC) == b"SLA_ERR_NOT_SYMMETRIC"
    # the borrowed views and the owned values copy
    rp, c, v, pm = (ctypes.c_void_p() for _ in range(4))
    assert lib.sla_csr_arrays(None, ctypes.byref(rp), ctypes.byref(c), ctypes.byref(v),
                              ctypes.byref(pm)) == K.ERR_ARG
    assert b"NULL handle" in lib.sla_last_error()
    assert lib.sla_csr_load_values(None, None, 1, K.VALUES_CSR, None) == K.ERR_ARG
    assert lib.sla_csr_destroy(None) == K.OK
