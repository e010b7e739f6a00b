"""CPU reference oracle for the CSR CG solve and its adjoint (ctypes shim).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``krylov_solvers_adjoint_amd``) never imports, links or calls it, and
the two share no code: both only consume the seeded inputs from
``workloads/``.

The arithmetic lives in ``oracle.c`` (plain C, fp64, ``-ffp-contract=off``);
this module only builds that file with gcc, marshals numpy arrays and
returns numpy arrays.  See ``oracle.c`` for the method's source (the
torch-sla explainer's technical summary: Methodology 1 and 2) and for the
readings taken where the pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK = 0
ERR_ARG = 1
ERR_CSR = 2
ERR_NOT_SPD = 5
ERR_NONFINITE = 6
ERR_NOT_SYMMETRIC = 7
ERR_BREAKDOWN = 8


_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
# Sanitizers: with SLA_ORACLE_SANITIZE=1 the oracle is built and loaded with
# AddressSanitizer and UndefinedBehaviorSanitizer (gcc; every finding aborts).
# The interpreter is not instrumented, so the process must preload the ASan
# runtime:  LD_PRELOAD=$(gcc -print-file-name=libasan.so)
#           ASAN_OPTIONS=detect_leaks=0 SLA_ORACLE_SANITIZE=1 python -m pytest ...
_SANITIZE = os.environ.get("SLA_ORACLE_SANITIZE", "") == "1"


def build(src: str = _SRC, out: str | None = None, sanitize: bool | None = None) -> str:
    """Compile the oracle with gcc (always recompiles); sanitize=True adds
    -fsanitize=address,undefined (default: the SLA_ORACLE_SANITIZE setting)."""
    san = _SANITIZE if sanitize is None else sanitize
    if out is None:
        out = _SAN_LIB if san else _LIB
    flags = (["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
              "-fno-sanitize-recover=all"] if san else ["-O2"])
    cmd = ["gcc", *flags, "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-shared", "-fPIC", "-std=c11", "-Wall", "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def _load(path: str | None = None):
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        lib_path = _SAN_LIB if _SANITIZE else _LIB
        if not os.path.exists(lib_path):
            build(out=lib_path, sanitize=_SANITIZE)
        _lib = _bind(ctypes.CDLL(lib_path))
    return _lib


class _Info(ctypes.Structure):
    _fields_ = [("iterations", ctypes.c_int64), ("rr", ctypes.c_double),
                ("bb", ctypes.c_double), ("converged", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_D = ctypes.c_double


def _bind(lib):
    lib.oracle_csr_from_coo.restype = _I64
    lib.oracle_csr_from_coo.argtypes = [_I64, _I64, _P, _P, _P, _P, _P]
    lib.oracle_values_from_coo.restype = None
    lib.oracle_values_from_coo.argtypes = [_I64, _I64, _P, _P, _P]
    lib.oracle_transpose.restype = None
    lib.oracle_transpose.argtypes = [_I64, _P, _P, _P, _P, _P, _P]
    lib.oracle_spmv.restype = None
    lib.oracle_spmv.argtypes = [_I64, _P, _P, _P, _P, _P]
    lib.oracle_dot.restype = _D
    lib.oracle_dot.argtypes = [_I64, _P, _P]
    lib.oracle_cg.restype = ctypes.c_int
    lib.oracle_cg.argtypes = [_I64, _P, _P, _P, _P, _P, _D, _I64, ctypes.c_int,
                              ctypes.POINTER(_Info), _P, _P, _P]
    lib.oracle_adjoint.restype = ctypes.c_int
    lib.oracle_adjoint.argtypes = [_I64, _P, _P, _P, _P, _P, _P, _P, _D, _I64,
                                   ctypes.POINTER(_Info)]
    lib.oracle_pattern_grad.restype = None
    lib.oracle_pattern_grad.argtypes = [_I64, _P, _P, _P, _P, _P]
    lib.oracle_pcg_jacobi.restype = ctypes.c_int
    lib.oracle_pcg_jacobi.argtypes = [_I64, _P, _P, _P, _P, _P, _D, _I64, ctypes.c_int,
                                      ctypes.POINTER(_Info), _P, _P, _P, _P]
    lib.oracle_adjoint_jacobi.restype = ctypes.c_int
    lib.oracle_adjoint_jacobi.argtypes = [_I64, _P, _P, _P, _P, _P, _P, _P, _D, _I64,
                                          ctypes.POINTER(_Info)]
    lib.oracle_matvec_grad.restype = None
    lib.oracle_matvec_grad.argtypes = [_I64, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_lanczos.restype = _I64
    lib.oracle_lanczos.argtypes = [_I64, _P, _P, _P, _P, _I64, _P, _P, _P]
    lib.oracle_eig_grad.restype = None
    lib.oracle_eig_grad.argtypes = [_I64, _P, _P, _P, _P]
    lib.oracle_bicgstab.restype = ctypes.c_int
    lib.oracle_bicgstab.argtypes = [_I64, _P, _P, _P, _P, _P, _D, _I64, ctypes.c_int,
                                    ctypes.POINTER(_Info), _P, _P, _P, _P]
    lib.oracle_adjoint_bicgstab.restype = ctypes.c_int
    lib.oracle_adjoint_bicgstab.argtypes = [_I64, _P, _P, _P, _P, _P, _P, _P, _D, _I64,
                                            ctypes.POINTER(_Info)]
    lib.oracle_set_threads.restype = None
    lib.oracle_bfs_order.argtypes = [_I64, _P, _P, _P]
    lib.oracle_bfs_order.restype = None
    lib.oracle_permute.argtypes = [_I64, _P, _P, _P, _P, _P, _P, _P, _P]
    lib.oracle_permute.restype = None
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_progress.restype = None
    lib.oracle_set_progress.argtypes = [_I64]
    lib.oracle_get_threads.restype = ctypes.c_int
    lib.oracle_get_threads.argtypes = []
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


@dataclass
class CGInfo:
    status: int
    iterations: int
    rr: float
    bb: float
    converged: bool

    @property
    def rel_residual(self) -> float:
        return float(np.sqrt(self.rr / self.bb)) if self.bb > 0 else 0.0


@dataclass
class CSR:
    """CSR matrix in the oracle's layout: int64 rowptr, int32 col, fp64 vals."""
    n: int
    rowptr: np.ndarray
    col: np.ndarray
    vals: np.ndarray

    @property
    def nnz(self) -> int:
        return int(self.rowptr[-1])

    def to_dense(self) -> np.ndarray:
        d = np.zeros((self.n, self.n))
        rows = np.repeat(np.arange(self.n), np.diff(self.rowptr))
        np.add.at(d, (rows, self.col.astype(np.int64)), self.vals)
        return d


def set_threads(t: int) -> None:
    _load().oracle_set_threads(int(t))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def set_progress(every: int) -> None:
    """Make cg() print one line to stderr every `every` iterations (0: off)."""
    _load().oracle_set_progress(int(every))


def host_threads() -> int:
    """Threads for the oracle: the process's CPU share (OMP_NUM_THREADS when
    the environment fixes it, else the CPUs this process may run on)."""
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    env = os.environ.get("OMP_NUM_THREADS", "").strip()
    if env.isdigit() and int(env) > 0:
        return min(int(env), avail)
    return avail


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ('unknown' if absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def csr_from_coo(n: int, row, col, lib=None):
    """(rowptr int64[n+1], col int32[nnz], perm int64[m]) of the merged pattern."""
    L = lib or _load()
    row = _c(row, np.int64)
    col = _c(col, np.int64)
    m = row.shape[0]
    rowptr = np.zeros(n + 1, np.int64)
    col_out = np.zeros(max(m, 1), np.int32)
    perm = np.zeros(max(m, 1), np.int64)
    nnz = L.oracle_csr_from_coo(n, m, _ptr(row), _ptr(col), _ptr(rowptr),
                                _ptr(col_out), _ptr(perm))
    if nnz < 0:
        raise ValueError("COO index out of range")
    return rowptr, col_out[:nnz].copy(), perm[:m].copy()


def values_from_coo(perm, nnz: int, coo_val, lib=None) -> np.ndarray:
    """Merged CSR values (one row per batch item if coo_val is 2-D)."""
    L = lib or _load()
    perm = _c(perm, np.int64)
    coo_val = np.asarray(coo_val, np.float64)
    if coo_val.ndim == 2:
        return np.stack([values_from_coo(perm, nnz, v, lib) for v in coo_val])
    coo_val = _c(coo_val, np.float64)
    vals = np.zeros(max(nnz, 1), np.float64)
    L.oracle_values_from_coo(perm.shape[0], nnz, _ptr(perm), _ptr(coo_val), _ptr(vals))
    return vals[:nnz].copy()


def transpose(A: CSR, lib=None) -> CSR:
    L = lib or _load()
    rp = _c(A.rowptr, np.int64)
    c = _c(A.col, np.int32)
    v = _c(A.vals, np.float64)
    rpt = np.zeros(A.n + 1, np.int64)
    ct = np.zeros(max(A.nnz, 1), np.int32)
    vt = np.zeros(max(A.nnz, 1), np.float64)
    L.oracle_transpose(A.n, _ptr(rp), _ptr(c), _ptr(v), _ptr(rpt), _ptr(ct), _ptr(vt))
    return CSR(A.n, rpt, ct[:A.nnz].copy(), vt[:A.nnz].copy())


def bfs_order(A: CSR, lib=None) -> np.ndarray:
    """Breadth-first (Cuthill-McKee level) order of the unknowns from a
    pseudo-peripheral node; order[t] = original index at position t."""
    L = lib or _load()
    order = np.zeros(max(A.n, 1), np.int64)
    L.oracle_bfs_order(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                       _ptr(order))
    return order[:A.n].copy()


def permute(A: CSR, order, lib=None):
    """(P A P^T, src): the matrix with unknown order[t] at position t, rows'
    columns ascending; src[s] = slot of A held by slot s."""
    L = lib or _load()
    o = _c(order, np.int64)
    rp = np.zeros(A.n + 1, np.int64)
    c = np.zeros(max(A.nnz, 1), np.int32)
    v = np.zeros(max(A.nnz, 1), np.float64)
    src = np.zeros(max(A.nnz, 1), np.int64)
    L.oracle_permute(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                     _ptr(_c(A.vals, np.float64)), _ptr(o), _ptr(rp), _ptr(c), _ptr(v),
                     _ptr(src))
    return CSR(A.n, rp, c[:A.nnz].copy(), v[:A.nnz].copy()), src[:A.nnz].copy()


def spmv(A: CSR, x, lib=None) -> np.ndarray:
    L = lib or _load()
    x = _c(x, np.float64)
    y = np.zeros(A.n, np.float64)
    L.oracle_spmv(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                  _ptr(_c(A.vals, np.float64)), _ptr(x), _ptr(y))
    return y


def dot(u, v, lib=None) -> float:
    L = lib or _load()
    u = _c(u, np.float64)
    v = _c(v, np.float64)
    return float(L.oracle_dot(u.shape[0], _ptr(u), _ptr(v)))


def cg(A: CSR, b, tol: float, maxit: int, x0=None, history: bool = False, lib=None):
    """x, CGInfo[, (alpha, beta, rr) history arrays]."""
    L = lib or _load()
    b = _c(b, np.float64)
    x = _c(x0, np.float64).copy() if x0 is not None else np.zeros(A.n, np.float64)
    info = _Info()
    ha = hb = hr = None
    if history:
        ha = np.zeros(max(maxit, 1))
        hb = np.zeros(max(maxit, 1))
        hr = np.zeros(max(maxit, 1))
    st = L.oracle_cg(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                     _ptr(_c(A.vals, np.float64)), _ptr(b), _ptr(x), float(tol),
                     int(maxit), 1 if x0 is not None else 0, ctypes.byref(info),
                     _ptr(ha), _ptr(hb), _ptr(hr))
    out = CGInfo(int(st), int(info.iterations), float(info.rr), float(info.bb),
                 bool(info.converged))
    if history:
        k = out.iterations
        return x, out, (ha[:k].copy(), hb[:k].copy(), hr[:k].copy())
    return x, out


def adjoint(A: CSR, x, g, tol: float, maxit: int, lib=None):
    """(grad_b = lambda, grad_vals in CSR slot order, CGInfo)."""
    L = lib or _load()
    x = _c(x, np.float64)
    g = _c(g, np.float64)
    gb = np.zeros(A.n, np.float64)
    gv = np.zeros(max(A.nnz, 1), np.float64)
    info = _Info()
    st = L.oracle_adjoint(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                          _ptr(_c(A.vals, np.float64)), _ptr(x), _ptr(g), _ptr(gb),
                          _ptr(gv), float(tol), int(maxit), ctypes.byref(info))
    return gb, gv[:A.nnz].copy(), CGInfo(int(st), int(info.iterations), float(info.rr),
                                         float(info.bb), bool(info.converged))


def bicgstab(A: CSR, b, tol: float, maxit: int, x0=None, history: bool = False, lib=None):
    """BiCGStab for a general A: x, CGInfo[, (rho, alpha, omega, rr) history]."""
    L = lib or _load()
    b = _c(b, np.float64)
    x = _c(x0, np.float64).copy() if x0 is not None else np.zeros(A.n, np.float64)
    info = _Info()
    hs = [None] * 4
    if history:
        hs = [np.zeros(max(maxit, 1)) for _ in range(4)]
    st = L.oracle_bicgstab(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                           _ptr(_c(A.vals, np.float64)), _ptr(b), _ptr(x), float(tol),
                           int(maxit), 1 if x0 is not None else 0, ctypes.byref(info),
                           *[_ptr(h) for h in hs])
    out = CGInfo(int(st), int(info.iterations), float(info.rr), float(info.bb),
                 bool(info.converged))
    if history:
        k = out.iterations
        return x, out, tuple(h[:k].copy() for h in hs)
    return x, out


def adjoint_bicgstab(A: CSR, x, g, tol: float, maxit: int, lib=None):
    """(grad_b = lambda solving A^T lambda = g by BiCGStab, grad_vals, CGInfo)."""
    L = lib or _load()
    x = _c(x, np.float64)
    g = _c(g, np.float64)
    gb = np.zeros(A.n, np.float64)
    gv = np.zeros(max(A.nnz, 1), np.float64)
    info = _Info()
    st = L.oracle_adjoint_bicgstab(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                                   _ptr(_c(A.vals, np.float64)), _ptr(x), _ptr(g), _ptr(gb),
                                   _ptr(gv), float(tol), int(maxit), ctypes.byref(info))
    return gb, gv[:A.nnz].copy(), CGInfo(int(st), int(info.iterations), float(info.rr),
                                         float(info.bb), bool(info.converged))


def pcg_jacobi(A: CSR, b, tol: float, maxit: int, x0=None, history: bool = False, lib=None):
    """Jacobi-preconditioned CG (M = diag(A)): x, CGInfo[, (alpha, beta, rr,
    rz) history arrays]."""
    L = lib or _load()
    b = _c(b, np.float64)
    x = _c(x0, np.float64).copy() if x0 is not None else np.zeros(A.n, np.float64)
    info = _Info()
    ha = hb = hr = hz = None
    if history:
        ha, hb, hr, hz = (np.zeros(max(maxit, 1)) for _ in range(4))
    st = L.oracle_pcg_jacobi(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                             _ptr(_c(A.vals, np.float64)), _ptr(b), _ptr(x), float(tol),
                             int(maxit), 1 if x0 is not None else 0, ctypes.byref(info),
                             _ptr(ha), _ptr(hb), _ptr(hr), _ptr(hz))
    out = CGInfo(int(st), int(info.iterations), float(info.rr), float(info.bb),
                 bool(info.converged))
    if history:
        k = out.iterations
        return x, out, (ha[:k].copy(), hb[:k].copy(), hr[:k].copy(), hz[:k].copy())
    return x, out


def adjoint_jacobi(A: CSR, x, g, tol: float, maxit: int, lib=None):
    """The adjoint of a Jacobi-PCG solve: (grad_b = lambda, grad_vals, CGInfo)."""
    L = lib or _load()
    x = _c(x, np.float64)
    g = _c(g, np.float64)
    gb = np.zeros(A.n, np.float64)
    gv = np.zeros(max(A.nnz, 1), np.float64)
    info = _Info()
    st = L.oracle_adjoint_jacobi(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                                 _ptr(_c(A.vals, np.float64)), _ptr(x), _ptr(g), _ptr(gb),
                                 _ptr(gv), float(tol), int(maxit), ctypes.byref(info))
    return gb, gv[:A.nnz].copy(), CGInfo(int(st), int(info.iterations), float(info.rr),
                                         float(info.bb), bool(info.converged))


def matvec_grad(A: CSR, x, g, lib=None):
    """Backward of y = A x for g = dL/dy: (grad_x = A^T g, grad_vals = g_i x_j
    on the stored slots)."""
    L = lib or _load()
    x = _c(x, np.float64)
    g = _c(g, np.float64)
    gx = np.zeros(A.n, np.float64)
    gv = np.zeros(max(A.nnz, 1), np.float64)
    L.oracle_matvec_grad(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                         _ptr(_c(A.vals, np.float64)), _ptr(x), _ptr(g), _ptr(gx), _ptr(gv))
    return gx, gv[:A.nnz].copy()


def lanczos(A: CSR, v0, m: int, lib=None):
    """m Lanczos steps with full reorthogonalisation (classical Gram-Schmidt
    twice) from v0: (alpha[steps], beta[steps], V[steps+1, n])."""
    L = lib or _load()
    v0 = _c(v0, np.float64)
    alpha = np.zeros(max(m, 1))
    beta = np.zeros(max(m, 1))
    V = np.zeros((m + 1, A.n))
    steps = int(L.oracle_lanczos(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                                 _ptr(_c(A.vals, np.float64)), _ptr(v0), int(m), _ptr(alpha),
                                 _ptr(beta), _ptr(V)))
    return alpha[:steps].copy(), beta[:steps].copy(), V[:steps + 1].copy()


def eigsh(A: CSR, k: int, which: str, v0, m: int, lib=None):
    """The .eigsh: k Ritz pairs of the m-step Lanczos process, the largest
    (which="LA") or the smallest ("SA") algebraic ones, ascending.  The
    tridiagonal eigenproblem is solved by a library routine (LAPACK stevr via
    scipy).  Returns (theta[k], X[k, n] unit Ritz vectors, residual
    estimates |beta_m y_m|[k])."""
    from scipy.linalg import eigh_tridiagonal
    alpha, beta, V = lanczos(A, v0, m, lib=lib)
    steps = alpha.shape[0]
    theta, Y = eigh_tridiagonal(alpha, beta[:steps - 1])
    sel = np.arange(steps - k, steps) if which == "LA" else np.arange(k)
    X = (V[:steps].T @ Y[:, sel]).T
    res = np.abs(beta[steps - 1] * Y[steps - 1, sel])
    return theta[sel], X, res


def eig_grad(A: CSR, v, lib=None) -> np.ndarray:
    """d lambda / d vals[k] = v_i v_j on every stored slot (Hellmann-Feynman)."""
    L = lib or _load()
    v = _c(v, np.float64)
    gv = np.zeros(max(A.nnz, 1), np.float64)
    L.oracle_eig_grad(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)), _ptr(v),
                      _ptr(gv))
    return gv[:A.nnz].copy()


def pattern_grad(A: CSR, lam, x, lib=None) -> np.ndarray:
    L = lib or _load()
    lam = _c(lam, np.float64)
    x = _c(x, np.float64)
    gv = np.zeros(max(A.nnz, 1), np.float64)
    L.oracle_pattern_grad(A.n, _ptr(_c(A.rowptr, np.int64)), _ptr(_c(A.col, np.int32)),
                          _ptr(lam), _ptr(x), _ptr(gv))
    return gv[:A.nnz].copy()


def cg_batched(rowptr, col, vals_b, b_b, tol: float, maxit: int, lib=None):
    """Shared-pattern batch: the single solve applied to each system in turn."""
    xs, infos = [], []
    for s in range(vals_b.shape[0]):
        A = CSR(len(rowptr) - 1, rowptr, col, vals_b[s])
        x, info = cg(A, b_b[s], tol, maxit, lib=lib)
        xs.append(x)
        infos.append(info)
    return np.stack(xs), infos


def adjoint_batched(rowptr, col, vals_b, x_b, g_b, tol: float, maxit: int, lib=None):
    gbs, gvs, infos = [], [], []
    for s in range(vals_b.shape[0]):
        A = CSR(len(rowptr) - 1, rowptr, col, vals_b[s])
        gb, gv, info = adjoint(A, x_b[s], g_b[s], tol, maxit, lib=lib)
        gbs.append(gb)
        gvs.append(gv)
        infos.append(info)
    return np.stack(gbs), np.stack(gvs), infos
