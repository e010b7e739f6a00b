"""Python face of ``libsla.so``: a sparse CG solve with an O(1)-graph adjoint.

Every function here only marshals arguments (torch CUDA tensors -> device
pointers, the current HIP stream) and calls the C ABI declared in
``include/sla.h`` under the same name; every step of the computation runs in
the library's HIP kernels.  PyTorch provides device memory, streams and the
autograd node.  The library must be built (``python
krylov_solvers_adjoint_amd/_build.py``); importing this package without it
raises ImportError: there is no fallback.

Source of the method: the torch-sla explainer (gist.science, arXiv
2601.13994), technical summary -- Methodology 1 (sparse tensors with
.solve/.matvec, shared-pattern batches) and Methodology 2 (linear-system
adjoint: A^T lambda = dL/dx, grad_b = lambda, grad_A = -lambda_i x_j on the
pattern; one graph node, O(n + nnz) memory).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch  # loads torch's HIP runtime first: the library then shares it

__all__ = [
    "SlaError", "CGInfo", "CSRPattern", "SparseTensor", "solve",
    "sla_csr_create", "sla_csr_create_from_csr", "sla_csr_values_from_coo",
    "sla_csr_grad_to_coo", "sla_spmv", "sla_cg_solve", "sla_cg_adjoint",
    "sla_cg_solve_batched", "sla_cg_adjoint_batched", "sla_pattern_grad",
    "sla_spmv_transpose", "sla_matvec_grad", "sla_eigsh", "sla_eig_grad", "EigInfo",
    "sla_bicgstab_solve", "sla_bicgstab_adjoint", "sla_bicgstab_history",
    "sla_solve_list", "sla_adjoint_list", "SparseTensorList",
    "sla_csr_reorder", "sla_csr_ordering", "sla_csr_load_values", "sla_csr_arrays",
    "sla_memory_usage",
    "LIB_PATH", "EXPORTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsla.so")

(OK, ERR_ARG, ERR_CSR, ERR_OOM, ERR_DEVICE, ERR_NOT_SPD, ERR_NONFINITE, ERR_KRYLOV,
 ERR_BREAKDOWN, ERR_NOT_SYMMETRIC) = range(10)
VALUES_CSR, VALUES_COO = 0, 1
EIG_SMALLEST, EIG_LARGEST = 0, 1
METHOD_CG, METHOD_BICGSTAB = 0, 1
I32, I64 = 4, 8
FLAG_X0, FLAG_HISTORY, FLAG_JACOBI = 1, 2, 4
ORDER_NONE, ORDER_BFS = 0, 1
ONE_GROUP_AUTO, ONE_GROUP_OFF = 0, 1

EXPORTS = [
    "sla_csr_create", "sla_csr_create_from_csr", "sla_csr_destroy", "sla_csr_get_info",
    "sla_csr_pattern", "sla_csr_copy_pattern", "sla_csr_values_from_coo",
    "sla_csr_grad_to_coo", "sla_csr_set_values", "sla_spmv", "sla_cg_solve",
    "sla_cg_adjoint", "sla_cg_solve_batched", "sla_cg_adjoint_batched", "sla_pattern_grad",
    "sla_cg_history", "sla_profile_iteration_kernels", "sla_csr_set_spmv_variant",
    "sla_csr_set_graph_block",
    "sla_csr_set_workgroups_per_cu", "sla_spmv_transpose", "sla_matvec_grad",
    "sla_eigsh", "sla_eig_grad", "sla_profile_lanczos_kernels",
    "sla_bicgstab_solve", "sla_bicgstab_adjoint", "sla_bicgstab_history",
    "sla_solve_list", "sla_adjoint_list", "sla_csr_reorder", "sla_csr_ordering",
    "sla_csr_set_one_group", "sla_resident_loop_ms", "sla_csr_load_values", "sla_csr_arrays",
    "sla_memory_usage",
    "sla_cg_solve_noalloc", "sla_last_error", "sla_status_string",
]

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python krylov_solvers_adjoint_amd/_build.py` "
        "(there is no CPU fallback)")


class _Info(ctypes.Structure):
    _fields_ = [("iterations", ctypes.c_int64), ("rel_residual", ctypes.c_double),
                ("converged", ctypes.c_int32), ("status", ctypes.c_int32)]


class _EigInfo(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("status", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_D = ctypes.c_double
_U32 = ctypes.c_uint32
_S = ctypes.c_int


def _bind(lib):
    sig = {
        "sla_csr_create": [_I64, _I64, _S, _P, _P, _S, _P, ctypes.POINTER(_P)],
        "sla_csr_create_from_csr": [_I64, _I64, _S, _P, _P, _P, ctypes.POINTER(_P)],
        "sla_csr_destroy": [_P],
        "sla_csr_get_info": [_P, ctypes.POINTER(_I64), ctypes.POINTER(_I64),
                             ctypes.POINTER(_I64), ctypes.POINTER(_S)],
        "sla_csr_pattern": [_P, ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P)],
        "sla_csr_copy_pattern": [_P, _P, _P, _P, _P],
        "sla_csr_values_from_coo": [_P, _P, _P, _I64, _P],
        "sla_csr_grad_to_coo": [_P, _P, _P, _I64, _P],
        "sla_csr_set_values": [_P, _P, _I64],
        "sla_spmv": [_P, _P, _P, _P],
        "sla_cg_solve": [_P, _P, _P, _D, _I64, _U32, _P, _P],
        "sla_cg_adjoint": [_P, _P, _P, _P, _P, _D, _I64, _U32, _P, _P],
        "sla_cg_solve_batched": [_P, _P, _P, _D, _I64, _U32, _P, _P],
        "sla_cg_adjoint_batched": [_P, _P, _P, _P, _P, _D, _I64, _U32, _P, _P],
        "sla_pattern_grad": [_P, _P, _P, _P, _P],
        "sla_cg_history": [_P, _I64, _P, _P, _P, _I64, ctypes.POINTER(_I64)],
        "sla_profile_iteration_kernels": [_P, _P, _P, _I64, _P, _P],
        "sla_csr_set_graph_block": [_P, _I64],
        "sla_csr_set_workgroups_per_cu": [_P, _S],
        "sla_spmv_transpose": [_P, _P, _P, _P],
        "sla_matvec_grad": [_P, _P, _P, _P, _P, _P],
        "sla_eigsh": [_P, _I64, _S, _I64, _P, _P, _P, _P, _P, _P],
        "sla_eig_grad": [_P, _I64, _P, _P, _P, _P],
        "sla_profile_lanczos_kernels": [_P, _I64, _I64, _P, _P],
        "sla_bicgstab_solve": [_P, _P, _P, _D, _I64, _U32, _P, _P],
        "sla_bicgstab_adjoint": [_P, _P, _P, _P, _P, _D, _I64, _U32, _P, _P],
        "sla_bicgstab_history": [_P, _I64, _P, _P, _P, _P, _I64, ctypes.POINTER(_I64)],
        "sla_solve_list": [_I64, _P, _P, _P, _D, _I64, _U32, _S, _P, _P],
        "sla_adjoint_list": [_I64, _P, _P, _P, _P, _P, _D, _I64, _U32, _S, _P, _P],
        "sla_csr_set_spmv_variant": [_P, _S, ctypes.POINTER(_S)],
        "sla_csr_reorder": [_P, _S, _P],
        "sla_csr_set_one_group": [_P, _S],
        "sla_resident_loop_ms": [_P, ctypes.POINTER(_D)],
        "sla_csr_ordering": [_P, _P, _P],
        "sla_csr_load_values": [_P, _P, _I64, _S, _P],
        "sla_csr_arrays": [_P, ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P),
                           ctypes.POINTER(_P)],
        "sla_memory_usage": [ctypes.POINTER(_I64), ctypes.POINTER(_I64), _S],
        "sla_cg_solve_noalloc": [_P, _P, _P, _D, _I64, _U32, _P, _P],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = _S
    lib.sla_last_error.argtypes = []
    lib.sla_last_error.restype = ctypes.c_char_p
    lib.sla_status_string.argtypes = [_S]
    lib.sla_status_string.restype = ctypes.c_char_p
    return lib


_lib = _bind(ctypes.CDLL(LIB_PATH))


class SlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        name = _lib.sla_status_string(status).decode()
        super().__init__(f"{name}: {message}")


def _check(status: int):
    if status != OK:
        raise SlaError(status, _lib.sla_last_error().decode(errors="replace"))


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dev(t: torch.Tensor, dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor (the library has no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


def _shape(t: torch.Tensor, shape: tuple, name: str):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _vec_shape(A: "CSRPattern", batch: int, like: torch.Tensor) -> tuple:
    return (A.n,) if like.dim() == 1 and batch == 1 else (batch, A.n)


def _idx_code(dtype) -> int:
    if dtype == torch.int32:
        return I32
    if dtype == torch.int64:
        return I64
    raise TypeError(f"index dtype must be int32 or int64, got {dtype}")


@dataclass
class CGInfo:
    iterations: int
    rel_residual: float
    converged: bool
    status: int


def _infos(arr) -> list:
    return [CGInfo(int(i.iterations), float(i.rel_residual), bool(i.converged), int(i.status))
            for i in arr]


# ---------------------------------------------------------------------------
# The pattern handle
# ---------------------------------------------------------------------------
class CSRPattern:
    """Owner of an ``sla_csr`` handle: the sparsity pattern in HBM (int32 or
    int64 row pointers, int32 columns) and the solver workspace."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)
        n, nnz, m = _I64(), _I64(), _I64()
        w = _S()
        _check(_lib.sla_csr_get_info(self._h, ctypes.byref(n), ctypes.byref(nnz),
                                     ctypes.byref(m), ctypes.byref(w)))
        self.n, self.nnz, self.nnz_coo = n.value, nnz.value, m.value
        self.rowptr_dtype = torch.int32 if w.value == I32 else torch.int64
        self._bound = None
        self._variant = 0
        self._reordered = False

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h is not None and self._h.value:
            _lib.sla_csr_destroy(self._h)
        self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def pattern(self):
        """(rowptr, col, perm) as new device tensors (perm None if built from CSR)."""
        dev = torch.device("cuda", torch.cuda.current_device())
        rowptr = torch.empty(self.n + 1, dtype=self.rowptr_dtype, device=dev)
        col = torch.empty(max(self.nnz, 0), dtype=torch.int32, device=dev)
        perm = (torch.empty(self.nnz_coo, dtype=torch.int64, device=dev)
                if self.nnz_coo > 0 else None)
        _check(_lib.sla_csr_copy_pattern(self._h, rowptr.data_ptr(), col.data_ptr(),
                                         perm.data_ptr() if perm is not None else None,
                                         _stream()))
        return rowptr, col, perm

    def bind(self, values: torch.Tensor) -> int:
        """Bind values [nnz] or [batch, nnz] (float64, CSR slot order)."""
        if values.dim() not in (1, 2):
            raise ValueError("values must be [nnz] or [batch, nnz]")
        batch = 1 if values.dim() == 1 else values.shape[0]
        if values.shape[-1] != self.nnz or batch < 1:
            raise ValueError(f"values has shape {tuple(values.shape)}, the pattern {self.nnz} slots")
        _check(_lib.sla_csr_set_values(self._h, _dev(values, torch.float64, "values"), batch))
        self._bound = values
        return batch

    def set_graph_block(self, iterations: int):
        _check(_lib.sla_csr_set_graph_block(self._h, int(iterations)))

    def set_workgroups_per_cu(self, workgroups: int):
        _check(_lib.sla_csr_set_workgroups_per_cu(self._h, int(workgroups)))

    def set_one_group(self, mode: str = "auto"):
        """"auto": systems of up to 2048 unknowns (a banded pattern, or
        64-row tiles of at most 336 stored entries) run the CG loop in one
        workgroup per system;
        "off": always the two-kernel loop."""
        _check(_lib.sla_csr_set_one_group(self._h, {"auto": ONE_GROUP_AUTO,
                                                    "off": ONE_GROUP_OFF}[mode]))

    def _kernels(self) -> int:
        b = _S()
        _check(_lib.sla_csr_set_spmv_variant(self._h, self._variant, ctypes.byref(b)))
        return b.value

    def set_spmv_variant(self, variant) -> bool:
        """"auto" (default), "csr", "banded", "split" or "lines" (see
        sla_csr_set_spmv_variant); returns whether mask-byte kernels (banded
        or line walk) are now in use."""
        self._variant = {"auto": 0, "csr": 1, "banded": 2, "split": 3, "lines": 4}[variant]
        return self._kernels() in (1, 3)

    @property
    def split(self) -> bool:
        """Whether the separate search-direction pass is in use."""
        return self._kernels() == 2

    @property
    def banded(self) -> bool:
        """Whether mask-byte kernels (banded or line walk) are in use."""
        return self._kernels() in (1, 3)

    @property
    def lines(self) -> bool:
        """Whether the CG iteration uses the line walk."""
        return self._kernels() == 3

    def reorder(self, ordering: str = "bfs", stream=None) -> "CSRPattern":
        """Renumber the unknowns for the CG calls (sla_csr_reorder): "bfs"
        (breadth-first order of the pattern's graph) or "none"."""
        sla_csr_reorder(self, ordering, stream)
        return self

    @property
    def reordered(self) -> bool:
        return self._reordered

    def history(self, system: int = 0, cap: int = 1 << 20):
        import numpy as np
        cnt = _I64()
        _check(_lib.sla_cg_history(self._h, system, None, None, None, 0, ctypes.byref(cnt)))
        k = min(cnt.value, cap)
        a, b, r = (np.zeros(max(k, 1)) for _ in range(3))
        _check(_lib.sla_cg_history(self._h, system, a.ctypes.data, b.ctypes.data,
                                   r.ctypes.data, k, ctypes.byref(cnt)))
        return a[:k], b[:k], r[:k]


# ---------------------------------------------------------------------------
# Same-named wrappers of the C ABI
# ---------------------------------------------------------------------------
def sla_csr_create(n: int, row: torch.Tensor, col: torch.Tensor,
                   rowptr_dtype=torch.int32, stream=None) -> CSRPattern:
    """COO coordinates (int32 or int64 device tensors) -> CSR pattern."""
    if row.shape != col.shape or row.dtype != col.dtype:
        raise ValueError("row and col must have the same shape and dtype")
    code = _idx_code(row.dtype)
    h = ctypes.c_void_p()
    m = row.numel()
    _check(_lib.sla_csr_create(int(n), m, code, _dev(row, row.dtype, "row") if m else None,
                               _dev(col, col.dtype, "col") if m else None,
                               _idx_code(rowptr_dtype), _stream(stream), ctypes.byref(h)))
    return CSRPattern(h.value)


def sla_csr_create_from_csr(rowptr: torch.Tensor, col: torch.Tensor, stream=None) -> CSRPattern:
    n = rowptr.numel() - 1
    h = ctypes.c_void_p()
    _check(_lib.sla_csr_create_from_csr(
        n, col.numel(), _idx_code(rowptr.dtype), _dev(rowptr, rowptr.dtype, "rowptr"),
        _dev(col, torch.int32, "col") if col.numel() else None, _stream(stream),
        ctypes.byref(h)))
    return CSRPattern(h.value)


def sla_csr_reorder(A: CSRPattern, ordering: str = "bfs", stream=None) -> None:
    """CG solves and adjoints on A run on P A P^T, P the breadth-first order
    of the pattern's graph ("bfs"), or on A as it is again ("none")."""
    code = {"none": ORDER_NONE, "bfs": ORDER_BFS}[ordering]
    _check(_lib.sla_csr_reorder(A.handle, code, _stream(stream)))
    A._reordered = code != ORDER_NONE


def sla_csr_ordering(A: CSRPattern, stream=None) -> torch.Tensor:
    """The ordering of a reordered handle: out[t] = original index of the
    unknown at position t (int32, on the device)."""
    out = torch.empty(A.n, dtype=torch.int32, device=torch.device("cuda", torch.cuda.current_device()))
    _check(_lib.sla_csr_ordering(A.handle, out.data_ptr() if A.n else None, _stream(stream)))
    return out


def sla_csr_load_values(A: CSRPattern, values: torch.Tensor, order: str = "csr",
                        stream=None) -> int:
    """Copy values into an array the handle owns and bind it: [nnz] or
    [batch, nnz] in CSR slot order ("csr"), or [nnz_coo] / [batch, nnz_coo]
    in the COO triplet order the pattern was built from ("coo").  Returns
    the batch size.  The later calls of this module bind the values they are
    given, so this serves callers of the C ABI that keep the handle's own
    copy (sla_csr_arrays gives its address)."""
    code = {"csr": VALUES_CSR, "coo": VALUES_COO}[order]
    width = A.nnz if code == VALUES_CSR else A.nnz_coo
    if values.dim() not in (1, 2) or values.shape[-1] != width:
        raise ValueError(f"values has shape {tuple(values.shape)}; expected [..., {width}]")
    batch = 1 if values.dim() == 1 else values.shape[0]
    _check(_lib.sla_csr_load_values(A.handle, _dev(values, torch.float64, "values"), batch,
                                    code, _stream(stream)))
    A._bound = None
    return batch


def sla_csr_arrays(A: CSRPattern) -> dict:
    """Device addresses of the handle's arrays (borrowed views): rowptr, col,
    the bound values (0 if none) and perm (0 for a handle made from CSR)."""
    rp, c, v, pm = _P(), _P(), _P(), _P()
    _check(_lib.sla_csr_arrays(A.handle, ctypes.byref(rp), ctypes.byref(c), ctypes.byref(v),
                               ctypes.byref(pm)))
    return {"rowptr": rp.value or 0, "col": c.value or 0, "vals": v.value or 0,
            "perm": pm.value or 0}


def sla_memory_usage(reset_peak: bool = False) -> tuple:
    """(live, peak) device bytes the library holds on the current device."""
    live, peak = _I64(), _I64()
    _check(_lib.sla_memory_usage(ctypes.byref(live), ctypes.byref(peak), 1 if reset_peak else 0))
    return live.value, peak.value


def sla_csr_values_from_coo(A: CSRPattern, coo_val: torch.Tensor, stream=None) -> torch.Tensor:
    batch = 1 if coo_val.dim() == 1 else coo_val.shape[0]
    if A.nnz_coo == 0 and A.nnz > 0:
        raise ValueError("pattern was not built from COO")
    _shape(coo_val, (A.nnz_coo,) if coo_val.dim() == 1 else (batch, A.nnz_coo), "coo_val")
    out = torch.empty((batch, A.nnz) if coo_val.dim() == 2 else (A.nnz,),
                      dtype=torch.float64, device=coo_val.device)
    _check(_lib.sla_csr_values_from_coo(A.handle, _dev(coo_val, torch.float64, "coo_val"),
                                        out.data_ptr(), batch, _stream(stream)))
    return out


def sla_csr_grad_to_coo(A: CSRPattern, grad_vals: torch.Tensor, stream=None) -> torch.Tensor:
    batch = 1 if grad_vals.dim() == 1 else grad_vals.shape[0]
    _shape(grad_vals, (A.nnz,) if grad_vals.dim() == 1 else (batch, A.nnz), "grad_vals")
    out = torch.empty((batch, A.nnz_coo) if grad_vals.dim() == 2 else (A.nnz_coo,),
                      dtype=torch.float64, device=grad_vals.device)
    _check(_lib.sla_csr_grad_to_coo(A.handle, _dev(grad_vals, torch.float64, "grad_vals"),
                                    out.data_ptr(), batch, _stream(stream)))
    return out


def sla_spmv(A: CSRPattern, values: torch.Tensor, x: torch.Tensor, stream=None) -> torch.Tensor:
    batch = A.bind(values)
    _shape(x, _vec_shape(A, batch, x), "x")
    y = torch.empty_like(x)
    _check(_lib.sla_spmv(A.handle, _dev(x, torch.float64, "x"), y.data_ptr(), _stream(stream)))
    return y


def sla_spmv_transpose(A: CSRPattern, values: torch.Tensor, x: torch.Tensor,
                       stream=None) -> torch.Tensor:
    """y = A^T x (every system of the batch)."""
    batch = A.bind(values)
    _shape(x, _vec_shape(A, batch, x), "x")
    y = torch.empty_like(x)
    _check(_lib.sla_spmv_transpose(A.handle, _dev(x, torch.float64, "x"), y.data_ptr(),
                                   _stream(stream)))
    return y


def sla_matvec_grad(A: CSRPattern, values: torch.Tensor, x: torch.Tensor, grad_y: torch.Tensor,
                    want_x: bool = True, want_vals: bool = True, stream=None):
    """Backward of y = A x: (grad_x = A^T grad_y or None, grad_vals = grad_y_i x_j or None)."""
    batch = A.bind(values)
    _shape(grad_y, _vec_shape(A, batch, grad_y), "grad_y")
    _shape(x, _vec_shape(A, batch, grad_y), "x")
    gx = torch.empty_like(grad_y) if want_x else None
    gv = (torch.empty((batch, A.nnz) if grad_y.dim() == 2 else (A.nnz,), dtype=torch.float64,
                      device=grad_y.device) if want_vals else None)
    _check(_lib.sla_matvec_grad(A.handle, _dev(x, torch.float64, "x"),
                                _dev(grad_y, torch.float64, "grad_y"),
                                gx.data_ptr() if gx is not None else None,
                                gv.data_ptr() if gv is not None else None, _stream(stream)))
    return gx, gv


@dataclass
class EigInfo:
    steps: int
    status: int


_WHICH = {"SA": EIG_SMALLEST, "LA": EIG_LARGEST}


def sla_eigsh(A: CSRPattern, values: torch.Tensor, k: int, which: str, m: int,
              v0: torch.Tensor, stream=None, check: bool = True):
    """k extreme Ritz pairs by m Lanczos steps (full reorthogonalisation).

    which "LA" (largest) or "SA" (smallest); v0 [n] or [batch, n].  Returns
    (theta [.., k] ascending, X [.., k, n] unit vectors, resid [.., k], infos).
    """
    batch = A.bind(values)
    if which not in _WHICH:
        raise ValueError(f"which must be 'LA' or 'SA', not {which!r}")
    _shape(v0, _vec_shape(A, batch, v0), "v0")
    lead = (batch,) if v0.dim() == 2 else ()
    theta = torch.empty(lead + (k,), dtype=torch.float64, device=v0.device)
    X = torch.empty(lead + (k, A.n), dtype=torch.float64, device=v0.device)
    resid = torch.empty(lead + (k,), dtype=torch.float64, device=v0.device)
    infos = (_EigInfo * batch)()
    st = _lib.sla_eigsh(A.handle, int(k), _WHICH[which], int(m), _dev(v0, torch.float64, "v0"),
                        theta.data_ptr(), X.data_ptr(), resid.data_ptr(), infos,
                        _stream(stream))
    if check:
        _check(st)
    return theta, X, resid, [EigInfo(int(i.steps), int(i.status)) for i in infos]


def sla_eig_grad(A: CSRPattern, values: torch.Tensor, X: torch.Tensor, grad_theta: torch.Tensor,
                 stream=None) -> torch.Tensor:
    """grad_vals[slot (i, j)] = sum_t grad_theta[t] X[t, i] X[t, j] (Hellmann-Feynman)."""
    batch = A.bind(values)
    k = grad_theta.shape[-1]
    want = (batch, k, A.n) if grad_theta.dim() == 2 else (k, A.n)
    _shape(X, want, "X")
    _shape(grad_theta, want[:-1], "grad_theta")
    gv = torch.empty((batch, A.nnz) if grad_theta.dim() == 2 else (A.nnz,), dtype=torch.float64,
                     device=X.device)
    _check(_lib.sla_eig_grad(A.handle, int(k), _dev(X, torch.float64, "X"),
                             _dev(grad_theta, torch.float64, "grad_theta"), gv.data_ptr(),
                             _stream(stream)))
    return gv


def sla_profile_lanczos_kernels(A: CSRPattern, nvec: int, reps: int = 10, stream=None) -> dict:
    """Mean ms of the Gram-Schmidt dot and update passes over nvec basis
    vectors (after an sla_eigsh call on A with m >= nvec)."""
    import numpy as np
    out = np.zeros(2, np.float64)
    _check(_lib.sla_profile_lanczos_kernels(A.handle, int(nvec), int(reps), out.ctypes.data,
                                            _stream(stream)))
    return dict(zip(("dot", "update"), out.tolist()))


def _solve_call(fn, A, b, x, tol, maxit, flags, batch, stream, check):
    _shape(b, _vec_shape(A, batch, b), "b")
    _shape(x, _vec_shape(A, batch, b), "x")
    infos = (_Info * batch)()
    st = fn(A.handle, _dev(b, torch.float64, "b"), _dev(x, torch.float64, "x"), float(tol),
            int(maxit), int(flags), infos, _stream(stream))
    if check:
        _check(st)
    return st, _infos(infos)


def _flags(x0, history, jacobi):
    return ((FLAG_X0 if x0 is not None else 0) | (FLAG_HISTORY if history else 0) |
            (FLAG_JACOBI if jacobi else 0))


def sla_cg_solve(A: CSRPattern, values: torch.Tensor, b: torch.Tensor, tol: float, maxit: int,
                 x0: torch.Tensor | None = None, history: bool = False, stream=None,
                 check: bool = True, jacobi: bool = False):
    """x, CGInfo.  Raises SlaError on breakdown unless check=False.  jacobi:
    preconditioned with M = diag(A)."""
    batch = A.bind(values)
    if batch != 1:
        raise ValueError("sla_cg_solve takes one system; use sla_cg_solve_batched")
    x = x0.clone() if x0 is not None else torch.empty_like(b)
    flags = _flags(x0, history, jacobi)
    st, infos = _solve_call(_lib.sla_cg_solve, A, b, x, tol, maxit, flags, 1, stream, check)
    return x, infos[0]


def sla_cg_solve_noalloc(A: CSRPattern, values: torch.Tensor, b: torch.Tensor, x: torch.Tensor,
                         tol: float, maxit: int, x0: bool = False, stream=None,
                         check: bool = True):
    """CGInfo of sla_cg_solve_noalloc: the solve of sla_cg_solve writing into
    the caller's x (its start vector when x0), with the library's static
    scratch as workspace; nothing is allocated (x must be given)."""
    if A.bind(values) != 1:
        raise ValueError("sla_cg_solve_noalloc takes one system")
    st, infos = _solve_call(_lib.sla_cg_solve_noalloc, A, b, x, tol, maxit,
                            FLAG_X0 if x0 else 0, 1, stream, check)
    return infos[0]


def sla_cg_solve_batched(A: CSRPattern, values: torch.Tensor, b: torch.Tensor, tol: float,
                         maxit: int, x0: torch.Tensor | None = None, history: bool = False,
                         stream=None, check: bool = True, jacobi: bool = False):
    batch = A.bind(values)
    if b.shape[0] != batch:
        raise ValueError("b must be [batch, n]")
    x = x0.clone() if x0 is not None else torch.empty_like(b)
    flags = _flags(x0, history, jacobi)
    st, infos = _solve_call(_lib.sla_cg_solve_batched, A, b, x, tol, maxit, flags, batch,
                            stream, check)
    return x, infos


def sla_bicgstab_solve(A: CSRPattern, values: torch.Tensor, b: torch.Tensor, tol: float,
                       maxit: int, x0: torch.Tensor | None = None, history: bool = False,
                       stream=None, check: bool = True):
    """BiCGStab for a general A: (x, [CGInfo per system]).  b [n] or [batch, n]."""
    batch = A.bind(values)
    x = x0.clone() if x0 is not None else torch.empty_like(b)
    st, infos = _solve_call(_lib.sla_bicgstab_solve, A, b, x, tol, maxit,
                            _flags(x0, history, False), batch, stream, check)
    return x, infos


def sla_bicgstab_adjoint(A: CSRPattern, values: torch.Tensor, x: torch.Tensor,
                         grad_x: torch.Tensor, tol: float, maxit: int, want_vals: bool = True,
                         history: bool = False, stream=None, check: bool = True):
    """(grad_b = lambda solving A^T lambda = grad_x, grad_vals = -lambda_i x_j or None,
    [CGInfo per system])."""
    batch = A.bind(values)
    return _adjoint_call(_lib.sla_bicgstab_adjoint, A, x, grad_x, tol, maxit, want_vals,
                         _flags(None, history, False), batch, stream, check)


def sla_bicgstab_history(A: CSRPattern, system: int = 0, cap: int = 1 << 20):
    """(rho, alpha, omega, rr) per iteration of the last BiCGStab run with history."""
    import numpy as np
    cnt = _I64()
    _check(_lib.sla_bicgstab_history(A.handle, system, None, None, None, None, 0,
                                     ctypes.byref(cnt)))
    k = min(cnt.value, cap)
    out = [np.zeros(max(k, 1)) for _ in range(4)]
    _check(_lib.sla_bicgstab_history(A.handle, system, *[o.ctypes.data for o in out], k,
                                     ctypes.byref(cnt)))
    return tuple(o[:k] for o in out)


_METHODS = {"cg": METHOD_CG, "bicgstab": METHOD_BICGSTAB}


def _ptr_array(items):
    arr = (_P * len(items))()
    for i, it in enumerate(items):
        arr[i] = it
    return arr


def _list_prepare(patterns, values, method):
    if method not in _METHODS:
        raise ValueError(f"unknown method {method!r}")
    if not (len(patterns) == len(values)) or not patterns:
        raise ValueError("patterns and values must be non-empty lists of one length")
    if len({id(P) for P in patterns}) != len(patterns):
        raise ValueError("a pattern appears twice in the list (use a batched SparseTensor)")
    for P, v in zip(patterns, values):
        if v.dim() != 1 or P.bind(v) != 1:
            raise ValueError("each list item binds exactly one system ([nnz] values)")
    return _ptr_array([P.handle for P in patterns])


def sla_solve_list(patterns: list, values: list, bs: list, tol: float, maxit: int,
                   method: str = "cg", jacobi: bool = False, stream=None, check: bool = True):
    """Solve a list of systems with distinct patterns (SparseTensorList):
    ([x_i], [CGInfo_i]).  Every system runs exactly as its single solve."""
    handles = _list_prepare(patterns, values, method)
    xs = []
    for P, b in zip(patterns, bs):
        _shape(b, (P.n,), "b")
        _dev(b, torch.float64, "b")
        xs.append(torch.empty_like(b))
    infos = (_Info * len(patterns))()
    st = _lib.sla_solve_list(len(patterns), handles, _ptr_array([b.data_ptr() for b in bs]),
                             _ptr_array([x.data_ptr() for x in xs]), float(tol), int(maxit),
                             _flags(None, False, jacobi), _METHODS[method], infos,
                             _stream(stream))
    if check:
        _check(st)
    return xs, _infos(infos)


def sla_adjoint_list(patterns: list, values: list, xs: list, grad_xs: list, tol: float,
                     maxit: int, method: str = "cg", want_vals=True, jacobi: bool = False,
                     stream=None, check: bool = True):
    """Backward of sla_solve_list: ([grad_b_i], [grad_vals_i or None], [CGInfo_i]).
    want_vals: one bool for all systems or a list of bools."""
    handles = _list_prepare(patterns, values, method)
    count = len(patterns)
    wv = want_vals if isinstance(want_vals, (list, tuple)) else [want_vals] * count
    gbs, gvs = [], []
    for P, x, g, w in zip(patterns, xs, grad_xs, wv):
        _shape(g, (P.n,), "grad_x")
        _shape(x, (P.n,), "x")
        _dev(g, torch.float64, "grad_x")
        _dev(x, torch.float64, "x")
        gbs.append(torch.empty_like(g))
        gvs.append(torch.empty(P.nnz, dtype=torch.float64, device=g.device) if w else None)
    infos = (_Info * count)()
    st = _lib.sla_adjoint_list(count, handles, _ptr_array([x.data_ptr() for x in xs]),
                               _ptr_array([g.data_ptr() for g in grad_xs]),
                               _ptr_array([g.data_ptr() for g in gbs]),
                               _ptr_array([g.data_ptr() if g is not None else None for g in gvs]),
                               float(tol), int(maxit), _flags(None, False, jacobi),
                               _METHODS[method], infos, _stream(stream))
    if check:
        _check(st)
    return gbs, gvs, _infos(infos)


def _adjoint_call(fn, A, x, grad_x, tol, maxit, want_vals, flags, batch, stream, check):
    _shape(grad_x, _vec_shape(A, batch, grad_x), "grad_x")
    _shape(x, _vec_shape(A, batch, grad_x), "x")
    grad_b = torch.empty_like(grad_x)
    grad_vals = (torch.empty((batch, A.nnz) if grad_x.dim() == 2 else (A.nnz,),
                             dtype=torch.float64, device=grad_x.device) if want_vals else None)
    infos = (_Info * batch)()
    st = fn(A.handle, _dev(x, torch.float64, "x"), _dev(grad_x, torch.float64, "grad_x"),
            grad_b.data_ptr(), grad_vals.data_ptr() if grad_vals is not None else None,
            float(tol), int(maxit), int(flags), infos, _stream(stream))
    if check:
        _check(st)
    return grad_b, grad_vals, _infos(infos)


def sla_cg_adjoint(A: CSRPattern, values: torch.Tensor, x: torch.Tensor, grad_x: torch.Tensor,
                   tol: float, maxit: int, want_vals: bool = True, history: bool = False,
                   stream=None, check: bool = True, jacobi: bool = False):
    """(grad_b = lambda, grad_vals or None, CGInfo)."""
    if A.bind(values) != 1:
        raise ValueError("sla_cg_adjoint takes one system; use sla_cg_adjoint_batched")
    gb, gv, infos = _adjoint_call(_lib.sla_cg_adjoint, A, x, grad_x, tol, maxit, want_vals,
                                  _flags(None, history, jacobi), 1, stream, check)
    return gb, gv, infos[0]


def sla_cg_adjoint_batched(A: CSRPattern, values: torch.Tensor, x: torch.Tensor,
                           grad_x: torch.Tensor, tol: float, maxit: int,
                           want_vals: bool = True, stream=None, check: bool = True,
                           jacobi: bool = False):
    batch = A.bind(values)
    return _adjoint_call(_lib.sla_cg_adjoint_batched, A, x, grad_x, tol, maxit, want_vals,
                         _flags(None, False, jacobi), batch, stream, check)


def sla_pattern_grad(A: CSRPattern, values_shape_ref: torch.Tensor, lam: torch.Tensor,
                     x: torch.Tensor, stream=None) -> torch.Tensor:
    """grad_vals = -lambda_i x_j on every stored slot (batch from the values)."""
    batch = A.bind(values_shape_ref)
    _shape(lam, _vec_shape(A, batch, lam), "lambda")
    _shape(x, _vec_shape(A, batch, lam), "x")
    out = torch.empty((batch, A.nnz) if lam.dim() == 2 else (A.nnz,), dtype=torch.float64,
                      device=lam.device)
    _check(_lib.sla_pattern_grad(A.handle, _dev(lam, torch.float64, "lambda"),
                                 _dev(x, torch.float64, "x"), out.data_ptr(), _stream(stream)))
    return out


def sla_resident_loop_ms(A: CSRPattern) -> float:
    """Duration (ms) of the last resident grid CG loop launched on A (events
    around the launch); SlaError if none has run."""
    ms = _D()
    _check(_lib.sla_resident_loop_ms(A.handle, ctypes.byref(ms)))
    return ms.value


def sla_profile_iteration_kernels(A: CSRPattern, values: torch.Tensor, b: torch.Tensor,
                                  reps: int = 20, stream=None) -> dict:
    """Mean duration (ms) of each CG iteration kernel, timed on its own."""
    if A.bind(values) != 1:
        raise ValueError("one system only")
    _shape(b, (A.n,), "b")
    x = torch.empty_like(b)
    import numpy as np
    out = np.zeros(2)
    _check(_lib.sla_profile_iteration_kernels(A.handle, _dev(b, torch.float64, "b"),
                                              x.data_ptr(), int(reps), out.ctypes.data,
                                              _stream(stream)))
    return dict(zip(("spmv_step", "residual_step"), out.tolist()))


# ---------------------------------------------------------------------------
# Autograd: one graph node per solve, saved state (values, x) = O(n + nnz)
# ---------------------------------------------------------------------------
class _CGSolve(torch.autograd.Function):
    @staticmethod
    def forward(ctx, values, b, pattern, tol, maxit, jacobi=False):
        batched = b.dim() == 2
        if batched:
            x, infos = sla_cg_solve_batched(pattern, values, b.contiguous(), tol, maxit,
                                            jacobi=jacobi)
        else:
            x, info = sla_cg_solve(pattern, values, b.contiguous(), tol, maxit, jacobi=jacobi)
            infos = [info]
        ctx.pattern, ctx.tol, ctx.maxit, ctx.batched = pattern, tol, maxit, batched
        ctx.jacobi = jacobi
        ctx.infos = infos
        ctx.save_for_backward(values, x)
        return x

    @staticmethod
    def backward(ctx, grad_x):
        values, x = ctx.saved_tensors
        want_vals = ctx.needs_input_grad[0]
        g = grad_x.contiguous()
        if ctx.batched:
            gb, gv, _ = sla_cg_adjoint_batched(ctx.pattern, values, x, g, ctx.tol, ctx.maxit,
                                               want_vals, jacobi=ctx.jacobi)
        else:
            gb, gv, _ = sla_cg_adjoint(ctx.pattern, values, x, g, ctx.tol, ctx.maxit, want_vals,
                                       jacobi=ctx.jacobi)
        return gv, gb, None, None, None, None


class _BiCGStabSolve(torch.autograd.Function):
    """x = A^{-1} b by BiCGStab (general A); backward: A^T lambda = g by
    BiCGStab, grad_b = lambda, grad_vals = -lambda_i x_j on the pattern."""

    @staticmethod
    def forward(ctx, values, b, pattern, tol, maxit):
        x, infos = sla_bicgstab_solve(pattern, values.detach().contiguous(), b.contiguous(), tol,
                                      maxit)
        ctx.pattern, ctx.tol, ctx.maxit = pattern, tol, maxit
        ctx.infos = infos
        ctx.save_for_backward(values, x)
        return x

    @staticmethod
    def backward(ctx, grad_x):
        values, x = ctx.saved_tensors
        gb, gv, _ = sla_bicgstab_adjoint(ctx.pattern, values.detach().contiguous(), x,
                                         grad_x.contiguous(), ctx.tol, ctx.maxit,
                                         want_vals=ctx.needs_input_grad[0])
        return gv, gb, None, None, None


class _ListSolve(torch.autograd.Function):
    """[x_i = A_i^{-1} b_i] for a list of systems with distinct patterns; one
    graph node; backward solves every adjoint system in one list call."""

    @staticmethod
    def forward(ctx, meta, *tensors):
        patterns, tol, maxit, method, jacobi = meta
        count = len(patterns)
        values = [t.detach().contiguous() for t in tensors[:count]]
        bs = [t.detach().contiguous() for t in tensors[count:]]
        xs, infos = sla_solve_list(patterns, values, bs, tol, maxit, method, jacobi)
        ctx.meta = meta
        ctx.infos = infos
        ctx.save_for_backward(*values, *xs)
        return tuple(xs)

    @staticmethod
    def backward(ctx, *grad_xs):
        patterns, tol, maxit, method, jacobi = ctx.meta
        count = len(patterns)
        saved = ctx.saved_tensors
        values, xs = list(saved[:count]), list(saved[count:])
        gx = [g.contiguous() if g is not None else torch.zeros_like(x)
              for g, x in zip(grad_xs, xs)]
        want = [ctx.needs_input_grad[1 + i] for i in range(count)]
        gbs, gvs, _ = sla_adjoint_list(patterns, values, xs, gx, tol, maxit, method, want,
                                       jacobi)
        return (None, *gvs, *gbs)


class _MatVec(torch.autograd.Function):
    """y = A x; backward grad_x = A^T g, grad_vals = g_i x_j on the pattern."""

    @staticmethod
    def forward(ctx, values, x, pattern):
        ctx.pattern = pattern
        ctx.save_for_backward(values, x)
        return sla_spmv(pattern, values.detach().contiguous(), x.detach().contiguous())

    @staticmethod
    def backward(ctx, grad_y):
        values, x = ctx.saved_tensors
        gx, gv = sla_matvec_grad(ctx.pattern, values.detach().contiguous(),
                                 x.detach().contiguous(), grad_y.contiguous(),
                                 want_x=ctx.needs_input_grad[1],
                                 want_vals=ctx.needs_input_grad[0])
        return gv, gx, None


class _EigSH(torch.autograd.Function):
    """theta, X = eigsh(A); backward d theta_t / d A_ij = X_ti X_tj on the
    pattern (Hellmann-Feynman).  X carries no gradient."""

    @staticmethod
    def forward(ctx, values, pattern, k, which, m, v0):
        theta, X, _, _ = sla_eigsh(pattern, values.detach().contiguous(), k, which, m,
                                   v0.contiguous())
        ctx.pattern = pattern
        ctx.save_for_backward(values, X)
        ctx.mark_non_differentiable(X)
        return theta, X

    @staticmethod
    def backward(ctx, grad_theta, grad_X):
        values, X = ctx.saved_tensors
        gv = None
        if ctx.needs_input_grad[0]:
            gv = sla_eig_grad(ctx.pattern, values.detach().contiguous(), X,
                              grad_theta.contiguous())
        return gv, None, None, None, None, None


class SparseTensor:
    """A sparse matrix (or a batch sharing one pattern) with .solve / .matvec.

    ``values`` is a float64 CUDA tensor [nnz] or [batch, nnz] in CSR slot
    order; it may require grad.  ``pattern`` is a CSRPattern.
    """

    def __init__(self, pattern: CSRPattern, values: torch.Tensor):
        if values.shape[-1] != pattern.nnz:
            raise ValueError("values do not match the pattern")
        self.pattern = pattern
        self.values = values

    @property
    def shape(self):
        return (self.pattern.n, self.pattern.n)

    def solve(self, b: torch.Tensor, tol: float = 1e-10, maxit: int = 10000,
              precond: str | None = None, method: str = "cg") -> torch.Tensor:
        """x = A^{-1} b: method "cg" (symmetric positive definite A; precond
        "jacobi" for diag(A)) or "bicgstab" (general A, no preconditioner)."""
        if method == "bicgstab":
            if precond is not None:
                raise ValueError("BiCGStab runs without a preconditioner")
            return _BiCGStabSolve.apply(self.values, b, self.pattern, float(tol), int(maxit))
        if method != "cg":
            raise ValueError(f"unknown method {method!r}")
        if precond not in (None, "jacobi"):
            raise ValueError(f"unknown preconditioner {precond!r}")
        return _CGSolve.apply(self.values, b, self.pattern, float(tol), int(maxit),
                              precond == "jacobi")

    def matvec(self, x: torch.Tensor) -> torch.Tensor:
        """y = A x, differentiable in the values and in x (one graph node)."""
        return _MatVec.apply(self.values, x, self.pattern)

    def eigsh(self, k: int = 6, which: str = "LA", m: int | None = None,
              v0: torch.Tensor | None = None):
        """(theta, X): the k largest ("LA") or smallest ("SA") eigenpairs of the
        symmetric matrix by m Lanczos steps (default min(n, max(2k + 1, 64)));
        theta is differentiable in the values (Hellmann-Feynman)."""
        n = self.pattern.n
        if m is None:
            m = min(n, max(2 * k + 1, 64))
        if v0 is None:
            g = torch.Generator().manual_seed(0)
            shape = (self.values.shape[0], n) if self.values.dim() == 2 else (n,)
            v0 = torch.randn(shape, generator=g, dtype=torch.float64).to(self.values.device)
        return _EigSH.apply(self.values, self.pattern, int(k), which, int(m), v0)


class SparseTensorList:
    """A list of sparse matrices with distinct patterns (and sizes): the
    ragged counterpart of a batched SparseTensor.  ``.solve`` solves all of
    them in one call of the library (up to 8 at once on the GPU) and is one
    autograd node; each item's values and right-hand side get gradients."""

    def __init__(self, tensors: list):
        if not tensors:
            raise ValueError("empty list")
        if len({id(t.pattern) for t in tensors}) != len(tensors):
            raise ValueError("every item needs a pattern of its own")
        self.tensors = list(tensors)

    def __len__(self):
        return len(self.tensors)

    def __getitem__(self, i):
        return self.tensors[i]

    def solve(self, bs: list, tol: float = 1e-10, maxit: int = 10000, method: str = "cg",
              precond: str | None = None) -> list:
        if len(bs) != len(self.tensors):
            raise ValueError("one right-hand side per matrix")
        if precond not in (None, "jacobi") or (precond and method != "cg"):
            raise ValueError(f"preconditioner {precond!r} not available for {method}")
        meta = ([t.pattern for t in self.tensors], float(tol), int(maxit), method,
                precond == "jacobi")
        return list(_ListSolve.apply(meta, *[t.values for t in self.tensors], *bs))

    def matvec(self, xs: list) -> list:
        return [t.matvec(x) for t, x in zip(self.tensors, xs)]


def solve(A: SparseTensor, b: torch.Tensor, tol: float = 1e-10, maxit: int = 10000,
          precond: str | None = None, method: str = "cg"):
    """x = A^{-1} b with the adjoint backward pass."""
    return A.solve(b, tol, maxit, precond, method)
