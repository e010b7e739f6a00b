"""Helpers shared by the GPU tests: move seeded inputs to the device, build
handles through the C ABI, compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

TOL_X = 1e-8       # relative L2 on x and lambda
TOL_GRAD = 1e-7    # relative L2 on grad_vals
ITER_FRAC = 0.02   # iteration counts within 2 %


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda", 0)


def t(a, dtype=None):
    import torch
    x = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        x = x.to(dtype)
    return x.to(dev())


def rel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def iters_close(a: int, b: int) -> bool:
    return abs(a - b) <= max(1, ITER_FRAC * max(a, b))


def csr_handle(rowptr, col, one_group="auto"):
    """A pattern handle; one_group="off" keeps small systems and single
    mid-size banded systems on the two-kernel CG loop (for tests of its kernel
    families)."""
    import krylov_solvers_adjoint_amd as K
    P = K.sla_csr_create_from_csr(t(rowptr), t(col.astype(np.int32)))
    if one_group != "auto":
        P.set_one_group(one_group)
    return P
