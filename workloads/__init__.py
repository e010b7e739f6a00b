"""Seeded synthetic inputs shared by the HIP library's tests, the oracle's
tests and the benchmark.

This module only *defines inputs*: matrix patterns and values, right-hand
sides and loss gradients, all from fixed seeds (numpy PCG64).  It contains
none of the solver's arithmetic (no CSR build from COO, no SpMV, no dot, no
CG) and imports neither the product library nor the oracle.

Workloads (the torch-sla explainer's experiments use 2D Poisson systems on
one GPU up to 169M unknowns; the unstructured and batched cases stand in for
its SparseTensor batching and graph-Laplacian use):

* Poisson 5-point Laplacian on an N x N interior grid, Dirichlet-zero
  boundary eliminated, diagonal 4, neighbours -1 (no 1/h^2 scaling),
  unknown (a, c) with 1 <= a, c <= N numbered i = (c-1) N + (a-1),
  columns ascending i-N, i-1, i, i+1, i+N.
* A shared-pattern batch: the same Laplacian plus a per-system diagonal
  shift c_s ~ U(0, 1).
* A random geometric graph Laplacian: points i.i.d. uniform in the unit
  square in sampling order (hence a random node order), an edge when two
  points are within r = sqrt(deg / (pi n)), one weight ~ U(0.5, 1.5) per
  undirected edge drawn in lexicographic (i < j) order, A = D - W + shift I.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "poisson_n", "poisson_nnz", "poisson_csr", "poisson_coo", "manufactured",
    "uniform_rhs", "normal_rhs", "batched_poisson", "rgg_coo", "shuffled_coo",
    "stencil_csr", "laplacian3d_csr", "nine_point_csr",
    "CONFIGS",
]


def poisson_n(N: int) -> int:
    return N * N


def poisson_nnz(N: int) -> int:
    return 5 * N * N - 4 * N


def _grid_line(N: int, has_down: bool, has_up: bool, diag: float, off: float):
    """Slots of one grid line of rows a = 0..N-1, in CSR order: column offsets
    relative to the line's first unknown, values, and per-row counts."""
    a = np.arange(N, dtype=np.int64)
    kinds = []  # (present mask, column offset relative to the row, value)
    if has_down:
        kinds.append((np.ones(N, bool), -N, off))
    kinds.append((a > 0, -1, off))
    kinds.append((np.ones(N, bool), 0, diag))
    kinds.append((a < N - 1, 1, off))
    if has_up:
        kinds.append((np.ones(N, bool), N, off))
    counts = sum(m.astype(np.int64) for m, _, _ in kinds)
    start = np.zeros(N, np.int64)
    start[1:] = np.cumsum(counts)[:-1]
    total = int(counts.sum())
    col = np.empty(total, np.int64)
    val = np.empty(total, np.float64)
    pos = start.copy()
    for m, o, v in kinds:
        idx = pos[m]
        col[idx] = a[m] + o
        val[idx] = v
        pos[m] += 1
    return col, val, counts


def poisson_csr(N: int, rowptr_dtype=np.int32, diag: float = 4.0, off: float = -1.0):
    """Closed-form CSR of the N x N 5-point Laplacian.

    Returns (rowptr[rowptr_dtype, n+1], col[int32, nnz], vals[float64, nnz]).
    Every interior grid line has the same pattern relative to its first
    unknown, so the matrix is assembled line by line from three templates.
    """
    n = N * N
    if N == 1:
        lines = [(_grid_line(1, False, False, diag, off), 1)]
    else:
        lines = [(_grid_line(N, False, True, diag, off), 1),
                 (_grid_line(N, True, True, diag, off), N - 2),
                 (_grid_line(N, True, False, diag, off), 1)]
    cols, vals, counts = [], [], []
    first = 0
    for (c, v, k), reps in lines:
        if reps == 0:
            continue
        bases = (np.arange(reps, dtype=np.int64) + first) * N
        cols.append(np.add.outer(bases.astype(np.int32 if n < 2**31 else np.int64),
                                 c.astype(np.int32 if n < 2**31 else np.int64)).ravel())
        vals.append(np.tile(v, reps))
        counts.append(np.tile(k, reps))
        first += reps
    col = np.concatenate(cols).astype(np.int32, copy=False)
    vals = np.concatenate(vals)
    rowptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(np.concatenate(counts), out=rowptr[1:])
    return rowptr.astype(rowptr_dtype, copy=False), col, vals


def convection_diffusion_csr(N: int, eps: float = 0.05, wind: float = 1.0,
                             rowptr_dtype=np.int32):
    """CSR of the N x N upwind convection-diffusion operator
    -eps Laplace(u) + wind du/da with h = 1/(N+1), zero Dirichlet boundary and
    the flow along the grid lines (+a): row i = (c-1) N + (a-1) holds
    -eps/h^2 (south, north, east), -eps/h^2 - wind/h (west, upwind) and
    4 eps/h^2 + wind/h (diagonal), columns ascending.  A non-symmetric
    M-matrix with the Poisson pattern.  Returns (rowptr, col, vals)."""
    n = N * N
    h = 1.0 / (N + 1)
    d, w = eps / h ** 2, wind / h
    i = np.arange(n, dtype=np.int64)
    a, c = i % N, i // N
    parts = [(i - N, -d, c > 0), (i - 1, -d - w, a > 0), (i, 4 * d + w, np.ones(n, bool)),
             (i + 1, -d, a < N - 1), (i + N, -d, c < N - 1)]
    counts = sum(m.astype(np.int64) for _, _, m in parts)
    rowptr = np.zeros(n + 1, np.int64)
    np.cumsum(counts, out=rowptr[1:])
    col = np.empty(rowptr[-1], np.int32)
    val = np.empty(rowptr[-1], np.float64)
    pos = rowptr[:-1].copy()
    for cols, v, m in parts:   # in ascending column order
        col[pos[m]] = cols[m]
        val[pos[m]] = v
        pos[m] += 1
    return rowptr.astype(rowptr_dtype, copy=False), col, val


def stencil_csr(shape, stencil, rowptr_dtype=np.int32):
    """CSR of a constant-coefficient stencil on a box grid with a zero
    Dirichlet boundary: `stencil` maps a displacement tuple (x fastest) to
    its value.  Columns come out ascending.  Small grids only (tests)."""
    dims = len(shape)
    n = int(np.prod(shape))
    idx = np.arange(n)
    coords = []
    rem = idx.copy()
    for d in range(dims):
        coords.append(rem % shape[d])
        rem //= shape[d]
    strides = np.cumprod([1] + list(shape[:-1]))
    entries = []
    for disp, v in stencil.items():
        ok = np.ones(n, bool)
        for d in range(dims):
            ok &= (coords[d] + disp[d] >= 0) & (coords[d] + disp[d] < shape[d])
        off = int(sum(disp[d] * strides[d] for d in range(dims)))
        entries.append((idx[ok], idx[ok] + off, np.full(ok.sum(), v, np.float64)))
    row = np.concatenate([e[0] for e in entries])
    col = np.concatenate([e[1] for e in entries])
    val = np.concatenate([e[2] for e in entries])
    order = np.lexsort((col, row))
    row, col, val = row[order], col[order], val[order]
    rowptr = np.zeros(n + 1, np.int64)
    np.add.at(rowptr, row + 1, 1)
    return np.cumsum(rowptr).astype(rowptr_dtype), col.astype(np.int32), val


def band_csr(n: int, offsets, diag: float, off: float = -1.0, rowptr_dtype=np.int32):
    """CSR of the n x n band matrix with `diag` on the diagonal and `off` at
    every column i + d (d in `offsets`, d != 0) that lies in [0, n).  Unlike
    a grid stencil, couplings cross the ends of grid lines and n need not be
    a multiple of the line length.  Columns come out ascending."""
    ds = sorted(set(int(d) for d in offsets) | {0})
    idx = np.arange(n)
    entries = []
    for d in ds:
        ok = (idx + d >= 0) & (idx + d < n)
        entries.append((idx[ok], idx[ok] + d, np.full(ok.sum(), diag if d == 0 else off)))
    row = np.concatenate([e[0] for e in entries])
    col = np.concatenate([e[1] for e in entries])
    val = np.concatenate([e[2] for e in entries])
    order = np.lexsort((col, row))
    row, col, val = row[order], col[order], val[order]
    rowptr = np.zeros(n + 1, np.int64)
    np.add.at(rowptr, row + 1, 1)
    return np.cumsum(rowptr).astype(rowptr_dtype), col.astype(np.int32), val


def rough_diffusion_csr(N: int, seed: int, spread: float, rowptr_dtype=np.int32):
    """CSR of the 5-point finite-volume diffusion operator on an N x N grid
    with a conductance per cell edge drawn log-uniform from [e^-spread,
    e^spread] (seeded) and the grid's boundary edges held at zero (their
    conductances on the diagonal): a_ij = -c_ij for neighbours, a_ii = the
    sum of the cell's edge conductances.  Symmetric positive definite, its
    condition number about e^(2 spread) times the Laplacian's.  Columns come
    out ascending."""
    rng = np.random.default_rng(seed)
    n = N * N
    cx = np.exp(rng.uniform(-spread, spread, (N, N + 1)))  # edges along a grid line
    cy = np.exp(rng.uniform(-spread, spread, (N + 1, N)))  # edges across grid lines
    i, j = np.divmod(np.arange(n), N)
    diag = cx[i, j] + cx[i, j + 1] + cy[i, j] + cy[i + 1, j]
    entries = [(np.arange(n), np.arange(n), diag)]
    ok = j + 1 < N
    entries.append((np.flatnonzero(ok), np.flatnonzero(ok) + 1, -cx[i[ok], j[ok] + 1]))
    ok = j > 0
    entries.append((np.flatnonzero(ok), np.flatnonzero(ok) - 1, -cx[i[ok], j[ok]]))
    ok = i + 1 < N
    entries.append((np.flatnonzero(ok), np.flatnonzero(ok) + N, -cy[i[ok] + 1, j[ok]]))
    ok = i > 0
    entries.append((np.flatnonzero(ok), np.flatnonzero(ok) - N, -cy[i[ok], j[ok]]))
    row = np.concatenate([e[0] for e in entries])
    col = np.concatenate([e[1] for e in entries])
    val = np.concatenate([e[2] for e in entries]).astype(np.float64)
    order = np.lexsort((col, row))
    row, col, val = row[order], col[order], val[order]
    rowptr = np.zeros(n + 1, np.int64)
    np.add.at(rowptr, row + 1, 1)
    return np.cumsum(rowptr).astype(rowptr_dtype), col.astype(np.int32), val


def laplacian3d_csr(N: int):
    """7-point Laplacian on an N^3 grid: diagonal 6, neighbours -1."""
    st = {(0, 0, 0): 6.0}
    for d in range(3):
        for s_ in (-1, 1):
            disp = [0, 0, 0]
            disp[d] = s_
            st[tuple(disp)] = -1.0
    return stencil_csr((N, N, N), st)


def nine_point_csr(N: int):
    """9-point Laplacian on an N^2 grid: diagonal 8, the 8 neighbours -1."""
    st = {(a, b): (8.0 if a == 0 and b == 0 else -1.0) for a in (-1, 0, 1) for b in (-1, 0, 1)}
    return stencil_csr((N, N), st)


def poisson_coo(N: int):
    """The same matrix as coordinate triplets (row, col int64; val float64)."""
    rowptr, col, vals = poisson_csr(N, np.int64)
    row = np.repeat(np.arange(N * N, dtype=np.int64), np.diff(rowptr))
    return row, col.astype(np.int64), vals


def manufactured(N: int):
    """u*(x, y) = sin(pi x) sin(pi y) at the interior nodes, h = 1/(N+1),
    and b = A u* written out with the 5-point stencil on the grid."""
    h = 1.0 / (N + 1)
    s = np.sin(np.pi * h * np.arange(1, N + 1))
    U = np.outer(s, s)  # U[c-1, a-1] = sin(pi a h) sin(pi c h)
    P = np.zeros((N + 2, N + 2))
    P[1:-1, 1:-1] = U
    B = 4.0 * U - P[1:-1, :-2] - P[1:-1, 2:] - P[:-2, 1:-1] - P[2:, 1:-1]
    return U.reshape(-1).copy(), B.reshape(-1).copy()


def uniform_rhs(n: int, seed: int) -> np.ndarray:
    return np.random.default_rng(seed).uniform(-1.0, 1.0, n)


def normal_rhs(n: int, seed: int, shape=None) -> np.ndarray:
    return np.random.default_rng(seed).standard_normal(shape if shape is not None else n)


def batched_poisson(N: int, batch: int, seed_shift: int, seed_rhs: int):
    """Shared 5-point pattern; system s has diagonal 4 + c_s, c_s ~ U(0, 1).

    Returns (rowptr, col, vals[batch, nnz], b[batch, n], shifts[batch]).
    """
    rowptr, col, base = poisson_csr(N, np.int32)
    shifts = np.random.default_rng(seed_shift).uniform(0.0, 1.0, batch)
    diag_slot = base == 4.0
    vals = np.repeat(base[None, :], batch, axis=0)
    vals[:, diag_slot] = 4.0 + shifts[:, None]
    b = np.random.default_rng(seed_rhs).standard_normal((batch, N * N))
    return rowptr, col, vals, b, shifts


def rgg_coo(n: int, seed_points: int, seed_weights: int, degree: float = 8.0,
            shift: float = 1e-2):
    """Random geometric graph Laplacian + shift*I as unsorted COO triplets.

    Entry order: (i, j) for every edge i < j, then (j, i) for the same
    edges, then the n diagonal entries; the matrix is symmetric bit for bit.
    Returns (row int64, col int64, val float64, points).
    """
    from scipy.spatial import cKDTree

    pts = np.random.default_rng(seed_points).random((n, 2))
    r = float(np.sqrt(degree / (np.pi * n)))
    pairs = cKDTree(pts).query_pairs(r, output_type="ndarray").astype(np.int64)
    order = np.lexsort((pairs[:, 1], pairs[:, 0]))
    i, j = pairs[order, 0], pairs[order, 1]
    w = np.random.default_rng(seed_weights).uniform(0.5, 1.5, i.shape[0])
    deg = np.bincount(i, weights=w, minlength=n) + np.bincount(j, weights=w, minlength=n)
    d = np.arange(n, dtype=np.int64)
    row = np.concatenate([i, j, d])
    col = np.concatenate([j, i, d])
    val = np.concatenate([-w, -w, deg + shift])
    return row, col, val, pts


def shuffled_coo(row, col, val, seed: int, dup_frac: float = 0.0):
    """A permutation of COO triplets, optionally with some entries split into
    duplicates whose values add up to the original only up to rounding (the
    test compares merged results, not the original values)."""
    rng = np.random.default_rng(seed)
    m = row.shape[0]
    if dup_frac > 0:
        k = rng.choice(m, size=max(1, int(dup_frac * m)), replace=False)
        extra = rng.uniform(-1.0, 1.0, k.shape[0])
        row = np.concatenate([row, row[k]])
        col = np.concatenate([col, col[k]])
        val = np.concatenate([val, extra])
    perm = rng.permutation(row.shape[0])
    return row[perm], col[perm], val[perm]


# The benchmark / parity workloads, named by what they are.
CONFIGS = {
    "poisson32": dict(kind="poisson", N=32, rhs="uniform", seed_b=0, seed_g=1,
                      tol=1e-10, maxit=10000, rowptr="i32"),
    "poisson1000_fixed1000": dict(kind="poisson", N=1000, rhs="manufactured",
                                  seed_g=1, tol=0.0, maxit=1000, rowptr="i32"),
    "batched64_poisson128": dict(kind="batched", N=128, batch=64, seed_shift=2,
                                 seed_b=3, tol=1e-8, maxit=10000, rowptr="i32"),
    "rgg4m": dict(kind="rgg", n=4_000_000, seed_points=4, seed_weights=5,
                  seed_b=6, seed_g=7, tol=1e-8, maxit=20000, rowptr="i32"),
    "poisson4000_fixed500": dict(kind="poisson", N=4000, rhs="uniform", seed_b=0,
                                 tol=0.0, maxit=500, rowptr="i32"),
    "poisson13000_fixed500": dict(kind="poisson", N=13000, rhs="uniform", seed_b=0,
                                  tol=0.0, maxit=500, rowptr="i64"),
}
