"""The synthetic input generators produce the matrices they describe
(CPU): the convection-diffusion CSR against a dense assembly written out
from its stencil, for grids of 1 to 9 points a side."""
import numpy as np
import pytest

import workloads as W


def _dense_convection_diffusion(N, eps=0.05, wind=1.0):
    h = 1.0 / (N + 1)
    M = np.zeros((N * N, N * N))
    for c in range(N):
        for a in range(N):
            i = c * N + a
            M[i, i] = 4 * eps / h ** 2 + wind / h
            if a > 0:
                M[i, i - 1] = -eps / h ** 2 - wind / h
            if a + 1 < N:
                M[i, i + 1] = -eps / h ** 2
            if c > 0:
                M[i, i - N] = -eps / h ** 2
            if c + 1 < N:
                M[i, i + N] = -eps / h ** 2
    return M


@pytest.mark.parametrize("N", [1, 2, 3, 9])
@pytest.mark.parametrize("dtype", [np.int32, np.int64])
def test_convection_diffusion_csr(N, dtype):
    rp, c, v = W.convection_diffusion_csr(N, rowptr_dtype=dtype)
    assert rp.dtype == dtype and c.dtype == np.int32
    n = N * N
    rows = np.repeat(np.arange(n), np.diff(rp))
    for i in range(n):   # strictly ascending columns per row
        assert np.all(np.diff(c[rp[i]:rp[i + 1]]) > 0)
    D = np.zeros((n, n))
    D[rows, c] = v
    assert np.array_equal(D, _dense_convection_diffusion(N))


@pytest.mark.parametrize("N", [1, 2, 5])
def test_rough_diffusion_csr(N):
    """The rough-coefficient operator against its definition written cell by
    cell: every edge's conductance on both its cells' diagonals and, between
    two cells, off the diagonal with a minus sign; symmetric positive
    definite; rows ascending; the same seed gives the same matrix."""
    rp, c, v = W.rough_diffusion_csr(N, 11, 2.0)
    n = N * N
    D = np.zeros((n, n))
    rows = np.repeat(np.arange(n), np.diff(rp))
    D[rows, c] = v
    for i in range(n):
        assert np.all(np.diff(c[rp[i]:rp[i + 1]]) > 0)
    rng = np.random.default_rng(11)
    cx = np.exp(rng.uniform(-2.0, 2.0, (N, N + 1)))
    cy = np.exp(rng.uniform(-2.0, 2.0, (N + 1, N)))
    M = np.zeros((n, n))
    for r in range(N):
        for q in range(N + 1):      # edge left of cell (r, q) / right of (r, q - 1)
            for cell in ((r, q - 1), (r, q)):
                if 0 <= cell[1] < N:
                    M[cell[0] * N + cell[1], cell[0] * N + cell[1]] += cx[r, q]
            if 0 < q < N:
                a, b = r * N + q - 1, r * N + q
                M[a, b] -= cx[r, q]
                M[b, a] -= cx[r, q]
    for r in range(N + 1):
        for q in range(N):          # edge above cell (r, q) / below (r - 1, q)
            for cell in ((r - 1, q), (r, q)):
                if 0 <= cell[0] < N:
                    M[cell[0] * N + cell[1], cell[0] * N + cell[1]] += cy[r, q]
            if 0 < r < N:
                a, b = (r - 1) * N + q, r * N + q
                M[a, b] -= cy[r, q]
                M[b, a] -= cy[r, q]
    assert np.allclose(D, M, rtol=1e-15, atol=0)
    assert np.array_equal(D, D.T)
    assert np.linalg.eigvalsh(D).min() > 0
    rp2, c2, v2 = W.rough_diffusion_csr(N, 11, 2.0)
    assert np.array_equal(v, v2) and np.array_equal(c, c2)
