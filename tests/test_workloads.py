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
