"""Closed forms of the 5-point Laplacian used to pin the oracle.

For the N x N interior grid with h = 1/(N+1), diagonal 4 and neighbours -1,
the eigenvectors are v_pq(a, c) = sin(p pi a h) sin(q pi c h) with
eigenvalues 4 - 2 cos(p pi h) - 2 cos(q pi h), 1 <= p, q <= N (the form the
benchmark configuration states for the Rayleigh-quotient checks).
"""
from __future__ import annotations

import numpy as np


def eigval(N: int, p: int, q: int) -> float:
    h = 1.0 / (N + 1)
    return 4.0 - 2.0 * np.cos(p * np.pi * h) - 2.0 * np.cos(q * np.pi * h)


def eigvec(N: int, p: int, q: int) -> np.ndarray:
    """Flattened in the grid numbering i = (c-1) N + (a-1)."""
    h = 1.0 / (N + 1)
    a = np.arange(1, N + 1)
    sx = np.sin(p * np.pi * a * h)
    sy = np.sin(q * np.pi * a * h)
    return np.outer(sy, sx).reshape(-1)  # row index c, column index a


def spectrum_bounds(N: int):
    h = 1.0 / (N + 1)
    return 4.0 - 4.0 * np.cos(np.pi * h), 4.0 + 4.0 * np.cos(np.pi * h)
