"""The banded SpMV kernels (mask byte per row instead of the column array):
detection, fallback, and bit-identity with the plain CSR kernels and the
oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from gpu_util import TOL_X, csr_handle, iters_close, rel, say, t

pytestmark = pytest.mark.gpu


def _spmv_both(rp, c, v, x):
    import torch
    import krylov_solvers_adjoint_amd as K
    P = csr_handle(rp, c)
    banded = P.set_spmv_variant("banded")
    y_auto = K.sla_spmv(P, t(v), t(x))
    P.set_spmv_variant("csr")
    y_csr = K.sla_spmv(P, t(v), t(x))
    torch.cuda.synchronize()
    yo = oracle.spmv(oracle.CSR(len(rp) - 1, rp.astype(np.int64), c, v), x)
    return banded, y_auto.cpu().numpy(), y_csr.cpu().numpy(), yo


@pytest.mark.parametrize("N", [1, 2, 5, 64, 301])
def test_poisson_banded_bitexact(N):
    rp, c, v = W.poisson_csr(N, np.int32)
    banded, ya, yc, yo = _spmv_both(rp, c, v, W.uniform_rhs(N * N, 3))
    assert banded == (N > 1) or N == 1
    assert np.array_equal(ya, yo) and np.array_equal(yc, yo)


def test_laplacian3d_seven_offsets():
    rp, c, v = W.laplacian3d_csr(21)
    banded, ya, yc, yo = _spmv_both(rp, c, v, W.normal_rhs(len(rp) - 1, 4))
    assert banded
    assert np.array_equal(ya, yo) and np.array_equal(yc, yo)


def test_nine_point_falls_back():
    rp, c, v = W.nine_point_csr(40)
    banded, ya, yc, yo = _spmv_both(rp, c, v, W.normal_rhs(len(rp) - 1, 5))
    assert not banded
    assert np.array_equal(ya, yo) and np.array_equal(yc, yo)


def test_verification_rejects_what_sampling_missed():
    """One far entry in a row the sampling does not look at: the device check
    refuses the band and the CSR kernels run."""
    N = 300
    rp, c, v = W.poisson_csr(N, np.int64)
    n = N * N
    i = 1234  # not in the sampled row blocks (starts at multiples of (n-1)/63)
    assert all(not (r0 <= i < r0 + 64) for r0 in [(n - 1) * s // 63 for s in range(64)])
    cols = list(c[rp[i]:rp[i + 1]]) + [n - 1]
    vals = list(v[rp[i]:rp[i + 1]]) + [0.5]
    c2 = np.concatenate([c[:rp[i]], np.array(cols, np.int32), c[rp[i + 1]:]])
    v2 = np.concatenate([v[:rp[i]], np.array(vals), v[rp[i + 1]:]])
    rp2 = rp.copy()
    rp2[i + 1:] += 1
    banded, ya, yc, yo = _spmv_both(rp2.astype(np.int32), c2, v2, W.uniform_rhs(n, 6))
    assert not banded
    assert np.array_equal(ya, yo) and np.array_equal(yc, yo)


@pytest.mark.parametrize("N,rpd", [(64, np.int32), (257, np.int64)])
def test_cg_adjoint_identical_bits_across_variants(N, rpd):
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.poisson_csr(N, rpd)
    n = N * N
    b = W.uniform_rhs(n, 0)
    g = W.normal_rhs(n, 1)
    out = []
    for variant in ("banded", "csr"):
        P = csr_handle(rp, c, one_group="off")  # the two-kernel loop's kernel families
        assert P.set_spmv_variant(variant) == (variant == "banded")
        x, info = K.sla_cg_solve(P, t(v), t(b), 1e-10, 20000)
        gb, gv, ai = K.sla_cg_adjoint(P, t(v), x, t(g), 1e-10, 20000)
        torch.cuda.synchronize()
        out.append((x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy(), info.iterations,
                    ai.iterations))
    a, bq = out
    for u, w in zip(a, bq):
        assert np.array_equal(np.asarray(u), np.asarray(w))
    xo, io = oracle.cg(oracle.CSR(n, rp.astype(np.int64), c, v), b, 1e-10, 20000)
    assert iters_close(a[3], io.iterations) and rel(a[0], xo) <= TOL_X


def test_laplacian3d_cg_against_oracle():
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.laplacian3d_csr(24)
    n = len(rp) - 1
    b = W.uniform_rhs(n, 8)
    P = csr_handle(rp, c)
    assert P.banded  # seven offsets: the automatic choice is the banded kernels
    x, info = K.sla_cg_solve(P, t(v), t(b), 1e-10, 5000)
    torch.cuda.synchronize()
    xo, io = oracle.cg(oracle.CSR(n, rp.astype(np.int64), c, v), b, 1e-10, 5000)
    say(f"3d: iterations {info.iterations}/{io.iterations} x {rel(x.cpu().numpy(), xo):.1e}")
    assert iters_close(info.iterations, io.iterations)
    assert rel(x.cpu().numpy(), xo) <= TOL_X


@pytest.mark.parametrize("variant", ["banded", "csr"])
def test_wide_band_panel_order(variant):
    """A 5000 x 40 grid: the +-5000 band is wider than 64 tiles, so the SpMV
    tiles are walked in panel order; CG and the adjoint still match the
    oracle and two runs give the same bits."""
    import torch
    import krylov_solvers_adjoint_amd as K
    st = {(0, 0): 4.0, (-1, 0): -1.0, (1, 0): -1.0, (0, -1): -1.0, (0, 1): -1.0}
    rp, c, v = W.stencil_csr((5000, 40), st)
    n = len(rp) - 1
    b = W.uniform_rhs(n, 11)
    g = W.normal_rhs(n, 12)
    runs = []
    for _ in range(2):
        P = csr_handle(rp, c)
        P.set_spmv_variant(variant)
        x, info = K.sla_cg_solve(P, t(v), t(b), 1e-10, 20000)
        gb, gv, ai = K.sla_cg_adjoint(P, t(v), x, t(g), 1e-10, 20000)
        y = K.sla_spmv(P, t(v), t(b))
        torch.cuda.synchronize()
        runs.append((x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy(), y.cpu().numpy(),
                     info.iterations, ai.iterations))
    for u, w in zip(*runs):
        assert np.array_equal(np.asarray(u), np.asarray(w))
    A = oracle.CSR(n, rp.astype(np.int64), c, v)
    assert np.array_equal(runs[0][3], oracle.spmv(A, b))
    xo, io = oracle.cg(A, b, 1e-10, 20000)
    gbo, gvo, aio = oracle.adjoint(A, xo, g, 1e-10, 20000)
    say(f"wide band {variant}: iterations {runs[0][4]}/{io.iterations}")
    assert iters_close(runs[0][4], io.iterations) and iters_close(runs[0][5], aio.iterations)
    assert rel(runs[0][0], xo) <= TOL_X and rel(runs[0][1], gbo) <= TOL_X
    assert rel(runs[0][2], gvo) <= 1e-7


def test_split_variant_random_graph():
    """The split variant (direction pass + product pass) on a random-order
    graph matches the oracle and is reproducible.  At 60000 nodes the column
    span of a tile is below the wide-tile threshold, so the automatic choice
    stays plain CSR and the variant is forced."""
    import torch
    import krylov_solvers_adjoint_amd as K
    n = 60000
    row, col, val, _ = W.rgg_coo(n, 4, 5)
    rp, c, perm = oracle.csr_from_coo(n, row, col)
    v = oracle.values_from_coo(perm, int(rp[-1]), val)
    b = W.normal_rhs(n, 6)
    g = W.normal_rhs(n, 7)
    runs = []
    for _ in range(2):
        P = csr_handle(rp.astype(np.int32), c)
        assert not P.split and not P.banded
        P.set_spmv_variant("split")
        assert P.split
        x, info = K.sla_cg_solve(P, t(v), t(b), 1e-8, 20000)
        gb, gv, ai = K.sla_cg_adjoint(P, t(v), x, t(g), 1e-8, 20000)
        torch.cuda.synchronize()
        runs.append((x.cpu().numpy(), gb.cpu().numpy(), gv.cpu().numpy(), info.iterations,
                     ai.iterations))
    for u, w in zip(*runs):
        assert np.array_equal(np.asarray(u), np.asarray(w))
    A = oracle.CSR(n, rp, c, v)
    xo, io = oracle.cg(A, b, 1e-8, 20000)
    gbo, gvo, aio = oracle.adjoint(A, xo, g, 1e-8, 20000)
    say(f"split rgg: iterations {runs[0][3]}/{io.iterations}, {runs[0][4]}/{aio.iterations}")
    assert iters_close(runs[0][3], io.iterations) and iters_close(runs[0][4], aio.iterations)
    assert rel(runs[0][0], xo) <= TOL_X and rel(runs[0][1], gbo) <= TOL_X
    assert rel(runs[0][2], gvo) <= 1e-7


@pytest.mark.parametrize("N", [1, 37, 300])
def test_split_variant_forced_poisson(N):
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, v = W.poisson_csr(N, np.int32)
    n = N * N
    b = W.uniform_rhs(n, 2)
    P = csr_handle(rp, c, one_group="off")  # small grids: keep the two-kernel loop
    P.set_spmv_variant("split")
    assert P.split
    x, info = K.sla_cg_solve(P, t(v), t(b), 1e-10, 20000, history=True)
    torch.cuda.synchronize()
    xo, io = oracle.cg(oracle.CSR(n, rp.astype(np.int64), c, v), b, 1e-10, 20000)
    assert iters_close(info.iterations, io.iterations) and rel(x.cpu().numpy(), xo) <= TOL_X
    assert len(P.history()[0]) == info.iterations
