"""GPU pattern construction vs the oracle: bit-exact rowptr, col, perm and
merged values; validation errors; grad mapping back to COO."""
import numpy as np
import pytest

import oracle
import oracle_pins
import workloads as W
from gpu_util import csr_handle, say, t

pytestmark = pytest.mark.gpu


def _build_and_compare(n, row, col, val, coo_dtype, rp_dtype):
    import torch
    import krylov_solvers_adjoint_amd as K
    rp_o, c_o, perm_o = oracle.csr_from_coo(n, row, col)
    v_o = oracle.values_from_coo(perm_o, int(rp_o[-1]), val)
    P = K.sla_csr_create(n, t(np.asarray(row), coo_dtype), t(np.asarray(col), coo_dtype),
                         rowptr_dtype=rp_dtype)
    rp, c, perm = P.pattern()
    vals = K.sla_csr_values_from_coo(P, t(np.asarray(val, np.float64)))
    torch.cuda.synchronize()
    assert P.nnz == int(rp_o[-1])
    assert np.array_equal(rp.cpu().numpy().astype(np.int64), rp_o)
    assert np.array_equal(c.cpu().numpy(), c_o)
    if len(row):
        assert np.array_equal(perm.cpu().numpy(), perm_o)
    assert np.array_equal(vals.cpu().numpy().view(np.int64), v_o.view(np.int64))
    return P, vals


@pytest.mark.parametrize("coo_w,rp_w", [("i32", "i32"), ("i64", "i64"), ("i64", "i32")])
def test_tiny_random_coo_bitexact(coo_w, rp_w):
    import torch
    cd = torch.int32 if coo_w == "i32" else torch.int64
    rd = torch.int32 if rp_w == "i32" else torch.int64
    for n, row, col, val in oracle_pins.tiny_coo_cases():
        _build_and_compare(n, np.array(row, np.int64), np.array(col, np.int64),
                           np.array(val, np.float64), cd, rd)


def test_poisson_shuffled_with_duplicates():
    import torch
    N = 70  # 4900 rows: 20 tiles, the last one ragged
    row, col, val = W.poisson_coo(N)
    r, c, v = W.shuffled_coo(row, col, val, seed=11, dup_frac=0.2)
    _build_and_compare(N * N, r, c, v, torch.int64, torch.int32)


def test_rgg_and_long_rows():
    """Random geometric graph (rows 1..~25) plus rows long enough for the
    workgroup sort (33..4096) and for the global sort (> 4096)."""
    import torch
    n = 20000
    row, col, val, _ = W.rgg_coo(n, 4, 5)
    rng = np.random.default_rng(3)
    extra_r = np.concatenate([np.full(5000, 7), np.full(300, 11), np.full(40, 13)])
    extra_c = np.concatenate([rng.integers(0, n, 5000), rng.integers(0, n, 300),
                              rng.integers(0, n, 40)])
    extra_v = rng.standard_normal(extra_r.shape[0])
    r = np.concatenate([row, extra_r])
    c = np.concatenate([col, extra_c])
    v = np.concatenate([val, extra_v])
    p = rng.permutation(r.shape[0])
    say(f"rgg+long: n={n} triplets={r.shape[0]}")
    _build_and_compare(n, r[p], c[p], v[p], torch.int32, torch.int32)


def test_grad_to_coo_and_batched_values():
    import torch
    import krylov_solvers_adjoint_amd as K
    n, row, col, val = oracle_pins.tiny_coo_cases()[10]
    row = np.array(row, np.int64)
    col = np.array(col, np.int64)
    rp_o, c_o, perm_o = oracle.csr_from_coo(n, row, col)
    P = K.sla_csr_create(n, t(row), t(col))
    vb = np.random.default_rng(0).standard_normal((3, len(row)))
    vals = K.sla_csr_values_from_coo(P, t(vb))
    gv = np.random.default_rng(1).standard_normal((3, P.nnz))
    gc = K.sla_csr_grad_to_coo(P, t(gv))
    torch.cuda.synchronize()
    for s in range(3):
        vo = oracle.values_from_coo(perm_o, P.nnz, vb[s])
        assert np.array_equal(vals[s].cpu().numpy().view(np.int64), vo.view(np.int64))
        assert np.array_equal(gc[s].cpu().numpy(), gv[s][perm_o])


def test_from_csr_validation():
    import torch
    import krylov_solvers_adjoint_amd as K
    rp, c, _ = W.poisson_csr(5, np.int32)
    ok = csr_handle(rp, c)
    assert ok.nnz == len(c)
    bad_cases = []
    r1 = rp.copy(); r1[0] = 1; bad_cases.append((r1, c))             # rowptr[0] != 0
    r2 = rp.copy(); r2[-1] -= 1; bad_cases.append((r2, c))           # rowptr[n] != nnz
    r3 = rp.copy(); r3[3], r3[4] = r3[4], r3[3]; bad_cases.append((r3, c))  # decreasing
    r4 = rp.copy(); r4[5] = 10**6; bad_cases.append((r4, c))         # beyond nnz
    c5 = c.copy(); c5[7] = 25; bad_cases.append((rp, c5))            # column out of range
    c6 = c.copy(); c6[0], c6[1] = c6[1], c6[0]; bad_cases.append((rp, c6))  # unsorted
    c7 = c.copy(); c7[1] = c7[0]; bad_cases.append((rp, c7))         # duplicate column
    for r_, c_ in bad_cases:
        with pytest.raises(K.SlaError) as e:
            csr_handle(r_, c_)
        assert e.value.status == K.ERR_CSR
    with pytest.raises(K.SlaError) as e:
        K.sla_csr_create(4, t(np.array([0, 5])), t(np.array([0, 0])))
    assert e.value.status == K.ERR_CSR
    torch.cuda.synchronize()
