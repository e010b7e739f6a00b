"""Planted mistakes: each mutation below is a plausible slip in the oracle
(a dropped term, a wrong sign, index or operand).  A mutated copy of
``oracle.c`` is compiled into a temporary directory and every pin is run
against it in a child process; at least one pin must fail.  The real oracle
source is never modified.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTATIONS = {
    "spmv_row_for_col": ("s = s + vals[k] * x[col[k]]", "s = s + vals[k] * x[i]"),
    "grad_sign": ("grad_vals[k] = -(lambda[i] * x[col[k]])", "grad_vals[k] = (lambda[i] * x[col[k]])"),
    "grad_transposed": ("grad_vals[k] = -(lambda[i] * x[col[k]])", "grad_vals[k] = -(lambda[col[k]] * x[i])"),
    "beta_inverted": ("double beta = rr_new / rr;", "double beta = rr / rr_new;"),
    "alpha_inverted": ("double alpha = rr / pq;", "double alpha = pq / rr;"),
    "residual_sign": ("r[i] = r[i] - alpha * q[i];", "r[i] = r[i] + alpha * q[i];"),
    "x_uses_q": ("x[i] = x[i] + alpha * p[i];\n        r[i] = r[i] - alpha * q[i];",
                 "x[i] = x[i] + alpha * q[i];\n        r[i] = r[i] - alpha * q[i];"),
    "p_drops_old_p": ("p[i] = r[i] + beta * p[i];", "p[i] = r[i] + beta * r[i];"),
    "dot_drops_last_block": ("for (int64_t b = 0; b < nb; ++b) total = total + part[b];",
                             "for (int64_t b = 0; b + 1 < nb; ++b) total = total + part[b];"),
    "merge_last_wins": ("vals[s] = vals[s] + coo_val[k];", "vals[s] = coo_val[k];"),
    "sort_ignores_col": ("  if (a->col != b->col) return a->col < b->col ? -1 : 1;\n", ""),
    "stop_strict": ("if (rr <= stop) break;", "if (rr < stop) break;"),
    "adjoint_rhs_is_x": ("oracle_cg(n, rowptr_t, col_t, vals_t, g, grad_b",
                         "oracle_cg(n, rowptr_t, col_t, vals_t, x, grad_b"),
    "rowptr_shifted": ("rowptr[keys[s].row + 1] += 1;", "rowptr[keys[s].row] += 1;"),
    "warm_start_sign": ("r[i] = b[i] - q[i];", "r[i] = q[i] - b[i];"),
    "transpose_keeps_rows": ("col_t[dst] = (int32_t)i;", "col_t[dst] = (int32_t)j;"),
    "pcg_beta_uses_rr": ("double beta = rz_new / rz;", "double beta = rr_new / rr;"),
    "pcg_alpha_uses_rr": ("double alpha = rz / pq;", "double alpha = rr / pq;"),
    "pcg_z_times_d": ("z[i] = r[i] / d[i];", "z[i] = r[i] * d[i];"),
    "pcg_p_from_r": ("p[i] = z[i] + beta * p[i];", "p[i] = r[i] + beta * p[i];"),
    "pcg_diag_from_row_start": ("if (col[s] == i) d[i] = vals[s];", "d[i] = vals[rowptr[i]];"),
    "pcg_adjoint_rhs_is_x": ("oracle_pcg_jacobi(n, rowptr_t, col_t, vals_t, g, grad_b",
                             "oracle_pcg_jacobi(n, rowptr_t, col_t, vals_t, x, grad_b"),
    "matvec_grad_sign": ("grad_vals[k] = g[i] * x[col[k]];", "grad_vals[k] = -(g[i] * x[col[k]]);"),
    "matvec_grad_no_transpose": ("oracle_spmv(n, rowptr_t, col_t, vals_t, g, grad_x);",
                                 "oracle_spmv(n, rowptr, col, vals, g, grad_x);"),
    "matvec_grad_swapped": ("grad_vals[k] = g[i] * x[col[k]];", "grad_vals[k] = g[col[k]] * x[i];"),
    "lanczos_one_pass": ("for (int pass = 0; pass < 2; ++pass) {", "for (int pass = 0; pass < 1; ++pass) {"),
    "lanczos_alpha_second_pass_only": ("a = a + h[j];", "a = h[j];"),
    "lanczos_beta_squared": ("double b = sqrt(oracle_dot(n, w, w));", "double b = oracle_dot(n, w, w);"),
    "eig_grad_diagonal_only": ("grad_vals[k] = v[i] * v[col[k]];", "grad_vals[k] = v[i] * v[i];"),
    "bicgstab_p_sign": ("p[i] = r[i] + beta * (p[i] - omega * v[i]);",
                        "p[i] = r[i] + beta * (p[i] + omega * v[i]);"),
    "bicgstab_omega_inverted": ("omega = ts / tt;", "omega = tt / ts;"),
    "bicgstab_beta_swapped": ("double beta = (rho / rho_prev) * (alpha / omega);",
                              "double beta = (rho / rho_prev) * (omega / alpha);"),
    "bicgstab_x_drops_omega_s": ("x[i] = (x[i] + alpha * p[i]) + omega * sv[i];",
                                 "x[i] = x[i] + alpha * p[i];"),
    "bicgstab_r_sign": ("r[i] = sv[i] - omega * t[i];", "r[i] = sv[i] + omega * t[i];"),
    "bicgstab_s_uses_p": ("sv[i] = r[i] - alpha * v[i];", "sv[i] = r[i] - alpha * p[i];"),
    "bicgstab_rho_prev_stale": ("    rho_prev = rho;\n  }\n  info->iterations = k;",
                                "  }\n  info->iterations = k;"),
    "bicgstab_half_step_no_x": ("      for (int64_t i = 0; i < n; ++i) x[i] = x[i] + alpha * p[i];\n      if (hist_omega) hist_omega[k] = 0.0;",
                                "      if (hist_omega) hist_omega[k] = 0.0;"),
    "bfs_far_node_largest": ("if (dist[order[t]] == depth && (s1 < 0 || order[t] < s1)) s1 = order[t];",
                             "if (dist[order[t]] == depth && (s1 < 0 || order[t] > s1)) s1 = order[t];"),
    "bfs_start_last_longest": ("if (rowptr[i + 1] - rowptr[i] > rowptr[s0 + 1] - rowptr[s0]) s0 = i;",
                               "if (rowptr[i + 1] - rowptr[i] >= rowptr[s0 + 1] - rowptr[s0]) s0 = i;"),
    "bfs_no_restart": ("if (dist[i] < 0) bfs_visit(rowptr, col, i, order, &len, dist);", ""),
    "bfs_start_is_s0": ("  bfs_visit(rowptr, col, s1, order, &len, dist);\n",
                        "  bfs_visit(rowptr, col, s0, order, &len, dist);\n"),
    "permute_unsorted": ("while (w > a && col_p[w - 1] > c) {", "while (0) {"),
    "bicgstab_adjoint_on_A": ("  int status = oracle_bicgstab(n, rowptr_t, col_t, vals_t, g, grad_b,",
                              "  int status = oracle_bicgstab(n, rowptr, col, vals, g, grad_b,"),
}

CHILD = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
lib = oracle._load({lib!r})
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib=lib)
    except Exception as e:
        failed.append(pin.__name__)
        break
print("FAILED:" + ",".join(failed))
"""


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    import oracle

    src = open(SRC).read()
    old, new = MUTATIONS[name]
    assert old in src, f"mutation anchor not found: {old!r}"
    with tempfile.TemporaryDirectory() as d:
        msrc = os.path.join(d, "oracle_mut.c")
        with open(msrc, "w") as f:
            f.write(src.replace(old, new))
        lib = os.path.join(d, "liboracle_mut.so")
        oracle.build(msrc, lib, sanitize=False)
        code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
        env = dict(os.environ, OMP_NUM_THREADS="1")
        p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                           timeout=300, env=env)
        out = p.stdout.strip().splitlines()
        caught = p.returncode != 0 or (out and out[-1] != "FAILED:")
        assert caught, f"mutation {name} survived every pin"
