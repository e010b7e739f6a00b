/*
 * CPU reference oracle for the CSR conjugate-gradient solve and its adjoint.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline use it.  It shares no code, header or constant with the HIP
 * library: both sides see only the seeded inputs made by `workloads/`.
 *
 * Source of the method: "torch-sla: Differentiable Sparse Linear Algebra with
 * Adjoint Solvers and Sparse Tensor Parallelism for PyTorch" (gist.science
 * explainer of arXiv 2601.13994), technical summary:
 *   - Methodology 1 (unified backend): the sparse tensor API (.solve, .matvec)
 *     and the shared-pattern SparseTensor; the CPU/GPU CG backends.
 *   - Methodology 2 (adjoint framework), linear systems: the backward pass
 *     solves A^T lambda = dL/dx and the matrix gradient is -lambda_i x_j,
 *     only on the sparsity pattern.
 *   - Methodology 2, complexity: O(1) graph nodes, O(n + nnz) memory.
 *   - Methodology 1 (.eigsh) and Methodology 2, eigenvalue problems: the
 *     eigenvalue gradient d lambda / d A_ij = v_i v_j on the pattern
 *     (Hellmann-Feynman); the Lanczos process below is this oracle's reading
 *     of .eigsh.
 * The CG steps themselves are the textbook Hestenes-Stiefel method that the
 * pages call "CG"; the pages fix no variant, so the plain one is used.
 *
 * Conventions (the pages are silent; these are the readings this oracle
 * takes):
 *   - x0 = 0 unless a start vector is supplied; stop when rr <= (tol*tol)*bb
 *     with rr the recursively updated residual norm squared and bb = b.b;
 *     the test is made before each iteration.
 *   - iterations = number of completed alpha updates.
 *   - breakdown: p.Ap not finite -> NONFINITE; p.Ap <= 0 -> NOT_SPD.
 *   - dot products: sequential sums over fixed 4096-element blocks, then a
 *     sequential sum of the block sums; the bits do not depend on the number
 *     of OpenMP threads.  The CG's element-wise loops split their index
 *     range over the threads; each element's arithmetic is unchanged.
 *   - SpMV: per row, ascending slot order, y = 0 then y = y + a*x per slot.
 *   - duplicate COO entries: merged into one CSR slot, values summed in
 *     input order, starting from the first value (not from 0.0).
 *   - built with -O2 -ffp-contract=off: every * and + is rounded on its own.
 *
 * Floating point is IEEE binary64 throughout.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_ARG 1
#define ORACLE_ERR_CSR 2
#define ORACLE_ERR_NOT_SPD 5
#define ORACLE_ERR_NONFINITE 6
#define ORACLE_ERR_NOT_SYMMETRIC 7
#define ORACLE_ERR_BREAKDOWN 8

#define DOT_BLOCK 4096

/* ------------------------------------------------------------------------ */
/* COO -> CSR                                                                */
/* ------------------------------------------------------------------------ */

typedef struct {
  int64_t row, col, pos;
} coo_key;

static int cmp_coo_key(const void* pa, const void* pb) {
  const coo_key* a = (const coo_key*)pa;
  const coo_key* b = (const coo_key*)pb;
  if (a->row != b->row) return a->row < b->row ? -1 : 1;
  if (a->col != b->col) return a->col < b->col ? -1 : 1;
  if (a->pos != b->pos) return a->pos < b->pos ? -1 : 1;
  return 0;
}

/*
 * Sparse matrix from coordinate triplets: sort the entries by (row, col),
 * ties kept in input order; equal (row, col) pairs become one stored slot.
 *
 *   rowptr[n+1]   out: row i's slots are rowptr[i] .. rowptr[i+1]-1
 *   col_out[<=m]  out: column of each slot, ascending inside a row
 *   perm[m]       out: perm[k] = slot that COO entry k was merged into
 * Returns the number of slots, or -1 if an index is out of range.
 */
int64_t oracle_csr_from_coo(int64_t n, int64_t m, const int64_t* row,
                            const int64_t* col, int64_t* rowptr,
                            int32_t* col_out, int64_t* perm) {
  for (int64_t k = 0; k < m; ++k)
    if (row[k] < 0 || row[k] >= n || col[k] < 0 || col[k] >= n) return -1;

  coo_key* keys = (coo_key*)malloc(sizeof(coo_key) * (size_t)(m > 0 ? m : 1));
  for (int64_t k = 0; k < m; ++k) {
    keys[k].row = row[k];
    keys[k].col = col[k];
    keys[k].pos = k;
  }
  /* (row, col, pos) is a total order, so qsort gives the one sorted result */
  qsort(keys, (size_t)m, sizeof(coo_key), cmp_coo_key);

  for (int64_t i = 0; i <= n; ++i) rowptr[i] = 0;
  int64_t slots = 0;
  for (int64_t s = 0; s < m; ++s) {
    int first = (s == 0) || keys[s].row != keys[s - 1].row ||
                keys[s].col != keys[s - 1].col;
    if (first) {
      col_out[slots] = (int32_t)keys[s].col;
      rowptr[keys[s].row + 1] += 1; /* count slots per row */
      slots += 1;
    }
    perm[keys[s].pos] = slots - 1;
  }
  for (int64_t i = 0; i < n; ++i) rowptr[i + 1] += rowptr[i];
  free(keys);
  return slots;
}

/*
 * Values of the merged matrix from COO values: every slot takes the values
 * of the COO entries mapped onto it, added in input order, starting from the
 * first one.
 */
void oracle_values_from_coo(int64_t m, int64_t nnz, const int64_t* perm,
                            const double* coo_val, double* vals) {
  char* seen = (char*)calloc((size_t)(nnz > 0 ? nnz : 1), 1);
  for (int64_t k = 0; k < m; ++k) {
    int64_t s = perm[k];
    if (!seen[s]) {
      vals[s] = coo_val[k];
      seen[s] = 1;
    } else {
      vals[s] = vals[s] + coo_val[k];
    }
  }
  free(seen);
}

/* Explicit transpose (A^T) of a CSR matrix; columns come out ascending. */
void oracle_transpose(int64_t n, const int64_t* rowptr, const int32_t* col,
                      const double* vals, int64_t* rowptr_t, int32_t* col_t,
                      double* vals_t) {
  int64_t nnz = rowptr[n];
  for (int64_t i = 0; i <= n; ++i) rowptr_t[i] = 0;
  for (int64_t k = 0; k < nnz; ++k) rowptr_t[col[k] + 1] += 1;
  for (int64_t i = 0; i < n; ++i) rowptr_t[i + 1] += rowptr_t[i];
  int64_t* fill = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) fill[i] = rowptr_t[i];
  /* walking rows in order puts each transposed row's columns in order */
  for (int64_t i = 0; i < n; ++i) {
    for (int64_t k = rowptr[i]; k < rowptr[i + 1]; ++k) {
      int64_t j = col[k];
      int64_t dst = fill[j]++;
      col_t[dst] = (int32_t)i;
      vals_t[dst] = vals[k];
    }
  }
  free(fill);
}

/* ------------------------------------------------------------------------ */
/* Vector kernels                                                            */
/* ------------------------------------------------------------------------ */

/* y = A x  (the sparse tensor's .matvec) */
void oracle_spmv(int64_t n, const int64_t* rowptr, const int32_t* col,
                 const double* vals, const double* x, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    double s = 0.0;
    for (int64_t k = rowptr[i]; k < rowptr[i + 1]; ++k) s = s + vals[k] * x[col[k]];
    y[i] = s;
  }
}

/* u . v, blocked so that the result is the same for any thread count */
double oracle_dot(int64_t n, const double* u, const double* v) {
  int64_t nb = (n + DOT_BLOCK - 1) / DOT_BLOCK;
  double* part = (double*)malloc(sizeof(double) * (size_t)(nb > 0 ? nb : 1));
#pragma omp parallel for schedule(static)
  for (int64_t b = 0; b < nb; ++b) {
    int64_t lo = b * DOT_BLOCK;
    int64_t hi = lo + DOT_BLOCK < n ? lo + DOT_BLOCK : n;
    double s = 0.0;
    for (int64_t i = lo; i < hi; ++i) s = s + u[i] * v[i];
    part[b] = s;
  }
  double total = 0.0;
  for (int64_t b = 0; b < nb; ++b) total = total + part[b];
  free(part);
  return total;
}

/* ------------------------------------------------------------------------ */
/* Conjugate gradient                                                        */
/* ------------------------------------------------------------------------ */

/* Long solves can report their own progress: every `progress_every`
 * completed iterations oracle_cg writes one line to stderr (0 = silent). */
static int64_t progress_every = 0;
void oracle_set_progress(int64_t every) { progress_every = every > 0 ? every : 0; }

typedef struct {
  int64_t iterations;
  double rr;        /* final recursive residual norm squared */
  double bb;        /* b . b */
  int32_t converged;
} oracle_cg_info;

/*
 * Solve A x = b for SPD A by plain CG.
 *   use_x0      : x holds the start vector on entry (else x0 = 0)
 *   hist_*      : optional (may be NULL), length >= maxit; per iteration k
 *                 alpha_k, beta_k and the residual norm squared after it.
 * Returns ORACLE_OK (converged or not), ORACLE_ERR_NOT_SPD or
 * ORACLE_ERR_NONFINITE; x then holds the last iterate.
 */
int oracle_cg(int64_t n, const int64_t* rowptr, const int32_t* col,
              const double* vals, const double* b, double* x, double tol,
              int64_t maxit, int use_x0, oracle_cg_info* info,
              double* hist_alpha, double* hist_beta, double* hist_rr) {
  size_t bytes = sizeof(double) * (size_t)(n > 0 ? n : 1);
  double* r = (double*)malloc(bytes);
  double* p = (double*)malloc(bytes);
  double* q = (double*)malloc(bytes);
  int status = ORACLE_OK;

  /* r0 = b - A x0 ; p0 = r0 */
  if (use_x0) {
    oracle_spmv(n, rowptr, col, vals, x, q);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) r[i] = b[i] - q[i];
  } else {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
      x[i] = 0.0;
      r[i] = b[i];
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) p[i] = r[i];

  double bb = oracle_dot(n, b, b);
  double rr = oracle_dot(n, r, r);
  double stop = (tol * tol) * bb;
  int64_t k = 0;
  if (!isfinite(bb) || !isfinite(rr)) {
    status = ORACLE_ERR_NONFINITE;
  } else {
    while (k < maxit) {
      if (rr <= stop) break;
      oracle_spmv(n, rowptr, col, vals, p, q); /* q = A p */
      double pq = oracle_dot(n, p, q);
      if (!isfinite(pq)) {
        status = ORACLE_ERR_NONFINITE;
        break;
      }
      if (!(pq > 0.0)) {
        status = ORACLE_ERR_NOT_SPD;
        break;
      }
      double alpha = rr / pq;
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < n; ++i) {
        x[i] = x[i] + alpha * p[i];
        r[i] = r[i] - alpha * q[i];
      }
      double rr_new = oracle_dot(n, r, r);
      if (!isfinite(rr_new)) {
        status = ORACLE_ERR_NONFINITE;
        break;
      }
      double beta = rr_new / rr;
#pragma omp parallel for schedule(static)
      for (int64_t i = 0; i < n; ++i) p[i] = r[i] + beta * p[i];
      if (hist_alpha) hist_alpha[k] = alpha;
      if (hist_beta) hist_beta[k] = beta;
      if (hist_rr) hist_rr[k] = rr_new;
      rr = rr_new;
      k = k + 1;
      if (progress_every && k % progress_every == 0) {
        fprintf(stderr, "[oracle cg] n=%lld iteration %lld of %lld, rr/bb %.3e\n",
                (long long)n, (long long)k, (long long)maxit, rr / bb);
        fflush(stderr);
      }
    }
  }
  info->iterations = k;
  info->rr = rr;
  info->bb = bb;
  info->converged = (status == ORACLE_OK && rr <= stop) ? 1 : 0;
  free(r);
  free(p);
  free(q);
  return status;
}

/* ------------------------------------------------------------------------ */
/* Adjoint of the linear solve                                               */
/* ------------------------------------------------------------------------ */

/*
 * Two stored values count as the same entry of a symmetric matrix when they
 * are equal or differ by at most 1e-12 of the larger magnitude: symmetric
 * expressions such as D A D round the two mirror entries differently by a
 * few ulps, far below what changes a CG solve.
 */
static int same_entry(double a, double b) {
  if (memcmp(&a, &b, sizeof(double)) == 0) return 1;
  double m = fabs(a) > fabs(b) ? fabs(a) : fabs(b);
  return fabs(a - b) <= 1e-12 * m;
}

/*
 * Backward pass of x = A^{-1} b for a loss L with g = dL/dx:
 *   A^T lambda = g          (solved by the same CG, on an explicit A^T)
 *   grad_b     = lambda
 *   grad_A     = -lambda_i x_j for every stored slot (i, j), nothing else.
 * Returns the CG status; ORACLE_ERR_NOT_SYMMETRIC if A^T differs from A
 * (pattern, or values beyond same_entry) (CG needs a symmetric matrix; the
 * solve is still done on A^T).
 */
int oracle_adjoint(int64_t n, const int64_t* rowptr, const int32_t* col,
                   const double* vals, const double* x, const double* g,
                   double* grad_b, double* grad_vals, double tol,
                   int64_t maxit, oracle_cg_info* info) {
  int64_t nnz = rowptr[n];
  int64_t* rowptr_t = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n + 1));
  int32_t* col_t = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
  double* vals_t = (double*)malloc(sizeof(double) * (size_t)(nnz > 0 ? nnz : 1));
  oracle_transpose(n, rowptr, col, vals, rowptr_t, col_t, vals_t);
  int symmetric = 1;
  for (int64_t i = 0; i <= n && symmetric; ++i)
    if (rowptr_t[i] != rowptr[i]) symmetric = 0;
  for (int64_t k = 0; k < nnz && symmetric; ++k)
    if (col_t[k] != col[k] || !same_entry(vals_t[k], vals[k])) symmetric = 0;

  int status = oracle_cg(n, rowptr_t, col_t, vals_t, g, grad_b, tol, maxit, 0,
                         info, NULL, NULL, NULL);
  const double* lambda = grad_b;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    for (int64_t k = rowptr[i]; k < rowptr[i + 1]; ++k)
      grad_vals[k] = -(lambda[i] * x[col[k]]);

  free(rowptr_t);
  free(col_t);
  free(vals_t);
  if (status == ORACLE_OK && !symmetric) status = ORACLE_ERR_NOT_SYMMETRIC;
  return status;
}

/* grad_vals[k] = -lambda_i x_j on every stored slot (the last step above) */
void oracle_pattern_grad(int64_t n, const int64_t* rowptr, const int32_t* col,
                         const double* lambda, const double* x,
                         double* grad_vals) {
  for (int64_t i = 0; i < n; ++i)
    for (int64_t k = rowptr[i]; k < rowptr[i + 1]; ++k)
      grad_vals[k] = -(lambda[i] * x[col[k]]);
}

/* ------------------------------------------------------------------------ */
/* Jacobi-preconditioned CG                                                  */
/* ------------------------------------------------------------------------ */

/*
 * Solve A x = b by CG preconditioned with M = diag(A), the preconditioner
 * the pages name for the PyTorch-native backend (Significance / limitations).
 * Textbook preconditioned CG, step by step:
 *   r0 = b - A x0;  z0 = r0 / d (elementwise, d = the stored diagonal);
 *   p0 = z0;  then per iteration
 *   q = A p;  alpha = (r.z) / (p.q);  x += alpha p;  r -= alpha q;
 *   z = r / d;  beta = (r.z)_new / (r.z);  p = z + beta p.
 * The stopping test is the plain CG one, on the residual itself:
 * r.r <= (tol*tol) * b.b before each iteration.  A missing or non-positive
 * diagonal entry (impossible for an SPD matrix) returns ORACLE_ERR_NOT_SPD
 * before any iteration.  hist_rr receives r.r after each iteration, hist_rz
 * (optional) r.z.
 */
int oracle_pcg_jacobi(int64_t n, const int64_t* rowptr, const int32_t* col,
                      const double* vals, const double* b, double* x, double tol,
                      int64_t maxit, int use_x0, oracle_cg_info* info,
                      double* hist_alpha, double* hist_beta, double* hist_rr,
                      double* hist_rz) {
  size_t bytes = sizeof(double) * (size_t)(n > 0 ? n : 1);
  double* r = (double*)malloc(bytes);
  double* z = (double*)malloc(bytes);
  double* p = (double*)malloc(bytes);
  double* q = (double*)malloc(bytes);
  double* d = (double*)malloc(bytes);
  int status = ORACLE_OK;
  int64_t k = 0;
  double bb = 0.0, rr = 0.0, rz = 0.0, stop = 0.0;

  /* the diagonal: the stored slot (i, i) of each row */
  for (int64_t i = 0; i < n; ++i) {
    d[i] = 0.0;
    for (int64_t s = rowptr[i]; s < rowptr[i + 1]; ++s)
      if (col[s] == i) d[i] = vals[s];
    if (!(d[i] > 0.0)) status = ORACLE_ERR_NOT_SPD;
  }
  if (status == ORACLE_OK) {
    if (use_x0) {
      oracle_spmv(n, rowptr, col, vals, x, q);
      for (int64_t i = 0; i < n; ++i) r[i] = b[i] - q[i];
    } else {
      for (int64_t i = 0; i < n; ++i) {
        x[i] = 0.0;
        r[i] = b[i];
      }
    }
    for (int64_t i = 0; i < n; ++i) {
      z[i] = r[i] / d[i];
      p[i] = z[i];
    }
    bb = oracle_dot(n, b, b);
    rr = oracle_dot(n, r, r);
    rz = oracle_dot(n, r, z);
    stop = (tol * tol) * bb;
    if (!isfinite(bb) || !isfinite(rr) || !isfinite(rz)) status = ORACLE_ERR_NONFINITE;
  } else if (!use_x0) {
    for (int64_t i = 0; i < n; ++i) x[i] = 0.0;
  }
  while (status == ORACLE_OK && k < maxit) {
    if (rr <= stop) break;
    oracle_spmv(n, rowptr, col, vals, p, q); /* q = A p */
    double pq = oracle_dot(n, p, q);
    if (!isfinite(pq)) {
      status = ORACLE_ERR_NONFINITE;
      break;
    }
    if (!(pq > 0.0)) {
      status = ORACLE_ERR_NOT_SPD;
      break;
    }
    double alpha = rz / pq;
    for (int64_t i = 0; i < n; ++i) {
      x[i] = x[i] + alpha * p[i];
      r[i] = r[i] - alpha * q[i];
    }
    for (int64_t i = 0; i < n; ++i) z[i] = r[i] / d[i];
    double rr_new = oracle_dot(n, r, r);
    double rz_new = oracle_dot(n, r, z);
    if (!isfinite(rr_new) || !isfinite(rz_new)) {
      status = ORACLE_ERR_NONFINITE;
      break;
    }
    double beta = rz_new / rz;
    for (int64_t i = 0; i < n; ++i) p[i] = z[i] + beta * p[i];
    if (hist_alpha) hist_alpha[k] = alpha;
    if (hist_beta) hist_beta[k] = beta;
    if (hist_rr) hist_rr[k] = rr_new;
    if (hist_rz) hist_rz[k] = rz_new;
    rr = rr_new;
    rz = rz_new;
    k = k + 1;
  }
  info->iterations = k;
  info->rr = rr;
  info->bb = bb;
  info->converged = (status == ORACLE_OK && rr <= stop) ? 1 : 0;
  free(r);
  free(z);
  free(p);
  free(q);
  free(d);
  return status;
}

/* The adjoint of a Jacobi-PCG solve: the same steps as oracle_adjoint, with
 * lambda from oracle_pcg_jacobi on the explicit A^T. */
int oracle_adjoint_jacobi(int64_t n, const int64_t* rowptr, const int32_t* col,
                          const double* vals, const double* x, const double* g,
                          double* grad_b, double* grad_vals, double tol,
                          int64_t maxit, oracle_cg_info* info) {
  int64_t nnz = rowptr[n];
  int64_t* rowptr_t = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n + 1));
  int32_t* col_t = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
  double* vals_t = (double*)malloc(sizeof(double) * (size_t)(nnz > 0 ? nnz : 1));
  oracle_transpose(n, rowptr, col, vals, rowptr_t, col_t, vals_t);
  int symmetric = 1;
  for (int64_t i = 0; i <= n && symmetric; ++i)
    if (rowptr_t[i] != rowptr[i]) symmetric = 0;
  for (int64_t k = 0; k < nnz && symmetric; ++k)
    if (col_t[k] != col[k] || !same_entry(vals_t[k], vals[k])) symmetric = 0;
  int status = oracle_pcg_jacobi(n, rowptr_t, col_t, vals_t, g, grad_b, tol, maxit, 0,
                                 info, NULL, NULL, NULL, NULL);
  oracle_pattern_grad(n, rowptr, col, grad_b, x, grad_vals);
  free(rowptr_t);
  free(col_t);
  free(vals_t);
  if (status == ORACLE_OK && !symmetric) status = ORACLE_ERR_NOT_SYMMETRIC;
  return status;
}

/* ------------------------------------------------------------------------ */
/* Backward pass of the product y = A x                                      */
/* ------------------------------------------------------------------------ */

/*
 * For a loss L with g = dL/dy (Methodology 1, the differentiable .matvec):
 *   grad_x    = A^T g                   (explicit transpose, then SpMV)
 *   grad_vals = g_i x_j on every stored slot (i, j), nothing else.
 */
void oracle_matvec_grad(int64_t n, const int64_t* rowptr, const int32_t* col,
                        const double* vals, const double* x, const double* g,
                        double* grad_x, double* grad_vals) {
  int64_t nnz = rowptr[n];
  int64_t* rowptr_t = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n + 1));
  int32_t* col_t = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
  double* vals_t = (double*)malloc(sizeof(double) * (size_t)(nnz > 0 ? nnz : 1));
  oracle_transpose(n, rowptr, col, vals, rowptr_t, col_t, vals_t);
  oracle_spmv(n, rowptr_t, col_t, vals_t, g, grad_x);
  for (int64_t i = 0; i < n; ++i)
    for (int64_t k = rowptr[i]; k < rowptr[i + 1]; ++k) grad_vals[k] = g[i] * x[col[k]];
  free(rowptr_t);
  free(col_t);
  free(vals_t);
}

/* ------------------------------------------------------------------------ */
/* Lanczos (the .eigsh of Methodology 1)                                     */
/* ------------------------------------------------------------------------ */

/*
 * The pages name .eigsh (Methodology 1) but not its algorithm; the reading
 * taken is the textbook one for a few extreme eigenpairs of a sparse
 * symmetric matrix through products with A alone:
 * m steps of the Lanczos process for symmetric A from the start vector v0,
 * with full reorthogonalisation by classical Gram-Schmidt applied twice:
 *   v_0 = v0 / |v0|;  for j = 0 .. m-1:
 *     w = A v_j;
 *     h = V_j^T w, w = w - V_j h;  h' = V_j^T w, w = w - V_j h'
 *       (V_j = [v_0 .. v_j]; dot products and updates in index order);
 *     alpha_j = h_j + h'_j;  beta_j = |w|;  v_{j+1} = w / beta_j.
 * T = tridiag(beta, alpha, beta) is then the matrix of A in the orthonormal
 * Krylov basis; its eigenpairs give the Ritz pairs (done by the caller).
 * Stops after step j when beta_j <= 1e-10 |A v_j| (the Krylov space is an
 * invariant subspace: what is left of w is rounding); returns the number of
 * completed steps.  V receives v_0 .. v_steps, row-major [steps+1][n] (room
 * for m+1 vectors).
 */
int64_t oracle_lanczos(int64_t n, const int64_t* rowptr, const int32_t* col,
                       const double* vals, const double* v0, int64_t m, double* alpha,
                       double* beta, double* V) {
  double* w = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double* h = (double*)malloc(sizeof(double) * (size_t)(m > 0 ? m + 1 : 1));
  double nv = sqrt(oracle_dot(n, v0, v0));
  for (int64_t i = 0; i < n; ++i) V[i] = v0[i] / nv;
  int64_t steps = 0;
  for (int64_t j = 0; j < m; ++j) {
    const double* vj = V + j * n;
    oracle_spmv(n, rowptr, col, vals, vj, w);
    double wn = sqrt(oracle_dot(n, w, w));
    double a = 0.0;
    for (int pass = 0; pass < 2; ++pass) {
      for (int64_t l = 0; l <= j; ++l) h[l] = oracle_dot(n, V + l * n, w);
      for (int64_t i = 0; i < n; ++i) {
        double s = w[i];
        for (int64_t l = 0; l <= j; ++l) s = s - V[l * n + i] * h[l];
        w[i] = s;
      }
      a = a + h[j];
    }
    alpha[j] = a;
    double b = sqrt(oracle_dot(n, w, w));
    beta[j] = b;
    steps = j + 1;
    if (!(b > 1e-10 * wn)) break;
    for (int64_t i = 0; i < n; ++i) V[(j + 1) * n + i] = w[i] / b;
  }
  free(w);
  free(h);
  return steps;
}

/* Hellmann-Feynman (Methodology 2, eigenvalue problems): for a simple
 * eigenvalue with unit eigenvector v, d lambda / d A_ij = v_i v_j, on every
 * stored slot (i, j) and nothing else. */
void oracle_eig_grad(int64_t n, const int64_t* rowptr, const int32_t* col, const double* v,
                     double* grad_vals) {
  for (int64_t i = 0; i < n; ++i)
    for (int64_t k = rowptr[i]; k < rowptr[i + 1]; ++k) grad_vals[k] = v[i] * v[col[k]];
}

/* ------------------------------------------------------------------------ */
/* BiCGStab (a CPU backend solver of Methodology 1) and its adjoint          */
/* ------------------------------------------------------------------------ */

/*
 * Solve A x = b for a general (non-symmetric) A by BiCGStab (van der Vorst),
 * without preconditioner.  The pages name the solver (SciPy and Eigen CPU
 * backends) but not its variant; the reading taken is the textbook one:
 *   r = b - A x0 (x0 = 0 unless use_x0), rhat = r, p = v = 0,
 *   rho_prev = alpha = omega = 1;  each iteration:
 *     rho = rhat . r                       (zero: breakdown)
 *     beta = (rho / rho_prev) (alpha / omega)
 *     p = r + beta (p - omega v)
 *     v = A p ; alpha = rho / (rhat . v)   (rhat . v zero: breakdown)
 *     s = r - alpha v
 *     if s . s <= tol^2 b . b: x = x + alpha p, done (a counted iteration)
 *     t = A s ; omega = (t . s) / (t . t)  (t . t or omega zero: breakdown)
 *     x = (x + alpha p) + omega s ; r = s - omega t
 * and it stops, as CG, when the recursive residual satisfies
 * r . r <= tol^2 b . b before an iteration, or after maxit iterations.
 * Returns ORACLE_OK (converged or not), ORACLE_ERR_BREAKDOWN or
 * ORACLE_ERR_NONFINITE; x holds the last iterate.  hist_* (may be NULL,
 * length >= maxit): rho, alpha, omega and the residual norm squared after
 * each iteration (s . s and omega = 0 for a half-step finish).
 */
int oracle_bicgstab(int64_t n, const int64_t* rowptr, const int32_t* col,
                    const double* vals, const double* b, double* x, double tol,
                    int64_t maxit, int use_x0, oracle_cg_info* info, double* hist_rho,
                    double* hist_alpha, double* hist_omega, double* hist_rr) {
  size_t bytes = sizeof(double) * (size_t)(n > 0 ? n : 1);
  double* r = (double*)malloc(bytes);
  double* rh = (double*)malloc(bytes);
  double* p = (double*)malloc(bytes);
  double* v = (double*)malloc(bytes);
  double* sv = (double*)malloc(bytes);
  double* t = (double*)malloc(bytes);
  int status = ORACLE_OK;
  if (use_x0) {
    oracle_spmv(n, rowptr, col, vals, x, v);
    for (int64_t i = 0; i < n; ++i) r[i] = b[i] - v[i];
  } else {
    for (int64_t i = 0; i < n; ++i) {
      x[i] = 0.0;
      r[i] = b[i];
    }
  }
  for (int64_t i = 0; i < n; ++i) {
    rh[i] = r[i];
    p[i] = 0.0;
    v[i] = 0.0;
  }
  double bb = oracle_dot(n, b, b);
  double rr = oracle_dot(n, r, r);
  double stop = (tol * tol) * bb;
  double rho_prev = 1.0, alpha = 1.0, omega = 1.0;
  int64_t k = 0;
  int done = 0;
  if (!isfinite(bb) || !isfinite(rr)) status = ORACLE_ERR_NONFINITE;
  while (status == ORACLE_OK && !done && k < maxit && rr > stop) {
    double rho = oracle_dot(n, rh, r);
    if (!isfinite(rho)) { status = ORACLE_ERR_NONFINITE; break; }
    if (rho == 0.0) { status = ORACLE_ERR_BREAKDOWN; break; }
    double beta = (rho / rho_prev) * (alpha / omega);
    for (int64_t i = 0; i < n; ++i) p[i] = r[i] + beta * (p[i] - omega * v[i]);
    oracle_spmv(n, rowptr, col, vals, p, v);
    double rv = oracle_dot(n, rh, v);
    if (!isfinite(rv)) { status = ORACLE_ERR_NONFINITE; break; }
    if (rv == 0.0) { status = ORACLE_ERR_BREAKDOWN; break; }
    alpha = rho / rv;
    for (int64_t i = 0; i < n; ++i) sv[i] = r[i] - alpha * v[i];
    double ss = oracle_dot(n, sv, sv);
    if (!isfinite(ss)) { status = ORACLE_ERR_NONFINITE; break; }
    if (hist_rho) hist_rho[k] = rho;
    if (hist_alpha) hist_alpha[k] = alpha;
    if (ss <= stop) {
      for (int64_t i = 0; i < n; ++i) x[i] = x[i] + alpha * p[i];
      if (hist_omega) hist_omega[k] = 0.0;
      if (hist_rr) hist_rr[k] = ss;
      rr = ss;
      k = k + 1;
      done = 1;
      break;
    }
    oracle_spmv(n, rowptr, col, vals, sv, t);
    double tt = oracle_dot(n, t, t);
    double ts = oracle_dot(n, t, sv);
    if (!isfinite(tt) || !isfinite(ts)) { status = ORACLE_ERR_NONFINITE; break; }
    if (tt == 0.0) { status = ORACLE_ERR_BREAKDOWN; break; }
    omega = ts / tt;
    for (int64_t i = 0; i < n; ++i) {
      x[i] = (x[i] + alpha * p[i]) + omega * sv[i];
      r[i] = sv[i] - omega * t[i];
    }
    rr = oracle_dot(n, r, r);
    if (hist_omega) hist_omega[k] = omega;
    if (hist_rr) hist_rr[k] = rr;
    k = k + 1;
    if (!isfinite(rr)) { status = ORACLE_ERR_NONFINITE; break; }
    if (omega == 0.0) { status = ORACLE_ERR_BREAKDOWN; break; }
    rho_prev = rho;
  }
  info->iterations = k;
  info->rr = rr;
  info->bb = bb;
  info->converged = (status == ORACLE_OK && rr <= stop) ? 1 : 0;
  free(r);
  free(rh);
  free(p);
  free(v);
  free(sv);
  free(t);
  return status;
}

/*
 * Backward pass of x = A^{-1} b (Methodology 2, linear systems) for a
 * general A: A^T lambda = g solved by the same BiCGStab on an explicit A^T;
 * grad_b = lambda, grad_vals[k] = -lambda_i x_j on the stored slots.
 */
int oracle_adjoint_bicgstab(int64_t n, const int64_t* rowptr, const int32_t* col,
                            const double* vals, const double* x, const double* g,
                            double* grad_b, double* grad_vals, double tol, int64_t maxit,
                            oracle_cg_info* info) {
  int64_t nnz = rowptr[n];
  int64_t* rowptr_t = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n + 1));
  int32_t* col_t = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nnz > 0 ? nnz : 1));
  double* vals_t = (double*)malloc(sizeof(double) * (size_t)(nnz > 0 ? nnz : 1));
  oracle_transpose(n, rowptr, col, vals, rowptr_t, col_t, vals_t);
  int status = oracle_bicgstab(n, rowptr_t, col_t, vals_t, g, grad_b, tol, maxit, 0, info,
                               NULL, NULL, NULL, NULL);
  oracle_pattern_grad(n, rowptr, col, grad_b, x, grad_vals);
  free(rowptr_t);
  free(col_t);
  free(vals_t);
  return status;
}

/* ------------------------------------------------------------------------ */
/* Locality ordering of the unknowns (not from the pages)                    */
/* ------------------------------------------------------------------------ */

/*
 * Breadth-first visit of the pattern's graph (an edge i -> j for every
 * stored slot (i, j), j != i) from `start`, restricted to unvisited nodes:
 * nodes are appended to order[] at *len in the order they are first reached,
 * each node's neighbours taken in its row's (ascending) column order.
 * dist[v] receives the number of edges from start.  Returns the last node
 * appended's distance (the depth of the visit).
 */
static int64_t bfs_visit(const int64_t* rowptr, const int32_t* col, int64_t start,
                         int64_t* order, int64_t* len, int64_t* dist) {
  int64_t head = *len;
  order[(*len)++] = start;
  dist[start] = 0;
  int64_t depth = 0;
  while (head < *len) {
    int64_t v = order[head++];
    for (int64_t k = rowptr[v]; k < rowptr[v + 1]; ++k) {
      int64_t u = col[k];
      if (dist[u] >= 0) continue;
      dist[u] = dist[v] + 1;
      if (dist[u] > depth) depth = dist[u];
      order[(*len)++] = u;
    }
  }
  return depth;
}

/*
 * A bandwidth-reducing order of the unknowns: the breadth-first order of the
 * pattern's graph (Cuthill-McKee's level structure, with each node's
 * children in column order instead of by degree) from a pseudo-peripheral
 * start node.
 *   s0 = the smallest index of largest row length (stored slots);
 *   s1 = the smallest index among the nodes farthest from s0 (in edges);
 *   a visit from s1, then from the smallest unvisited index while nodes
 *   remain (every connected piece in turn).
 * order[t] = the original index of the unknown at position t.
 */
void oracle_bfs_order(int64_t n, const int64_t* rowptr, const int32_t* col, int64_t* order) {
  if (n <= 0) return;
  int64_t* dist = (int64_t*)malloc(sizeof(int64_t) * (size_t)n);
  int64_t s0 = 0;
  for (int64_t i = 1; i < n; ++i)
    if (rowptr[i + 1] - rowptr[i] > rowptr[s0 + 1] - rowptr[s0]) s0 = i;
  for (int64_t i = 0; i < n; ++i) dist[i] = -1;
  int64_t len = 0;
  int64_t depth = bfs_visit(rowptr, col, s0, order, &len, dist);
  int64_t s1 = -1;
  for (int64_t t = 0; t < len; ++t)
    if (dist[order[t]] == depth && (s1 < 0 || order[t] < s1)) s1 = order[t];
  for (int64_t i = 0; i < n; ++i) dist[i] = -1;
  len = 0;
  bfs_visit(rowptr, col, s1, order, &len, dist);
  for (int64_t i = 0; i < n; ++i)
    if (dist[i] < 0) bfs_visit(rowptr, col, i, order, &len, dist);
  free(dist);
}

/*
 * The symmetrically permuted matrix B = P A P^T of an order (B's row t is
 * A's row order[t], its columns renumbered by pos[order[t]] = t and sorted
 * ascending).  src[s] receives the slot of A that B's slot s holds.
 */
void oracle_permute(int64_t n, const int64_t* rowptr, const int32_t* col, const double* vals,
                    const int64_t* order, int64_t* rowptr_p, int32_t* col_p, double* vals_p,
                    int64_t* src) {
  int64_t* pos = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t t = 0; t < n; ++t) pos[order[t]] = t;
  rowptr_p[0] = 0;
  for (int64_t t = 0; t < n; ++t)
    rowptr_p[t + 1] = rowptr_p[t] + (rowptr[order[t] + 1] - rowptr[order[t]]);
  for (int64_t t = 0; t < n; ++t) {
    int64_t i = order[t], a = rowptr_p[t];
    int64_t len = rowptr[i + 1] - rowptr[i];
    /* insertion sort of the row's slots by new column */
    for (int64_t q = 0; q < len; ++q) {
      int64_t k = rowptr[i] + q;
      int64_t c = pos[col[k]];
      int64_t w = a + q;
      while (w > a && col_p[w - 1] > c) {
        col_p[w] = col_p[w - 1];
        src[w] = src[w - 1];
        --w;
      }
      col_p[w] = (int32_t)c;
      src[w] = k;
    }
    for (int64_t q = 0; q < len; ++q) vals_p[a + q] = vals[src[a + q]];
  }
  free(pos);
}

/* ------------------------------------------------------------------------ */
/* Threads                                                                   */
/* ------------------------------------------------------------------------ */
#ifdef _OPENMP
#include <omp.h>
void oracle_set_threads(int t) { omp_set_num_threads(t > 0 ? t : 1); }
int oracle_get_threads(void) { return omp_get_max_threads(); }
#else
void oracle_set_threads(int t) { (void)t; }
int oracle_get_threads(void) { return 1; }
#endif
