/*
 * sla.h -- C ABI of the MI355X (gfx950) sparse CG solver with an adjoint
 * backward pass.
 *
 * The operations are those of the torch-sla explainer (gist.science, arXiv
 * 2601.13994), technical summary:
 *   - Methodology 1 (unified backend abstraction): a sparse tensor with a
 *     .matvec and a .solve; a SparseTensor is one matrix or a batch of
 *     matrices sharing one sparsity pattern.
 *   - Methodology 2 (adjoint differentiation framework), linear systems: the
 *     backward pass of x = A^{-1} b solves A^T lambda = dL/dx, returns
 *     dL/db = lambda and dL/dA = -lambda_i x_j only on the sparsity pattern;
 *     the graph is O(1) nodes and the memory O(n + nnz), whatever the number
 *     of solver iterations.
 *   - Experimental results: the CG backend on 2D Poisson systems.
 * The solver is plain (unpreconditioned) conjugate gradients for symmetric
 * positive definite A, so A^T = A and the adjoint reuses A.
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers unless the name ends in _host.
 *   - Floating point is IEEE binary64.  Column indices are int32 (n < 2^31);
 *     row pointers are int32 or int64 (sla_index), chosen per matrix.
 *   - Batched arrays are system-major: values [batch][nnz], vectors
 *     [batch][n], contiguous.
 *   - Work is enqueued on `stream` (0 = the null stream).  Calls that fill a
 *     _host output synchronise `stream` before returning; the others are
 *     asynchronous.
 *   - No C++ exception crosses this boundary.  Every call returns an
 *     sla_status; on failure sla_last_error() gives a message (per thread).
 *     Arguments are checked before anything is launched.
 *   - A handle is not thread-safe: calls on one handle must not overlap.
 */
#ifndef SLA_H_
#define SLA_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLA_OK = 0,
  SLA_ERR_ARG = 1,        /* bad argument (null pointer, size, flag)          */
  SLA_ERR_CSR = 2,        /* malformed pattern (range, order, duplicates)     */
  SLA_ERR_OOM = 3,        /* device allocation failed                          */
  SLA_ERR_DEVICE = 4,     /* a HIP call failed                                  */
  SLA_ERR_NOT_SPD = 5,    /* CG breakdown: p.Ap <= 0                            */
  SLA_ERR_NONFINITE = 6,  /* b.b, p.Ap or r.r is not finite                     */
  SLA_ERR_KRYLOV = 7,     /* eigsh: the Lanczos process ended (an invariant
                             subspace was reached) after fewer than k steps   */
  SLA_ERR_BREAKDOWN = 8,  /* BiCGStab: rhat.r, rhat.v or t.t became 0          */
  SLA_ERR_NOT_SYMMETRIC = 9 /* CG: the pattern (solve, adjoint) or the values
                             (adjoint) are not symmetric                      */
} sla_status;

typedef enum { SLA_I32 = 4, SLA_I64 = 8 } sla_index;

/* Result of one solve (one system of a batch). */
typedef struct {
  int64_t iterations;   /* completed CG iterations (alpha updates)            */
  double rel_residual;  /* sqrt(rr / bb), rr the recursive residual norm^2    */
  int32_t converged;    /* rr <= (tol*tol) * bb                               */
  int32_t status;       /* sla_status of this system                          */
} sla_cg_info;

enum {
  SLA_FLAG_X0 = 1,      /* x holds the start vector (default: x0 = 0)        */
  SLA_FLAG_HISTORY = 2, /* record alpha, beta, rr of every iteration         */
  SLA_FLAG_JACOBI = 4   /* Jacobi preconditioning, M = diag(A) (see below)   */
};

/* Opaque matrix handle: the sparsity pattern (owned by the library, copied
 * or built at creation), the values -- either a copy the handle owns
 * (sla_csr_load_values) or a caller's array it reads in place
 * (sla_csr_set_values) -- and the solver workspace. */
typedef struct sla_csr_s* sla_csr;

/*
 * Build a CSR pattern from COO coordinates (Methodology 1: SparseTensor).
 *   n            matrix order (square), 1 <= n < 2^31
 *   nnz_coo      number of triplets, 0 <= nnz_coo < 2^32
 *   coo_idx      width of coo_row / coo_col entries (SLA_I32 or SLA_I64)
 *   rowptr_idx   width of the CSR row pointer to build (SLA_I32 needs the
 *                merged nnz < 2^31)
 * The result is the unique sorted pattern: entries ordered by (row, col);
 * equal (row, col) pairs merge into one slot; explicit zeros are kept.  It is
 * bit-identical on every run.  sla_csr_values_from_coo maps values onto it.
 * Errors: SLA_ERR_ARG (sizes, nulls), SLA_ERR_CSR (an index out of range),
 * SLA_ERR_OOM.  *out is set only on SLA_OK.  Synchronises `stream`.
 */
sla_status sla_csr_create(int64_t n, int64_t nnz_coo, sla_index coo_idx,
                          const void* coo_row, const void* coo_col,
                          sla_index rowptr_idx, hipStream_t stream, sla_csr* out);

/*
 * Take a CSR pattern as given: rowptr [n+1] (rowptr_idx wide), col [nnz].
 * Validated (rowptr[0] = 0, rowptr[n] = nnz, non-decreasing; columns in range
 * and strictly increasing inside each row) and copied.  Errors: SLA_ERR_ARG,
 * SLA_ERR_CSR, SLA_ERR_OOM.  Synchronises `stream`.
 */
sla_status sla_csr_create_from_csr(int64_t n, int64_t nnz, sla_index rowptr_idx,
                                   const void* rowptr, const int32_t* col,
                                   hipStream_t stream, sla_csr* out);

/* Free the handle and everything the library allocated for it (the sparse
 * tensor's lifetime, Methodology 1).  Waits for the device first.  NULL is
 * accepted. */
sla_status sla_csr_destroy(sla_csr A);

/* Sizes of the sparse tensor (Methodology 1): order, stored slots, COO
 * triplets it was built from (0 if from CSR), row-pointer width.  Any output
 * pointer may be NULL. */
sla_status sla_csr_get_info(sla_csr A, int64_t* n_host, int64_t* nnz_host,
                            int64_t* nnz_coo_host, sla_index* rowptr_idx_host);

/* Borrowed device views of the pattern (Methodology 1: the shared sparsity
 * pattern), valid until destroy.  perm[k] is the CSR slot COO triplet k was
 * merged into; NULL for a handle made from CSR.  sla_csr_arrays gives the
 * same views plus the bound values. */
sla_status sla_csr_pattern(sla_csr A, const void** rowptr_host,
                           const int32_t** col_host, const int64_t** perm_host);

/* Copy the pattern (Methodology 1) into caller buffers (any may be NULL):
 * rowptr_out [n+1] of the handle's row-pointer width, col_out [nnz],
 * perm_out [nnz_coo] (COO-built handles only).  Asynchronous on `stream`. */
sla_status sla_csr_copy_pattern(sla_csr A, void* rowptr_out, int32_t* col_out,
                                int64_t* perm_out, hipStream_t stream);

/*
 * CSR values from COO values (Methodology 1: a SparseTensor built from
 * coordinates): vals[s][slot] = the COO values mapped onto that slot, added
 * in input order starting from the first one.  coo_val [batch][nnz_coo],
 * vals [batch][nnz], caller-owned device memory.  Needs a COO-built handle.
 * Asynchronous.
 */
sla_status sla_csr_values_from_coo(sla_csr A, const double* coo_val, double* vals,
                                   int64_t batch, hipStream_t stream);

/* Gradient of COO values from the gradient of CSR values (Methodology 2:
 * the matrix gradient lives on the pattern; a merged duplicate is one
 * parameter of the slot): grad_coo[s][k] = grad_vals[s][perm[k]].
 * Asynchronous. */
sla_status sla_csr_grad_to_coo(sla_csr A, const double* grad_vals, double* grad_coo,
                               int64_t batch, hipStream_t stream);

/*
 * Bind the values (Methodology 1: a SparseTensor is one matrix or a batch of
 * matrices on one pattern): vals [batch][nnz] in CSR slot order, owned by the
 * caller, read in place by every later spmv / solve / adjoint until re-bound.
 * The caller keeps the array alive and unchanged while work that reads it is
 * queued.  batch >= 1.  A copy the handle owns (sla_csr_load_values) stays
 * allocated; passing its pointer (from sla_csr_arrays) binds it again.
 */
sla_status sla_csr_set_values(sla_csr A, const double* vals, int64_t batch);

/*
 * Copy values into an array the handle owns and bind it (Methodology 1: the
 * sparse tensor holds its values; a batch shares the pattern).  order
 * SLA_VALUES_CSR: vals [batch][nnz] in CSR slot order; SLA_VALUES_COO: vals
 * [batch][nnz_coo] in the COO triplet order the handle was built from,
 * merged into the slots as sla_csr_values_from_coo does (COO-built handles
 * only).  The copy is enqueued on `stream`; the caller's array may be freed
 * once that work is done.  The owned array lives until the handle is
 * destroyed or a load with another batch size replaces it; sla_csr_arrays
 * gives its device address, where callers may update values in place
 * between calls (a training step, say).  Errors: SLA_ERR_ARG, SLA_ERR_OOM.
 */
enum { SLA_VALUES_CSR = 0, SLA_VALUES_COO = 1 };
sla_status sla_csr_load_values(sla_csr A, const double* vals, int64_t batch, int order,
                               hipStream_t stream);

/*
 * Borrowed device views of the handle's arrays (any output may be NULL),
 * valid until the handle is destroyed (vals: until the values are re-bound
 * or reloaded): rowptr [n+1] (of the handle's row-pointer width), col [nnz],
 * the bound values [batch][nnz] (the handle's own copy after
 * sla_csr_load_values, else the caller's array; NULL if none is bound), and
 * perm [nnz_coo] (COO triplet -> slot; NULL for a handle made from CSR).
 */
sla_status sla_csr_arrays(sla_csr A, const void** rowptr_host, const int32_t** col_host,
                          double** vals_host, const int64_t** perm_host);

/*
 * Device memory held by the library on the current device, over every handle
 * and workspace: *live_host the bytes allocated now, *peak_host the most at
 * any time since the process started or the last reset (either may be NULL);
 * reset_peak != 0 then sets the peak to the live bytes.  Pinned host memory
 * (a few small per-handle buffers) is not counted.  Compare with the adjoint
 * memory the pages report (Experimental results, memory efficiency).
 */
sla_status sla_memory_usage(int64_t* live_host, int64_t* peak_host, int reset_peak);

/* y[s] = A_s x[s] for every system s of the bound batch: the sparse
 * tensor's .matvec (Methodology 1, unified backend abstraction).  Row i is
 * summed in ascending slot order, y = 0 then y = y + a x, each product and
 * sum rounded on its own.  x, y [batch][n] device memory.  Asynchronous. */
sla_status sla_spmv(sla_csr A, const double* x, double* y, hipStream_t stream);

/*
 * y[s] = A_s^T x[s] for every system s of the bound batch: the transposed
 * product the backward pass of .matvec needs (Methodology 1).  The first call
 * builds the transposed pattern and keeps it with the handle (a COO -> CSR
 * build of the slots with rows and columns swapped, with a map from each of
 * its slots to the slot of A it transposes; about 24 more bytes per slot);
 * the bound values are read in place through that map.  Row j of A^T is
 * summed in ascending original row i, as an explicit transpose followed by
 * sla_spmv would, bit for bit.  x, y [batch][n], device memory.
 */
sla_status sla_spmv_transpose(sla_csr A, const double* x, double* y, hipStream_t stream);

/*
 * Backward pass of y = A x (Methodology 1, the differentiable .matvec) for a
 * loss L with grad_y = dL/dy: grad_x = A^T grad_y [batch][n] (may be NULL:
 * not computed) and grad_vals[k] = grad_y_i x_j for every stored slot
 * k = (i, j) [batch][nnz] (may be NULL), nothing for absent entries.
 */
sla_status sla_matvec_grad(sla_csr A, const double* x, const double* grad_y, double* grad_x,
                           double* grad_vals, hipStream_t stream);

/*
 * Solve A x = b by CG (bound batch must be 1): the sparse tensor's .solve
 * with the PyTorch-native iterative (CG) backend (Methodology 1), as
 * benchmarked on 2D Poisson systems (Experimental results).  CG needs a
 * symmetric positive definite A: a pattern that is not symmetric (checked
 * once per handle) returns SLA_ERR_NOT_SYMMETRIC before any iteration, x
 * untouched.  x0 = 0 unless SLA_FLAG_X0.
 * Stops when rr <= (tol*tol)*bb with rr the recursive residual norm squared
 * and bb = b.b (checked before each iteration), or after maxit iterations;
 * tol = 0 runs exactly maxit iterations.  Not converging is SLA_OK with
 * info.converged = 0.  SLA_ERR_NOT_SPD / SLA_ERR_NONFINITE leave the last
 * iterate in x.  The loop runs on the device (alpha, beta and the stopping
 * test never leave it); the host polls a small status word between blocks
 * of iterations.  info_host may be NULL.  Synchronises `stream`.
 *
 * SLA_FLAG_JACOBI: preconditioned CG with M = diag(A), the preconditioner the
 * pages name for the PyTorch-native backend (Significance / limitations):
 * z = r / d elementwise (d = the stored diagonal entries), alpha = r.z / p.Ap,
 * beta = r.z (new) / r.z, p = z + beta p; the stopping test stays on r.r.
 * A missing or non-positive diagonal entry returns SLA_ERR_NOT_SPD before
 * any iteration.  Needs 2 n + 1 more workspace doubles per system.  The flag
 * applies to the adjoint solve in the same way.
 */
sla_status sla_cg_solve(sla_csr A, const double* b, double* x, double tol,
                        int64_t maxit, uint32_t flags, sla_cg_info* info_host,
                        hipStream_t stream);

/*
 * sla_cg_solve for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same CG iteration as sla_cg_solve on the same handle (the same
 * kernels and grid, so the same results bit for bit), except that a system
 * sla_cg_solve would give the resident grid loop (sla_csr_set_one_group),
 * whose exchange buffers are allocated, runs the two-kernel loop here (the
 * bits of sla_cg_solve with SLA_ONE_GROUP_OFF); with its workspace
 * (r, p, q, partials, scalars) in a static device array of the library
 * instead of the handle's: 64 MiB, which every GPU the library runs on holds
 * until the process ends (not counted by sla_memory_usage).  The call
 * allocates nothing; the caller still provides b and x (device memory).
 * Kernels are launched one by one (no graphs, no events) and the host waits
 * for `stream` every 32 iterations to read the running count.
 * Limits: exactly one system bound; 4 n + 7 G doubles of scratch (G the
 * solver grid) within the 64 MiB, i.e. n up to about 2.09 million unknowns
 * (larger n returns SLA_ERR_ARG, message giving the limit); flags
 * SLA_FLAG_X0 only; a handle without a locality ordering.  The first call
 * on a device looks up the array's address there (set-up).
 * Every call on one GPU shares that GPU's array and overwrites what the last
 * call left in it: calls that overlap on one GPU (other host threads, other
 * streams) race and give wrong results.  Statuses as sla_cg_solve (a pattern
 * that is not symmetric returns SLA_ERR_NOT_SYMMETRIC).  Synchronises
 * `stream`.
 */
sla_status sla_cg_solve_noalloc(sla_csr A, const double* b, double* x, double tol,
                                int64_t maxit, uint32_t flags, sla_cg_info* info_host,
                                hipStream_t stream);

/*
 * Backward pass of x = A^{-1} b (Methodology 2, linear systems): given x and
 * grad_x = dL/dx, solve A^T lambda = grad_x by the same CG (A^T = A for the
 * SPD matrices CG accepts), write grad_b = lambda and
 * grad_vals[k] = -lambda_i x_j for every stored slot k = (i, j).  grad_vals
 * may be NULL (then only grad_b).  Memory: O(n + nnz), independent of the
 * iteration count.  Same stopping rule and statuses as sla_cg_solve.  Since
 * the solve uses A in place of A^T, every call first checks the bound values
 * (each stored a_ij against a_ji, one pass over the values; equal, or within
 * 1e-12 of the larger magnitude, as symmetric expressions such as D A D
 * round mirror entries a few ulps apart); a mismatch returns
 * SLA_ERR_NOT_SYMMETRIC before any iteration (grad_b and grad_vals
 * untouched).
 */
sla_status sla_cg_adjoint(sla_csr A, const double* x, const double* grad_x,
                          double* grad_b, double* grad_vals, double tol,
                          int64_t maxit, uint32_t flags, sla_cg_info* info_host,
                          hipStream_t stream);

/* Shared-pattern batch (Methodology 1, SparseTensor batching): every system
 * of the bound batch solved independently, each with its own scalars and
 * stopping test.  b, x [batch][n]; info_host [batch] (may be NULL).  Returns
 * the first non-OK system status, else SLA_OK.  The symmetry checks are
 * those of sla_cg_solve / sla_cg_adjoint (the adjoint's over every system's
 * values). */
sla_status sla_cg_solve_batched(sla_csr A, const double* b, double* x, double tol,
                                int64_t maxit, uint32_t flags, sla_cg_info* info_host,
                                hipStream_t stream);

sla_status sla_cg_adjoint_batched(sla_csr A, const double* x, const double* grad_x,
                                  double* grad_b, double* grad_vals, double tol,
                                  int64_t maxit, uint32_t flags,
                                  sla_cg_info* info_host, hipStream_t stream);

/* The pattern gradient alone (Methodology 2, linear systems: the matrix
 * gradient only on the sparsity pattern): grad_vals[s][k] = -lambda[s][i] *
 * x[s][j] for every stored slot k = (i, j), one correctly rounded product.
 * lambda, x [batch][n]; grad_vals [batch][nnz].  Asynchronous. */
sla_status sla_pattern_grad(sla_csr A, const double* lambda, const double* x,
                            double* grad_vals, hipStream_t stream);

/* After a solve with SLA_FLAG_HISTORY: copy system `system`'s per-iteration
 * alpha_k, beta_k and r.r after iteration k (host arrays of length cap; any
 * may be NULL).  *count_host = iterations recorded.  The scalars of the CG
 * the pages call "CG" (Methodology 1, iterative backend), for tracing and
 * for checks (the CG-Lanczos Ritz values, the energy identity). */
sla_status sla_cg_history(sla_csr A, int64_t system, double* alpha_host,
                          double* beta_host, double* rr_host, int64_t cap,
                          int64_t* count_host);

/*
 * Instrumentation for the measurements of the pages' kind (Experimental
 * results: CG on 2D Poisson) at the kernel level (batch 1): set up the solve
 * of A x = b as
 * sla_cg_solve does (tol 0) and run one iteration, then launch each of the
 * two kernels of a CG iteration `reps` times on `stream`, each launch
 * bracketed by start/stop events recorded around the kernel itself, and
 * return the mean durations in milliseconds: avg_ms_host[0] the SpMV step
 * (sum of the r.r partials, beta, stopping test, new search direction,
 * deferred x update, q = A p, p.Ap partials); [1] the residual step (sum of
 * the p.Ap partials, alpha, breakdown test, r -= alpha q, r.r partials).
 * Repeated launches redo the same work, so x and the workspace hold
 * meaningless values afterwards.  Synchronises `stream`.
 */
sla_status sla_profile_iteration_kernels(sla_csr A, const double* b, double* x,
                                         int64_t reps, double* avg_ms_host,
                                         hipStream_t stream);

/*
 * The .eigsh of Methodology 1 ("torch-sla" summary): the k extreme eigenpairs
 * of each bound system by m steps of the Lanczos process from the start
 * vector v0.  A must be symmetric (not checked; for a non-symmetric A the
 * results mean nothing).  The pages name the operation
 * but not its algorithm; this library takes the textbook one:
 *   v_0 = v0 / |v0|; for j = 0 .. m-1:
 *     w = A v_j; h = V_j^T w, w -= V_j h; h' = V_j^T w, w -= V_j h'
 *     (full reorthogonalisation: classical Gram-Schmidt applied twice);
 *     alpha_j = h_j + h'_j, beta_j = |w|, v_{j+1} = w / beta_j;
 *   the process ends early when beta_j <= 1e-10 |A v_j| (an invariant
 *   subspace).  The eigenpairs (theta, y) of the tridiagonal T =
 *   tridiag(beta, alpha, beta) over the completed steps give the Ritz pairs
 *   (theta, V y).
 *   which   SLA_EIG_SMALLEST (0): the k smallest algebraic Ritz values;
 *           SLA_EIG_LARGEST (1): the k largest.  Ascending in both cases.
 *   m       Lanczos steps, k <= m <= n.
 *   v0      [batch][n] start vectors (device); must not be zero.
 *   theta   [batch][k] Ritz values (device), ascending.
 *   X       [batch][k][n] unit Ritz vectors (device); the sign of each is
 *           fixed by making the largest component of y positive.
 *   resid   [batch][k] |beta_{steps-1} y_{steps-1}| = |A x - theta x|
 *           (device): how far each pair is from an eigenpair of A.
 *   info_host [batch] steps completed and status per system (may be NULL).
 * Returns the first non-OK system status: SLA_ERR_ARG for a zero v0,
 * SLA_ERR_NONFINITE, SLA_ERR_KRYLOV when fewer than k steps completed; a
 * failed system's theta, X and resid are left untouched.  Workspace of
 * (m + 1) n doubles is kept with the handle.  Synchronises `stream`.
 */
enum { SLA_EIG_SMALLEST = 0, SLA_EIG_LARGEST = 1 };
typedef struct {
  int64_t steps;    /* Lanczos steps completed                             */
  int32_t status;   /* sla_status of this system                           */
  int32_t reserved;
} sla_eig_info;
sla_status sla_eigsh(sla_csr A, int64_t k, int which, int64_t m, const double* v0,
                     double* theta, double* X, double* resid, sla_eig_info* info_host,
                     hipStream_t stream);

/*
 * Gradient of the eigenvalues (Methodology 2, eigenvalue problems: the
 * Hellmann-Feynman relation d lambda / d A_ij = v_i v_j for a simple
 * eigenvalue with unit eigenvector v, on the sparsity pattern only): for a
 * loss with grad_theta = dL/dtheta [batch][k],
 *   grad_vals[s][slot (i, j)] = sum_t grad_theta[s][t] X[s][t][i] X[s][t][j]
 * on every stored slot [batch][nnz], the terms added in ascending t.
 * X [batch][k][n] unit eigenvectors (as sla_eigsh returns them).  All
 * device memory.
 */
sla_status sla_eig_grad(sla_csr A, int64_t k, const double* X, const double* grad_theta,
                        double* grad_vals, hipStream_t stream);

/*
 * Solve A x = b for a general (non-symmetric) A by BiCGStab, one of the
 * solvers the torch-sla summary lists for its CPU backends (Methodology 1),
 * here on the GPU, for every system of the bound batch (shared pattern).
 * The pages name the solver, not its variant; this is the textbook
 * unpreconditioned method:
 *   r = b - A x0 (x0 = 0 unless SLA_FLAG_X0), rhat = r, p = v = 0,
 *   rho_prev = alpha = omega = 1; each iteration:
 *     rho = rhat.r, beta = (rho / rho_prev)(alpha / omega),
 *     p = r + beta (p - omega v), v = A p, alpha = rho / rhat.v,
 *     s = r - alpha v; if s.s <= tol^2 b.b: x += alpha p and stop (the
 *     iteration counts); t = A s, omega = t.s / t.t,
 *     x = (x + alpha p) + omega s, r = s - omega t.
 * Stops, as the CG solve, when the recursive residual has r.r <= tol^2 b.b
 * before an iteration, or after maxit iterations (SLA_OK, converged = 0).
 * rhat.r, rhat.v or t.t equal to 0, or omega = 0, is SLA_ERR_BREAKDOWN;
 * a non-finite dot product SLA_ERR_NONFINITE (x holds the last iterate).
 * flags: SLA_FLAG_X0, SLA_FLAG_HISTORY (rho, alpha, omega, r.r per
 * iteration, read with sla_bicgstab_history).  b, x [batch][n] device
 * memory; info_host [batch] (may be NULL).  Returns the first non-OK system
 * status.  Synchronises `stream`.
 */
sla_status sla_bicgstab_solve(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                              uint32_t flags, sla_cg_info* info_host, hipStream_t stream);

/*
 * Backward pass of x = A^{-1} b solved by BiCGStab (Methodology 2, linear
 * systems): A^T lambda = grad_x by the same BiCGStab on the transposed
 * pattern (built once per handle; the values are gathered into its slot
 * order on each call), grad_b = lambda [batch][n], and
 * grad_vals[k] = -lambda_i x_j on every stored slot [batch][nnz] (may be
 * NULL; computed also after a breakdown, from the last iterate).  flags:
 * SLA_FLAG_HISTORY only.  Synchronises `stream`.
 */
sla_status sla_bicgstab_adjoint(sla_csr A, const double* x, const double* grad_x,
                                double* grad_b, double* grad_vals, double tol, int64_t maxit,
                                uint32_t flags, sla_cg_info* info_host, hipStream_t stream);

/*
 * rho, alpha, omega (0 for a half-step finish) and the residual norm squared
 * after each iteration of system `system` of the last BiCGStab solve or
 * adjoint run with SLA_FLAG_HISTORY.  Host arrays of length cap (each may be
 * NULL); *count_host = the iterations recorded.
 */
sla_status sla_bicgstab_history(sla_csr A, int64_t system, double* rho_host,
                                double* alpha_host, double* omega_host, double* rr_host,
                                int64_t cap, int64_t* count_host);

/*
 * Lists of independent systems, each with its own pattern and size (the
 * SparseTensorList of Methodology 1: distinct patterns per batch item).
 * A[i] is a handle with exactly one system bound; no handle may appear
 * twice.  method SLA_METHOD_CG (SPD systems; flags as sla_cg_solve, so
 * SLA_FLAG_JACOBI too) or SLA_METHOD_BICGSTAB (flags as sla_bicgstab_solve).
 * Every system is solved exactly as by the single-system call on its
 * handle (the same kernels and bits), except that CG systems never take the
 * resident grid loop (sla_csr_set_one_group): its cooperative launch holds
 * every CU and would serialize the list, so such a system gets the
 * two-kernel loop's bits (those of SLA_ONE_GROUP_OFF); up to 8 systems run
 * at once, each on
 * a worker stream of the library's (created once per device, default
 * priority) that first waits for the work already queued on `stream`.
 * Host arrays of device pointers: b[i], x[i] [n_i].  info_host [count]
 * (may be NULL).  Returns the first failing system's status (its message
 * names the system).  Returns when every system is done.
 */
enum { SLA_METHOD_CG = 0, SLA_METHOD_BICGSTAB = 1 };
sla_status sla_solve_list(int64_t count, const sla_csr* A, const double* const* b,
                          double* const* x, double tol, int64_t maxit, uint32_t flags, int method,
                          sla_cg_info* info_host, hipStream_t stream);

/*
 * Backward pass of sla_solve_list (Methodology 2, linear systems, per
 * system): grad_b[i] = lambda_i solving A_i^T lambda_i = grad_x[i], and
 * grad_vals[i][k] = -lambda_i x_j on the stored slots of A_i.  grad_vals
 * (the array) may be NULL, and so may any of its entries (that system's
 * values gradient is then not formed).  flags: SLA_FLAG_HISTORY, and
 * SLA_FLAG_JACOBI for CG.
 */
sla_status sla_adjoint_list(int64_t count, const sla_csr* A, const double* const* x,
                            const double* const* grad_x, double* const* grad_b,
                            double* const* grad_vals, double tol, int64_t maxit, uint32_t flags,
                            int method, sla_cg_info* info_host, hipStream_t stream);

/*
 * Measurement aid for sla_eigsh: after an sla_eigsh call on this handle with
 * m >= nvec, launch the Gram-Schmidt dot pass (V_nvec^T w plus w.w) and the
 * update pass (w -= V_nvec h) over the first nvec basis vectors `reps`
 * times each on `stream` and return their mean durations in milliseconds:
 * avg_ms_host[0] dot, [1] update.  The Lanczos workspace holds meaningless
 * values afterwards (earlier results in the caller's buffers are not
 * touched).  SLA_ERR_ARG without such a call.  Synchronises `stream`.
 */
sla_status sla_profile_lanczos_kernels(sla_csr A, int64_t nvec, int64_t reps,
                                      double* avg_ms_host, hipStream_t stream);

/*
 * SpMV kernel family (the .matvec and the SpMV inside the CG iteration,
 * Methodology 1; a choice of this library, not on the pages).  At creation
 * the pattern analysis checks whether every
 * stored column j of every row i equals i + d for one of at most 8 fixed
 * offsets d (a banded or stencil pattern such as the 5-point Laplacian); if
 * so, the banded kernels can read a mask byte per row and one row pointer per
 * 64 rows instead of the column array and per-row row pointers.  If moreover
 * every offset of magnitude 64 or more is +-L for one L >= 961 (a stencil on
 * a grid whose lines hold L points), the CG iteration can use the line walk:
 * each wave walks a column of 64-point tiles down the grid lines and keeps
 * the neighbouring lines' search direction in registers, so that r and
 * p_{k-1} are read from memory once per row.
 *   SLA_SPMV_AUTO (0, default): the line walk when it applies, else the
 *     banded kernels when the pattern is banded, else the CSR kernels, or
 *     the split form below for CSR patterns without column locality.
 *   SLA_SPMV_CSR (1): always the CSR kernels.
 *   SLA_SPMV_BANDED (2): the banded kernels whenever the pattern is banded
 *     (never the line walk).
 *   SLA_SPMV_SPLIT (3): the CSR kernels with the search-direction update in a
 *     pass of its own, so that the SpMV gathers one vector instead of two;
 *     AUTO picks it for non-banded patterns whose 64-row tiles reach columns
 *     more than 2^17 apart (no reuse of gathered values from cache).
 *   SLA_SPMV_LINES (4): the line walk when it applies, else as BANDED.
 * SpMV results are bit-identical in every case; CG results are identical
 * between CSR and BANDED, and differ only in the order of the p.Ap partial
 * sums (each workgroup's share of rows) under SPLIT and LINES.  *kernels_host (may be NULL) receives the
 * family now in use: 0 CSR, 1 banded, 2 CSR with the separate direction
 * pass, 3 line walk.
 */
enum {
  SLA_SPMV_AUTO = 0,
  SLA_SPMV_CSR = 1,
  SLA_SPMV_BANDED = 2,
  SLA_SPMV_SPLIT = 3,
  SLA_SPMV_LINES = 4
};
sla_status sla_csr_set_spmv_variant(sla_csr A, int variant, int* kernels_host);

/* Iterations per captured HIP graph block (default 32; 0 = launch kernels
 * one by one without graphs): the remedy here for the kernel-launch cost of
 * iterative solvers (Problem statement).  Affects speed only, never
 * results. */
sla_status sla_csr_set_graph_block(sla_csr A, int64_t iterations);

/* Solver workgroups per compute unit (a tuning knob of the CG backend,
 * Methodology 1; 1024 threads each; 512 in the line walk): 0 (default:
 * automatic: 1 for solves of at most 2^21 unknowns over
 * the batch, where the kernels' fixed costs dominate, and for line-walk
 * patterns (2D stencils), whose waves then walk longer chunks, and on
 * reordered handles (sla_csr_reorder), whose gathers hit the L2; else 2), 1
 * (fewer DRAM pages open at once) or 2 (twice the waves to hide latency).
 * The grid sets the number and
 * order of the dot-product partial sums, so CG results differ in the last
 * bits between grids; each setting is reproducible.  SpMV results do not
 * change. */
sla_status sla_csr_set_workgroups_per_cu(sla_csr A, int workgroups);

/*
 * Locality ordering of the unknowns for the iterative solvers.  The pages fix
 * no storage order; this is the library's own remedy for patterns whose
 * unknowns come in an order unrelated to the graph (a random geometric graph
 * whose nodes are numbered in the order the points were drawn, say), where
 * every gathered vector entry of the SpMV misses the caches.
 *
 * SLA_ORDER_BFS renumbers the unknowns in the breadth-first order of the
 * pattern's graph (an edge i -> j for every stored slot (i, j), j != i):
 * from s1, the smallest index among the nodes farthest (in edges) from s0,
 * the smallest index of largest row length; each node's unvisited
 * neighbours are appended in ascending column order; when a visit ends and
 * nodes remain, the next starts at the smallest unvisited index.  Computed on
 * the device (integer work, the same order on every run), together with
 * B = P A P^T (pattern, slot map and solver workspace: about 12 bytes per
 * slot + 8 per slot and system for B's values + 20 bytes per unknown and
 * system).  Synchronises `stream`.  Needs nnz < 2^32.
 *
 * Afterwards the CG and BiCGStab solves and adjoints (sla_cg_solve,
 * sla_cg_solve_batched, sla_cg_adjoint, sla_cg_adjoint_batched,
 * sla_bicgstab_solve, sla_bicgstab_adjoint, and those of sla_solve_list /
 * sla_adjoint_list), sla_cg_history, sla_bicgstab_history and
 * sla_profile_iteration_kernels run on B: every call gathers the bound values
 * into B's slot order and b (or grad_x, and x under SLA_FLAG_X0) into B's
 * unknown order, and scatters x (or grad_b) back; grad_vals is formed on A's
 * own slots.  Inputs and outputs keep A's numbering.  The iterates are A's,
 * permuted, in exact arithmetic (the BiCGStab adjoint runs on
 * (P A P^T)^T = P A^T P^T); in floating point the row sums and dot products
 * are taken in another order, so results differ from the unordered solve by
 * rounding.  Every other call (spmv, the transposed product, eigsh, ...)
 * still uses A as it is.
 * SLA_ORDER_NONE drops the ordering and its memory.
 */
enum { SLA_ORDER_NONE = 0, SLA_ORDER_BFS = 1 };
sla_status sla_csr_reorder(sla_csr A, int ordering, hipStream_t stream);

/* The ordering of a reordered handle: order_out [n] (int32, device) receives
 * the original index of the unknown at each position.  Asynchronous on
 * `stream`.  SLA_ERR_ARG if the handle is not reordered. */
sla_status sla_csr_ordering(sla_csr A, int32_t* order_out, hipStream_t stream);

/*
 * CG loops in one launch.  SLA_ONE_GROUP_AUTO (default): a system of at
 * most 2048 unknowns with a banded pattern (at most 8 column offsets), or
 * whose 64-row tiles hold at most 336 stored entries each (and whose vectors
 * fit one workgroup's LDS), runs its whole CG loop in one
 * workgroup (one launch per solve, one workgroup per system of the batch,
 * workgroup barriers only),
 * instead of two kernels over the whole GPU per iteration, whose launch gaps
 * and partial sums dominate at such sizes (Problem statement: launch costs
 * of iterative solvers on small problems).  A single banded system (no
 * preconditioner) of 2049 to about a million unknowns whose rows fit the
 * chip (at most 8 rows per thread of one 512-thread workgroup per CU, its
 * largest column offset at most 1024 and at most the rows of a workgroup)
 * runs its whole CG loop in one cooperative launch with the system held in
 * registers and LDS (the resident grid loop): the matrix is read once per
 * solve, and the workgroups exchange only halo rows and the partial sums of
 * each iteration.  Both loops run CG in its single-reduction form
 * (Chronopoulos and Gear: r.r and r.Ar summed together, p.Ap from them; with
 * Jacobi, r.r, z.Az and r.z), so one grid-wide or workgroup sum per
 * iteration: the same iterates, scalars, stopping rule, statuses and history
 * in exact arithmetic, results that differ from the two-kernel loop's by
 * rounding (relative 1e-13 in x after 1000 iterations at 10^6 unknowns).  A
 * grid-wide wait of the resident
 * loop that exceeds its poll limit (seconds) ends the solve with
 * SLA_ERR_DEVICE.  SLA_ONE_GROUP_OFF: always the two-kernel loop.  Applies to
 * sla_cg_solve / _batched, the adjoint solves and the CG lists.
 */
enum { SLA_ONE_GROUP_AUTO = 0, SLA_ONE_GROUP_OFF = 1 };
sla_status sla_csr_set_one_group(sla_csr A, int mode);

/*
 * Instrumentation (Experimental results: CG on 2D Poisson, timed per solve):
 * the duration in milliseconds of the last resident grid CG loop launched on
 * this handle (see sla_csr_set_one_group), from events recorded on its
 * stream just before and after the cooperative launch; *ms_host receives it.
 * Waits for that launch.  SLA_ERR_ARG if no resident loop has run since the
 * handle's workspace was last built.
 */
sla_status sla_resident_loop_ms(sla_csr A, double* ms_host);

/* Message of the last failed call on this thread ("" if none): the error
 * reporting of this boundary (not on the pages). */
const char* sla_last_error(void);

/* Name of a status code (not on the pages). */
const char* sla_status_string(sla_status s);

#ifdef __cplusplus
}
#endif
#endif /* SLA_H_ */
