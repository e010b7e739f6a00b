// C ABI of the library (declared in include/sla.h).  Every entry point checks
// its arguments before launching anything, converts every failure into an
// sla_status, and never lets a C++ exception escape.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <map>
#include <mutex>
#include <new>
#include <set>
#include <string>
#include <thread>
#include <vector>

#include "handle.h"

namespace sla {

static thread_local char g_err[1024] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}
void clear_error() { g_err[0] = '\0'; }

// Every device allocation of the library goes through dev_alloc / dev_free,
// which keep the live and peak bytes per device (sla_memory_usage).
namespace {
struct MemBook {
  std::mutex mu;
  std::map<void*, std::pair<int, size_t>> blocks;  // pointer -> (device, bytes)
  std::map<int, int64_t> live, peak;
};
MemBook& mem_book() {
  static MemBook* b = new MemBook();  // never destroyed: frees may come at exit
  return *b;
}
}  // namespace

sla_status dev_alloc(void** p, size_t bytes, const char* what) {
  *p = nullptr;
  const size_t sz = bytes == 0 ? 1 : bytes;
  hipError_t e = hipMalloc(p, sz);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    set_error("out of device memory allocating %zu bytes for %s", bytes, what);
    return SLA_ERR_OOM;
  }
  int dev = 0;
  (void)hipGetDevice(&dev);
  MemBook& b = mem_book();
  std::lock_guard<std::mutex> lock(b.mu);
  b.blocks[*p] = {dev, sz};
  int64_t& live = b.live[dev];
  live += int64_t(sz);
  int64_t& peak = b.peak[dev];
  if (live > peak) peak = live;
  return SLA_OK;
}

void dev_free(void* p) {
  if (!p) return;
  {
    MemBook& b = mem_book();
    std::lock_guard<std::mutex> lock(b.mu);
    auto it = b.blocks.find(p);
    if (it != b.blocks.end()) {
      b.live[it->second.first] -= int64_t(it->second.second);
      b.blocks.erase(it);
    }
  }
  (void)hipFree(p);
}

void memory_usage(int dev, int64_t* live, int64_t* peak, bool reset) {
  MemBook& b = mem_book();
  std::lock_guard<std::mutex> lock(b.mu);
  const int64_t l = b.live.count(dev) ? b.live[dev] : 0;
  if (live) *live = l;
  if (peak) *peak = b.peak.count(dev) ? b.peak[dev] : 0;
  if (reset) b.peak[dev] = l;
}

int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  cache[dev] = cus;
  return cus;
}

}  // namespace sla

using namespace sla;

#define API_BEGIN try {
#define API_END                                                                \
  }                                                                            \
  catch (const std::bad_alloc&) {                                              \
    set_error("host out of memory");                                           \
    return SLA_ERR_OOM;                                                        \
  }                                                                            \
  catch (...) {                                                                \
    set_error("internal error");                                               \
    return SLA_ERR_DEVICE;                                                     \
  }

#define REQUIRE(cond, ...)                                                     \
  do {                                                                         \
    if (!(cond)) {                                                             \
      set_error(__VA_ARGS__);                                                  \
      return SLA_ERR_ARG;                                                      \
    }                                                                          \
  } while (0)

static bool valid_index(sla_index v) { return v == SLA_I32 || v == SLA_I64; }

namespace sla {
void free_handle(sla_csr A) {
  if (!A) return;
  release_workspace(A);
  release_eig_work(A);
  release_bs_work(A);
  release_reorder(A);
  free_handle(A->trans);
  dev_free(A->rowptr);
  dev_free(A->col);
  dev_free(A->perm);
  dev_free(A->sorted_idx);
  dev_free(A->grp);
  dev_free(A->band_mask);
  dev_free(A->vals_owned);
  dev_free(A->sym_flag);
  delete A;
}
}  // namespace sla

static void destroy_handle(sla_csr A) { free_handle(A); }

extern "C" {

const char* sla_last_error(void) { return g_err; }

const char* sla_status_string(sla_status s) {
  switch (s) {
    case SLA_OK: return "SLA_OK";
    case SLA_ERR_ARG: return "SLA_ERR_ARG";
    case SLA_ERR_CSR: return "SLA_ERR_CSR";
    case SLA_ERR_OOM: return "SLA_ERR_OOM";
    case SLA_ERR_DEVICE: return "SLA_ERR_DEVICE";
    case SLA_ERR_NOT_SPD: return "SLA_ERR_NOT_SPD";
    case SLA_ERR_NONFINITE: return "SLA_ERR_NONFINITE";
    case SLA_ERR_KRYLOV: return "SLA_ERR_KRYLOV";
    case SLA_ERR_BREAKDOWN: return "SLA_ERR_BREAKDOWN";
    case SLA_ERR_NOT_SYMMETRIC: return "SLA_ERR_NOT_SYMMETRIC";
  }
  return "SLA_UNKNOWN";
}

sla_status sla_csr_create(int64_t n, int64_t nnz_coo, sla_index coo_idx, const void* coo_row,
                          const void* coo_col, sla_index rowptr_idx, hipStream_t stream,
                          sla_csr* out) {
  API_BEGIN
  clear_error();
  REQUIRE(out != nullptr, "sla_csr_create: out is NULL");
  REQUIRE(n >= 1 && n < (int64_t(1) << 31) - 1, "sla_csr_create: n=%lld out of range",
          (long long)n);
  REQUIRE(nnz_coo >= 0 && nnz_coo < (int64_t(1) << 32),
          "sla_csr_create: nnz_coo=%lld out of range", (long long)nnz_coo);
  REQUIRE(valid_index(coo_idx) && valid_index(rowptr_idx), "sla_csr_create: bad index width");
  REQUIRE(nnz_coo == 0 || (coo_row != nullptr && coo_col != nullptr),
          "sla_csr_create: NULL coordinates");
  sla_csr A = new sla_csr_s();
  (void)hipGetDevice(&A->device);
  A->n = n;
  A->nnz_coo = nnz_coo;
  A->rp_idx = rowptr_idx;
  sla_status s = build_from_coo(A, coo_idx, coo_row, coo_col, stream);
  if (s == SLA_OK) s = analyse_pattern(A, stream);
  if (s != SLA_OK) {
    destroy_handle(A);
    return s;
  }
  *out = A;
  return SLA_OK;
  API_END
}

sla_status sla_csr_create_from_csr(int64_t n, int64_t nnz, sla_index rowptr_idx,
                                   const void* rowptr, const int32_t* col, hipStream_t stream,
                                   sla_csr* out) {
  API_BEGIN
  clear_error();
  REQUIRE(out != nullptr, "sla_csr_create_from_csr: out is NULL");
  REQUIRE(n >= 1 && n < (int64_t(1) << 31) - 1, "sla_csr_create_from_csr: n out of range");
  REQUIRE(valid_index(rowptr_idx), "sla_csr_create_from_csr: bad index width");
  REQUIRE(nnz >= 0 && (rowptr_idx == SLA_I64 || nnz < (int64_t(1) << 31)),
          "sla_csr_create_from_csr: nnz=%lld does not fit the row pointer", (long long)nnz);
  REQUIRE(rowptr != nullptr && (nnz == 0 || col != nullptr),
          "sla_csr_create_from_csr: NULL array");
  sla_csr A = new sla_csr_s();
  (void)hipGetDevice(&A->device);
  A->n = n;
  A->nnz = nnz;
  A->rp_idx = rowptr_idx;
  sla_status s = build_from_csr(A, rowptr, col, stream);
  if (s == SLA_OK) s = analyse_pattern(A, stream);
  if (s != SLA_OK) {
    destroy_handle(A);
    return s;
  }
  *out = A;
  return SLA_OK;
  API_END
}

sla_status sla_csr_destroy(sla_csr A) {
  API_BEGIN
  if (A) {
    (void)hipDeviceSynchronize();
    destroy_handle(A);
  }
  return SLA_OK;
  API_END
}

sla_status sla_csr_get_info(sla_csr A, int64_t* n, int64_t* nnz, int64_t* nnz_coo,
                            sla_index* rowptr_idx) {
  REQUIRE(A != nullptr, "sla_csr_get_info: NULL handle");
  if (n) *n = A->n;
  if (nnz) *nnz = A->nnz;
  if (nnz_coo) *nnz_coo = A->nnz_coo;
  if (rowptr_idx) *rowptr_idx = A->rp_idx;
  return SLA_OK;
}

sla_status sla_csr_pattern(sla_csr A, const void** rowptr, const int32_t** col,
                           const int64_t** perm) {
  REQUIRE(A != nullptr, "sla_csr_pattern: NULL handle");
  if (rowptr) *rowptr = A->rowptr;
  if (col) *col = A->col;
  if (perm) *perm = A->perm;
  return SLA_OK;
}

sla_status sla_csr_copy_pattern(sla_csr A, void* rowptr_out, int32_t* col_out,
                                int64_t* perm_out, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_copy_pattern: NULL handle");
  REQUIRE(perm_out == nullptr || A->perm != nullptr,
          "sla_csr_copy_pattern: handle was not built from COO (no perm)");
  if (rowptr_out)
    SLA_TRY_HIP(hipMemcpyAsync(rowptr_out, A->rowptr, size_t(A->n + 1) * A->rp_idx,
                               hipMemcpyDeviceToDevice, stream));
  if (col_out && A->nnz > 0)
    SLA_TRY_HIP(hipMemcpyAsync(col_out, A->col, sizeof(int32_t) * A->nnz,
                               hipMemcpyDeviceToDevice, stream));
  if (perm_out && A->nnz_coo > 0)
    SLA_TRY_HIP(hipMemcpyAsync(perm_out, A->perm, sizeof(int64_t) * A->nnz_coo,
                               hipMemcpyDeviceToDevice, stream));
  return SLA_OK;
  API_END
}

sla_status sla_csr_values_from_coo(sla_csr A, const double* coo_val, double* vals,
                                   int64_t batch, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_values_from_coo: NULL handle");
  REQUIRE(A->perm != nullptr, "sla_csr_values_from_coo: handle was not built from COO");
  REQUIRE(batch >= 1 && batch <= 65535, "sla_csr_values_from_coo: batch out of range");
  REQUIRE(A->nnz == 0 || (coo_val != nullptr && vals != nullptr),
          "sla_csr_values_from_coo: NULL array");
  return launch_values_from_coo(A, coo_val, vals, batch, stream);
  API_END
}

sla_status sla_csr_grad_to_coo(sla_csr A, const double* grad_vals, double* grad_coo,
                               int64_t batch, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_grad_to_coo: NULL handle");
  REQUIRE(A->perm != nullptr, "sla_csr_grad_to_coo: handle was not built from COO");
  REQUIRE(batch >= 1 && batch <= 65535, "sla_csr_grad_to_coo: batch out of range");
  REQUIRE(A->nnz_coo == 0 || (grad_vals != nullptr && grad_coo != nullptr),
          "sla_csr_grad_to_coo: NULL array");
  return launch_grad_to_coo(A, grad_vals, grad_coo, batch, stream);
  API_END
}

sla_status sla_csr_set_values(sla_csr A, const double* vals, int64_t batch) {
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_set_values: NULL handle");
  REQUIRE(batch >= 1 && batch <= 65535, "sla_csr_set_values: batch out of range");
  REQUIRE(A->nnz == 0 || vals != nullptr, "sla_csr_set_values: NULL values");
  REQUIRE(vals == nullptr || vals != A->vals_owned || batch <= A->owned_batch,
          "sla_csr_set_values: the handle's own values hold %lld systems",
          (long long)A->owned_batch);
  A->vals = vals;
  A->batch = batch;
  return SLA_OK;
}

sla_status sla_csr_load_values(sla_csr A, const double* vals, int64_t batch, int order,
                               hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_load_values: NULL handle");
  REQUIRE(batch >= 1 && batch <= 65535, "sla_csr_load_values: batch out of range");
  REQUIRE(order == SLA_VALUES_CSR || order == SLA_VALUES_COO,
          "sla_csr_load_values: bad order %d", order);
  REQUIRE(order == SLA_VALUES_CSR || A->perm != nullptr,
          "sla_csr_load_values: COO values need a handle built from COO");
  const int64_t len = order == SLA_VALUES_CSR ? A->nnz : A->nnz_coo;
  REQUIRE(len == 0 || vals != nullptr, "sla_csr_load_values: NULL values");
  REQUIRE(vals == nullptr || A->vals_owned == nullptr || vals != A->vals_owned,
          "sla_csr_load_values: the source is the handle's own array");
  if (A->vals_owned == nullptr || A->owned_batch != batch) {
    if (A->vals_owned != nullptr) {
      // the old copy may still be read by queued work
      SLA_TRY_HIP(hipStreamSynchronize(stream));
      if (A->vals == A->vals_owned) {
        A->vals = nullptr;
        A->batch = 0;
      }
      dev_free(A->vals_owned);
      A->vals_owned = nullptr;
      A->owned_batch = 0;
    }
    SLA_TRY(dev_alloc(&A->vals_owned, size_t(batch) * size_t(A->nnz > 0 ? A->nnz : 1),
                      "the handle's values"));
    A->owned_batch = batch;
  }
  if (order == SLA_VALUES_CSR) {
    if (A->nnz > 0)
      SLA_TRY_HIP(hipMemcpyAsync(A->vals_owned, vals, sizeof(double) * size_t(batch) * A->nnz,
                                 hipMemcpyDeviceToDevice, stream));
  } else {
    SLA_TRY(launch_values_from_coo(A, vals, A->vals_owned, batch, stream));
  }
  A->vals = A->vals_owned;
  A->batch = batch;
  return SLA_OK;
  API_END
}

sla_status sla_csr_arrays(sla_csr A, const void** rowptr, const int32_t** col, double** vals,
                          const int64_t** perm) {
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_arrays: NULL handle");
  if (rowptr) *rowptr = A->rowptr;
  if (col) *col = A->col;
  if (vals) *vals = const_cast<double*>(A->vals);
  if (perm) *perm = A->perm;
  return SLA_OK;
}

sla_status sla_memory_usage(int64_t* live_host, int64_t* peak_host, int reset_peak) {
  API_BEGIN
  clear_error();
  int dev = 0;
  SLA_TRY_HIP(hipGetDevice(&dev));
  memory_usage(dev, live_host, peak_host, reset_peak != 0);
  return SLA_OK;
  API_END
}

sla_status sla_spmv(sla_csr A, const double* x, double* y, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_spmv: NULL handle");
  REQUIRE(A->batch >= 1, "sla_spmv: no values bound (sla_csr_set_values)");
  REQUIRE(x != nullptr && y != nullptr, "sla_spmv: NULL vector");
  return launch_spmv(A, A->vals, A->batch, x, y, stream);
  API_END
}

sla_status sla_spmv_transpose(sla_csr A, const double* x, double* y, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_spmv_transpose: NULL handle");
  REQUIRE(A->batch >= 1, "sla_spmv_transpose: no values bound (sla_csr_set_values)");
  REQUIRE(x != nullptr && y != nullptr, "sla_spmv_transpose: NULL vector");
  return launch_spmv_transpose(A, x, y, stream);
  API_END
}

sla_status sla_matvec_grad(sla_csr A, const double* x, const double* grad_y, double* grad_x,
                           double* grad_vals, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_matvec_grad: NULL handle");
  REQUIRE(A->batch >= 1, "sla_matvec_grad: no values bound (sla_csr_set_values)");
  REQUIRE(grad_y != nullptr, "sla_matvec_grad: NULL grad_y");
  REQUIRE(grad_vals == nullptr || A->nnz == 0 || x != nullptr, "sla_matvec_grad: grad_vals needs x");
  if (grad_x != nullptr) SLA_TRY(launch_spmv_transpose(A, grad_y, grad_x, stream));
  if (grad_vals != nullptr && A->nnz > 0)
    SLA_TRY(launch_slot_products(A, A->batch, grad_y, x, grad_vals, false, stream));
  return SLA_OK;
  API_END
}

sla_status sla_eigsh(sla_csr A, int64_t k, int which, int64_t m, const double* v0,
                     double* theta, double* X, double* resid, sla_eig_info* info_host,
                     hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_eigsh: NULL handle");
  REQUIRE(A->batch >= 1, "sla_eigsh: no values bound (sla_csr_set_values)");
  REQUIRE(v0 != nullptr && theta != nullptr && X != nullptr && resid != nullptr,
          "sla_eigsh: NULL vector");
  REQUIRE(which == SLA_EIG_SMALLEST || which == SLA_EIG_LARGEST, "sla_eigsh: bad `which` %d",
          which);
  REQUIRE(k >= 1 && k <= m && m <= A->n, "sla_eigsh: need 1 <= k <= m <= n (k=%lld m=%lld n=%lld)",
          (long long)k, (long long)m, (long long)A->n);
  return run_eigsh(A, k, which, m, v0, theta, X, resid, info_host, stream);
  API_END
}

sla_status sla_eig_grad(sla_csr A, int64_t k, const double* X, const double* grad_theta,
                        double* grad_vals, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_eig_grad: NULL handle");
  REQUIRE(A->batch >= 1, "sla_eig_grad: no values bound (sla_csr_set_values)");
  REQUIRE(k >= 1, "sla_eig_grad: k must be >= 1");
  REQUIRE(X != nullptr && grad_theta != nullptr && grad_vals != nullptr,
          "sla_eig_grad: NULL vector");
  if (A->nnz == 0) return SLA_OK;
  return launch_eig_grad(A, k, X, grad_theta, grad_vals, stream);
  API_END
}

static sla_status check_solve(sla_csr A, const void* b, const void* x, double tol,
                              int64_t maxit, uint32_t flags, const char* who) {
  REQUIRE(A != nullptr, "%s: NULL handle", who);
  REQUIRE(A->batch >= 1, "%s: no values bound (sla_csr_set_values)", who);
  REQUIRE(b != nullptr && x != nullptr, "%s: NULL vector", who);
  REQUIRE(std::isfinite(tol) && tol >= 0.0, "%s: tol must be finite and >= 0", who);
  REQUIRE(maxit >= 0, "%s: maxit must be >= 0", who);
  REQUIRE((flags & ~uint32_t(SLA_FLAG_X0 | SLA_FLAG_HISTORY | SLA_FLAG_JACOBI)) == 0,
          "%s: unknown flags", who);
  return SLA_OK;
}

// CG needs A^T = A.  The pattern's symmetry is checked once per handle (the
// first CG call); a handle whose pattern is not symmetric is refused by
// every CG solve and adjoint.  The adjoint, which solves with A in place of
// A^T, also checks the bound values on every call (mirror entries equal to
// within 1e-12 relative).
static const char kValuesNotSymmetric[] =
    "%s: the values are not symmetric (a_ij and a_ji differ by more than 1e-12 relative); "
    "the adjoint solves with A in place of A^T";

static sla_status require_symmetric(sla_csr A, bool values, const char* who,
                                    hipStream_t stream) {
  if (A->sym_pattern < 0) {
    int bad = 0;
    SLA_TRY(check_symmetry(A, false, &bad, stream));
    A->sym_pattern = (bad & 1) ? 0 : 1;
  }
  if (!A->sym_pattern) {
    set_error("%s: the pattern is not symmetric (a stored (i, j) without (j, i)); CG needs "
              "A^T = A (BiCGStab takes general matrices)", who);
    return SLA_ERR_NOT_SYMMETRIC;
  }
  if (values) {
    int bad = 0;
    SLA_TRY(check_symmetry(A, true, &bad, stream));
    if (bad) {
      set_error(kValuesNotSymmetric, who);
      return SLA_ERR_NOT_SYMMETRIC;
    }
  }
  return SLA_OK;
}

static void fill_status(sla_cg_info* info, int64_t batch, sla_status s) {
  if (!info) return;
  for (int64_t i = 0; i < batch; ++i) {
    info[i].iterations = 0;
    info[i].rel_residual = 0.0;
    info[i].converged = 0;
    info[i].status = s;
  }
}

sla_status sla_cg_solve_batched(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                                uint32_t flags, sla_cg_info* info, hipStream_t stream) {
  API_BEGIN
  clear_error();
  SLA_TRY(check_solve(A, b, x, tol, maxit, flags, "sla_cg_solve_batched"));
  const sla_status sym = require_symmetric(A, false, "sla_cg_solve_batched", stream);
  if (sym != SLA_OK) {
    fill_status(info, A->batch, sym);
    return sym;
  }
  return run_cg_any(A, b, x, tol, maxit, flags, info, stream);
  API_END
}

sla_status sla_cg_solve(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                        uint32_t flags, sla_cg_info* info, hipStream_t stream) {
  API_BEGIN
  clear_error();
  SLA_TRY(check_solve(A, b, x, tol, maxit, flags, "sla_cg_solve"));
  REQUIRE(A->batch == 1, "sla_cg_solve: %lld systems bound; use sla_cg_solve_batched",
          (long long)A->batch);
  const sla_status sym = require_symmetric(A, false, "sla_cg_solve", stream);
  if (sym != SLA_OK) {
    fill_status(info, 1, sym);
    return sym;
  }
  return run_cg_any(A, b, x, tol, maxit, flags, info, stream);
  API_END
}

// A^T lambda = grad_x with A^T = A (CG requires a symmetric matrix; checked
// first), then the pattern gradient (also from the last iterate after a
// breakdown), on A's own slots whether or not the solve ran on a reordered
// copy.  Systems on the one-workgroup loop take the values' check on the
// device: its flag stops the solve and the pattern gradient there, and one
// read-back at the end reports the refusal (no round trip before the solve,
// which at such sizes costs more than the solve's own launch).
static sla_status run_cg_adjoint(sla_csr A, const double* x, const double* grad_x,
                                 double* grad_b, double* grad_vals, double tol, int64_t maxit,
                                 uint32_t flags, sla_cg_info* info, hipStream_t stream) {
  if (A->ro == nullptr &&
      (use_one_group(A) || ((flags & kFlagNoResident) == 0 &&
                            use_grid(A, A->batch, (flags & SLA_FLAG_JACOBI) != 0)))) {
    const sla_status ps = require_symmetric(A, false, "sla_cg_adjoint", stream);
    if (ps != SLA_OK) {
      fill_status(info, A->batch, ps);
      return ps;
    }
    int* gate = nullptr;
    SLA_TRY(enqueue_symmetry_check(A, true, stream, &gate));
    AdjointTail tail;
    tail.gate = gate;
    tail.x = x;
    tail.grad_vals = grad_vals;
    const sla_status s = run_cg(A, grad_x, grad_b, tol, maxit, flags, info, stream, &tail);
    if (s == SLA_ERR_NOT_SYMMETRIC) set_error(kValuesNotSymmetric, "sla_cg_adjoint");
    return s;
  }
  const sla_status sym = require_symmetric(A, true, "sla_cg_adjoint", stream);
  if (sym != SLA_OK) {
    fill_status(info, A->batch, sym);
    return sym;
  }
  sla_status s = run_cg_any(A, grad_x, grad_b, tol, maxit, flags, info, stream);
  if (grad_vals != nullptr && (s == SLA_OK || s == SLA_ERR_NOT_SPD || s == SLA_ERR_NONFINITE)) {
    sla_status g = launch_pattern_grad(A, A->batch, grad_b, x, grad_vals, stream);
    if (g != SLA_OK) return g;
    if (hipStreamSynchronize(stream) != hipSuccess) {
      set_error("sla_cg_adjoint: synchronisation failed");
      return SLA_ERR_DEVICE;
    }
  }
  return s;
}

sla_status sla_cg_adjoint_batched(sla_csr A, const double* x, const double* grad_x,
                                  double* grad_b, double* grad_vals, double tol, int64_t maxit,
                                  uint32_t flags, sla_cg_info* info, hipStream_t stream) {
  API_BEGIN
  clear_error();
  SLA_TRY(check_solve(A, grad_x, grad_b, tol, maxit, flags, "sla_cg_adjoint"));
  REQUIRE((flags & SLA_FLAG_X0) == 0, "sla_cg_adjoint: SLA_FLAG_X0 is not supported");
  REQUIRE(grad_vals == nullptr || x != nullptr, "sla_cg_adjoint: grad_vals needs x");
  return run_cg_adjoint(A, x, grad_x, grad_b, grad_vals, tol, maxit, flags, info, stream);
  API_END
}

// ---------------------------------------------------------------------------
// Lists of systems with their own patterns (SparseTensorList)
// ---------------------------------------------------------------------------

extern "C++" {
// Worker streams, created once per device and kept for the process.
static constexpr int kListWorkers = 8;
static sla_status list_streams(int device, hipStream_t* out) {
  static std::mutex mu;
  static std::map<int, std::vector<hipStream_t>> pools;
  std::lock_guard<std::mutex> lock(mu);
  auto& v = pools[device];
  while (int(v.size()) < kListWorkers) {
    hipStream_t st = nullptr;
    SLA_TRY_HIP(hipStreamCreateWithFlags(&st, hipStreamNonBlocking));
    v.push_back(st);
  }
  for (int i = 0; i < kListWorkers; ++i) out[i] = v[size_t(i)];
  return SLA_OK;
}

// Runs one(i, stream, &info[i]) for i < count on up to kListWorkers host
// threads, each with a stream of its own that first waits for the work
// queued on `stream`; returns when every system is done.  A failing system's
// status and message are reported for the first such i.
template <typename F>
static sla_status run_list(int64_t count, sla_cg_info* info, hipStream_t stream, F&& one) {
  int device = 0;
  SLA_TRY_HIP(hipGetDevice(&device));
  hipStream_t streams[kListWorkers];
  SLA_TRY(list_streams(device, streams));
  hipEvent_t ready = nullptr;
  SLA_TRY_HIP(hipEventCreateWithFlags(&ready, hipEventDisableTiming));
  if (hipEventRecord(ready, stream) != hipSuccess) {
    (void)hipEventDestroy(ready);
    set_error("solve list: event record failed");
    return SLA_ERR_DEVICE;
  }
  const int workers = int(count < kListWorkers ? count : kListWorkers);
  std::atomic<int64_t> next{0};
  const size_t cnt = static_cast<size_t>(count);
  std::vector<sla_status> status(cnt, SLA_OK);
  std::vector<std::string> message(cnt);
  std::vector<sla_cg_info> local(cnt);
  std::vector<std::thread> pool;
  for (int w = 0; w < workers; ++w) {
    pool.emplace_back([&, w]() {
      hipStream_t st = streams[w];
      bool ok = hipSetDevice(device) == hipSuccess && hipStreamWaitEvent(st, ready, 0) == hipSuccess;
      for (;;) {
        const int64_t i = next.fetch_add(1);
        if (i >= count) break;
        if (!ok) {
          status[size_t(i)] = SLA_ERR_DEVICE;
          message[size_t(i)] = "worker stream set-up failed";
          continue;
        }
        clear_error();
        sla_status s = SLA_ERR_DEVICE;
        try {
          s = one(i, st, &local[size_t(i)]);
        } catch (...) {
          set_error("unexpected exception");
        }
        status[size_t(i)] = s;
        if (s != SLA_OK) message[size_t(i)] = sla_last_error();
      }
      (void)hipStreamSynchronize(st);
    });
  }
  for (auto& t : pool) t.join();
  (void)hipEventDestroy(ready);
  if (info)
    for (int64_t i = 0; i < count; ++i) info[i] = local[size_t(i)];
  for (int64_t i = 0; i < count; ++i)
    if (status[size_t(i)] != SLA_OK) {
      set_error("system %lld: %s", (long long)i, message[size_t(i)].c_str());
      return status[size_t(i)];
    }
  clear_error();
  return SLA_OK;
}

static sla_status check_list(int64_t count, const sla_csr* A, int method, uint32_t flags,
                             const char* who) {
  REQUIRE(count >= 1 && A != nullptr, "%s: empty list", who);
  REQUIRE(method == SLA_METHOD_CG || method == SLA_METHOD_BICGSTAB, "%s: unknown method %d", who,
          method);
  REQUIRE(method == SLA_METHOD_CG || (flags & SLA_FLAG_JACOBI) == 0,
          "%s: BiCGStab takes no preconditioner", who);
  std::set<const void*> seen;
  for (int64_t i = 0; i < count; ++i) {
    REQUIRE(A[i] != nullptr, "%s: handle %lld is NULL", who, (long long)i);
    REQUIRE(A[i]->batch == 1, "%s: handle %lld must have exactly one system bound", who,
            (long long)i);
    REQUIRE(seen.insert(A[i]).second, "%s: handle %lld appears twice", who, (long long)i);
  }
  return SLA_OK;
}
}  // extern "C++"

sla_status sla_solve_list(int64_t count, const sla_csr* A, const double* const* b,
                          double* const* x, double tol, int64_t maxit, uint32_t flags, int method,
                          sla_cg_info* info, hipStream_t stream) {
  API_BEGIN
  clear_error();
  SLA_TRY(check_list(count, A, method, flags, "sla_solve_list"));
  REQUIRE(b != nullptr && x != nullptr, "sla_solve_list: NULL vector array");
  for (int64_t i = 0; i < count; ++i)
    SLA_TRY(check_solve(A[i], b[i], x[i], tol, maxit, flags, "sla_solve_list"));
  return run_list(count, info, stream, [&](int64_t i, hipStream_t st, sla_cg_info* in) {
    if (method == SLA_METHOD_CG) {
      const sla_status sym = require_symmetric(A[i], false, "sla_solve_list", st);
      if (sym != SLA_OK) {
        fill_status(in, 1, sym);
        return sym;
      }
      return run_cg_any(A[i], b[i], x[i], tol, maxit, flags | kFlagNoResident, in, st);
    }
    return run_bicgstab_any(A[i], b[i], x[i], tol, maxit, flags, in, st);
  });
  API_END
}

sla_status sla_adjoint_list(int64_t count, const sla_csr* A, const double* const* x,
                            const double* const* grad_x, double* const* grad_b,
                            double* const* grad_vals, double tol, int64_t maxit, uint32_t flags,
                            int method, sla_cg_info* info, hipStream_t stream) {
  API_BEGIN
  clear_error();
  SLA_TRY(check_list(count, A, method, flags, "sla_adjoint_list"));
  REQUIRE((flags & SLA_FLAG_X0) == 0, "sla_adjoint_list: SLA_FLAG_X0 is not supported");
  REQUIRE(grad_x != nullptr && grad_b != nullptr, "sla_adjoint_list: NULL vector array");
  for (int64_t i = 0; i < count; ++i) {
    SLA_TRY(check_solve(A[i], grad_x[i], grad_b[i], tol, maxit, flags, "sla_adjoint_list"));
    REQUIRE(grad_vals == nullptr || grad_vals[i] == nullptr || (x != nullptr && x[i] != nullptr),
            "sla_adjoint_list: grad_vals needs x");
  }
  return run_list(count, info, stream, [&](int64_t i, hipStream_t st, sla_cg_info* in) {
    double* gv = grad_vals ? grad_vals[i] : nullptr;
    const double* xi = x ? x[i] : nullptr;
    return method == SLA_METHOD_CG
               ? run_cg_adjoint(A[i], xi, grad_x[i], grad_b[i], gv, tol, maxit,
                                flags | kFlagNoResident, in, st)
               : run_bicgstab_adjoint_any(A[i], xi, grad_x[i], grad_b[i], gv, tol, maxit, flags, in,
                                      st);
  });
  API_END
}

sla_status sla_bicgstab_solve(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                              uint32_t flags, sla_cg_info* info, hipStream_t stream) {
  API_BEGIN
  clear_error();
  SLA_TRY(check_solve(A, b, x, tol, maxit, flags & ~uint32_t(SLA_FLAG_JACOBI), "sla_bicgstab_solve"));
  REQUIRE((flags & SLA_FLAG_JACOBI) == 0, "sla_bicgstab_solve: no preconditioner is supported");
  return run_bicgstab_any(A, b, x, tol, maxit, flags, info, stream);
  API_END
}

sla_status sla_bicgstab_adjoint(sla_csr A, const double* x, const double* grad_x,
                                double* grad_b, double* grad_vals, double tol, int64_t maxit,
                                uint32_t flags, sla_cg_info* info, hipStream_t stream) {
  API_BEGIN
  clear_error();
  SLA_TRY(check_solve(A, grad_x, grad_b, tol, maxit, flags, "sla_bicgstab_adjoint"));
  REQUIRE((flags & ~uint32_t(SLA_FLAG_HISTORY)) == 0,
          "sla_bicgstab_adjoint: only SLA_FLAG_HISTORY is supported");
  REQUIRE(grad_vals == nullptr || x != nullptr, "sla_bicgstab_adjoint: grad_vals needs x");
  return run_bicgstab_adjoint_any(A, x, grad_x, grad_b, grad_vals, tol, maxit, flags, info,
                                  stream);
  API_END
}

sla_status sla_bicgstab_history(sla_csr A, int64_t system, double* rho, double* alpha,
                                double* omega, double* rr, int64_t cap, int64_t* count) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_bicgstab_history: NULL handle");
  REQUIRE(cap >= 0, "sla_bicgstab_history: cap < 0");
  return bicgstab_history(solver_handle(A), system, rho, alpha, omega, rr, cap, count);
  API_END
}

sla_status sla_cg_adjoint(sla_csr A, const double* x, const double* grad_x, double* grad_b,
                          double* grad_vals, double tol, int64_t maxit, uint32_t flags,
                          sla_cg_info* info, hipStream_t stream) {
  REQUIRE(A != nullptr, "sla_cg_adjoint: NULL handle");
  REQUIRE(A->batch == 1, "sla_cg_adjoint: %lld systems bound; use sla_cg_adjoint_batched",
          (long long)A->batch);
  return sla_cg_adjoint_batched(A, x, grad_x, grad_b, grad_vals, tol, maxit, flags, info,
                                stream);
}

sla_status sla_pattern_grad(sla_csr A, const double* lambda, const double* x, double* grad_vals,
                            hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_pattern_grad: NULL handle");
  REQUIRE(A->batch >= 1, "sla_pattern_grad: no batch bound (sla_csr_set_values)");
  REQUIRE(lambda != nullptr && x != nullptr && (A->nnz == 0 || grad_vals != nullptr),
          "sla_pattern_grad: NULL array");
  return launch_pattern_grad(A, A->batch, lambda, x, grad_vals, stream);
  API_END
}

sla_status sla_resident_loop_ms(sla_csr A, double* ms_host) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr && ms_host != nullptr, "sla_resident_loop_ms: NULL argument");
  A = solver_handle(A);
  const sla_status s = grid_loop_ms(A, ms_host);
  if (s == SLA_ERR_ARG)
    set_error("sla_resident_loop_ms: no resident CG loop has run on this handle");
  return s;
  API_END
}

sla_status sla_cg_history(sla_csr A, int64_t system, double* alpha, double* beta, double* rr,
                          int64_t cap, int64_t* count) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_cg_history: NULL handle");
  A = solver_handle(A);
  REQUIRE(A->hist != nullptr && A->scal_host != nullptr,
          "sla_cg_history: no solve with SLA_FLAG_HISTORY yet");
  REQUIRE(system >= 0 && system < A->ws_batch, "sla_cg_history: system out of range");
  REQUIRE(cap >= 0, "sla_cg_history: cap < 0");
  const int64_t it = std::min<int64_t>(A->scal_host[system].it, A->hist_cap);
  const int64_t k = std::min<int64_t>(it, cap);
  if (count) *count = it;
  if (k > 0) {
    double* h = new double[size_t(k) * 3];
    hipError_t e = hipMemcpy(h, A->hist + size_t(system) * A->hist_cap * 3,
                             sizeof(double) * 3 * k, hipMemcpyDeviceToHost);
    if (e != hipSuccess) {
      delete[] h;
      set_error("sla_cg_history: copy failed: %s", hipGetErrorString(e));
      return SLA_ERR_DEVICE;
    }
    for (int64_t j = 0; j < k; ++j) {
      if (alpha) alpha[j] = h[3 * j];
      if (beta) beta[j] = h[3 * j + 1];
      if (rr) rr[j] = h[3 * j + 2];
    }
    delete[] h;
  }
  return SLA_OK;
  API_END
}

sla_status sla_profile_iteration_kernels(sla_csr A, const double* b, double* x, int64_t reps,
                                         double* avg_ms_host, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_profile_iteration_kernels: NULL handle");
  REQUIRE(A->batch == 1, "sla_profile_iteration_kernels: bind exactly one system");
  REQUIRE(b != nullptr && x != nullptr && avg_ms_host != nullptr,
          "sla_profile_iteration_kernels: NULL pointer");
  REQUIRE(reps >= 1 && reps <= 100000, "sla_profile_iteration_kernels: reps out of range");
  return profile_kernels_any(A, b, x, reps, avg_ms_host, stream);
  API_END
}

sla_status sla_profile_lanczos_kernels(sla_csr A, int64_t nvec, int64_t reps,
                                      double* avg_ms_host, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_profile_lanczos_kernels: NULL handle");
  REQUIRE(avg_ms_host != nullptr, "sla_profile_lanczos_kernels: NULL pointer");
  REQUIRE(reps >= 1 && reps <= 100000, "sla_profile_lanczos_kernels: reps out of range");
  return profile_lanczos_kernels(A, nvec, reps, avg_ms_host, stream);
  API_END
}

sla_status sla_csr_set_spmv_variant(sla_csr A, int variant, int* kernels) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_set_spmv_variant: NULL handle");
  REQUIRE(variant >= SLA_SPMV_AUTO && variant <= SLA_SPMV_LINES,
          "sla_csr_set_spmv_variant: unknown variant %d", variant);
  for (sla_csr H : {A, solver_handle(A)}) {
    if (variant != H->spmv_variant) {
      (void)hipDeviceSynchronize();
      release_workspace(H);  // the captured graphs hold the old kernels
      H->spmv_variant = variant;
    }
  }
  // the family the CG solves use (those of the reordered copy, if any)
  const sla_csr K = solver_handle(A);
  if (kernels) *kernels = use_split(K) ? 2 : (use_lines(K) ? 3 : (use_band(K) ? 1 : 0));
  return SLA_OK;
  API_END
}

sla_status sla_csr_set_graph_block(sla_csr A, int64_t iterations) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_set_graph_block: NULL handle");
  REQUIRE(iterations >= 0 && iterations <= 4096, "sla_csr_set_graph_block: out of range");
  for (sla_csr H : {A, solver_handle(A)}) {
    if (iterations != H->graph_block) {
      (void)hipDeviceSynchronize();
      release_workspace(H);  // drops the captured graphs with the workspace
      H->graph_block = iterations;
    }
  }
  return SLA_OK;
  API_END
}

sla_status sla_csr_set_workgroups_per_cu(sla_csr A, int workgroups) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_set_workgroups_per_cu: NULL handle");
  REQUIRE(workgroups >= 0 && workgroups <= 2, "sla_csr_set_workgroups_per_cu: must be 0, 1 or 2");
  for (sla_csr H : {A, solver_handle(A)}) {
    if (workgroups != H->wg_per_cu) {
      (void)hipDeviceSynchronize();
      release_workspace(H);  // the grid sizes the partial-sum arrays and the graphs
      H->wg_per_cu = workgroups;
    }
  }
  return SLA_OK;
  API_END
}

sla_status sla_csr_set_one_group(sla_csr A, int mode) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_set_one_group: NULL handle");
  REQUIRE(mode == SLA_ONE_GROUP_AUTO || mode == SLA_ONE_GROUP_OFF,
          "sla_csr_set_one_group: unknown mode %d", mode);
  for (sla_csr H : {A, solver_handle(A)}) H->one_group = mode;
  return SLA_OK;
  API_END
}

sla_status sla_csr_reorder(sla_csr A, int ordering, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_reorder: NULL handle");
  REQUIRE(ordering == SLA_ORDER_NONE || ordering == SLA_ORDER_BFS,
          "sla_csr_reorder: unknown ordering %d", ordering);
  if (ordering == SLA_ORDER_NONE) {
    if (A->ro != nullptr) {
      SLA_TRY_HIP(hipStreamSynchronize(stream));
      (void)hipDeviceSynchronize();
      release_reorder(A);
    }
    return SLA_OK;
  }
  if (A->ro != nullptr) return SLA_OK;  // the order is a function of the pattern
  return make_reorder(A, stream);
  API_END
}

sla_status sla_csr_ordering(sla_csr A, int32_t* order_out, hipStream_t stream) {
  API_BEGIN
  clear_error();
  REQUIRE(A != nullptr, "sla_csr_ordering: NULL handle");
  REQUIRE(A->ro != nullptr, "sla_csr_ordering: the handle is not reordered (sla_csr_reorder)");
  REQUIRE(order_out != nullptr || A->n == 0, "sla_csr_ordering: NULL output");
  return copy_order(A, order_out, stream);
  API_END
}

}  // extern "C"
