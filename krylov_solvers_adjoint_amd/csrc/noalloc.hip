// The CG solve for callers that cannot allocate device memory: code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
// The solver's workspace lives in one static device array of this file,
// `scratch`; host code never passes the array's name to a kernel or a copy
// (on the host it is only a stand-in for the symbol): the array's device
// address is looked up once per device with hipGetSymbolAddress, and that
// address is what the kernels receive.  Calls on one GPU share its array, so
// calls that overlap on one GPU race.
#include <cmath>
#include <mutex>
#include <new>

#include "handle.h"

namespace sla {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // per GPU, held until the process ends
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Per-device set-up state: the array's device address, and the host copies
// of the context and the scalar record (static storage: nothing is
// allocated on the host either).
struct DeviceState {
  void* ptr = nullptr;
  Ctx ctx_host;
  Scal scal_host;
  int poll_host[2] = {0, 0};
};
DeviceState g_state[kMaxDevices];
std::mutex g_setup_mu;

// Byte offsets of the pieces of one solve's state inside the array, each
// 256-byte aligned: the context and the system's scalar record, two ints
// (the running count, the symmetry flag), the partials, r, p (two buffers), q.
struct Layout {
  size_t ctx, flags, part, r, p0, p1, q, total;
};

size_t up256(size_t v) { return (v + 255) / 256 * 256; }

Layout layout(int64_t n, int32_t grid) {
  Layout L{};
  size_t off = 0;
  L.ctx = off;
  off += up256(sizeof(Ctx) + sizeof(Scal));
  L.flags = off;
  off += 256;
  L.part = off;
  off += up256(sizeof(double) * size_t(kPartSets) * size_t(grid));
  const size_t vec = up256(sizeof(double) * size_t(n));
  L.r = off;
  off += vec;
  L.p0 = off;
  off += vec;
  L.p1 = off;
  off += vec;
  L.q = off;
  off += vec;
  L.total = off;
  return L;
}

// The device address of `scratch` on device `dev` (current), looked up on
// the first call on that device; also warms the device attribute cache the
// launch helpers read, so later calls touch no host allocator either.
sla_status scratch_on(int dev, unsigned char** out) {
  std::lock_guard<std::mutex> lock(g_setup_mu);
  DeviceState& d = g_state[dev];
  if (d.ptr == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      set_error("sla_cg_solve_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
                hipGetErrorString(e));
      return SLA_ERR_DEVICE;
    }
    (void)device_cus();
    d.ptr = p;
  }
  *out = static_cast<unsigned char*>(d.ptr);
  return SLA_OK;
}

sla_status solve_noalloc(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                         uint32_t flags, sla_cg_info* info, hipStream_t stream) {
  if (A == nullptr) {
    set_error("sla_cg_solve_noalloc: NULL handle");
    return SLA_ERR_ARG;
  }
  if (A->batch != 1) {
    set_error("sla_cg_solve_noalloc: needs exactly one system bound (%lld bound)",
              (long long)A->batch);
    return SLA_ERR_ARG;
  }
  if (b == nullptr || x == nullptr) {
    set_error("sla_cg_solve_noalloc: NULL vector");
    return SLA_ERR_ARG;
  }
  if (!std::isfinite(tol) || tol < 0.0 || maxit < 0) {
    set_error("sla_cg_solve_noalloc: tol must be finite and >= 0, maxit >= 0");
    return SLA_ERR_ARG;
  }
  if ((flags & ~uint32_t(SLA_FLAG_X0)) != 0) {
    set_error("sla_cg_solve_noalloc: only SLA_FLAG_X0 is supported (history and Jacobi "
              "preconditioning need the handle's workspace)");
    return SLA_ERR_ARG;
  }
  if (A->ro != nullptr) {
    set_error("sla_cg_solve_noalloc: the handle is reordered (sla_csr_reorder); its "
              "permuted copies need memory of their own");
    return SLA_ERR_ARG;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_error("sla_cg_solve_noalloc: no usable current device");
    return SLA_ERR_DEVICE;
  }
  const int32_t grid = solver_grid(A, 1);
  const Layout L = layout(A->n, grid);
  if (L.total > kScratchBytes) {
    set_error("sla_cg_solve_noalloc: n = %lld needs %zu bytes of scratch; the limit is %zu "
              "bytes (about %lld unknowns); use sla_cg_solve", (long long)A->n, L.total,
              kScratchBytes,
              (long long)((kScratchBytes - layout(0, grid).total) / (4 * sizeof(double))));
    return SLA_ERR_ARG;
  }
  unsigned char* base = nullptr;
  SLA_TRY(scratch_on(dev, &base));
  int* flags_dev = reinterpret_cast<int*>(base + L.flags);
  // CG needs a symmetric pattern (checked once per handle, as sla_cg_solve does)
  if (A->sym_pattern < 0) {
    int bad = 0;
    SLA_TRY(check_symmetry(A, false, &bad, stream, flags_dev + 1));
    A->sym_pattern = (bad & 1) ? 0 : 1;
  }
  if (!A->sym_pattern) {
    if (info) {
      info->iterations = 0;
      info->rel_residual = 0.0;
      info->converged = 0;
      info->status = SLA_ERR_NOT_SYMMETRIC;
    }
    set_error("sla_cg_solve_noalloc: the pattern is not symmetric; CG needs A^T = A");
    return SLA_ERR_NOT_SYMMETRIC;
  }
  DeviceState& d = g_state[dev];
  CgSpace sp;
  sp.ctx_dev = reinterpret_cast<Ctx*>(base + L.ctx);
  sp.n_running = flags_dev;
  sp.part = reinterpret_cast<double*>(base + L.part);
  sp.r = reinterpret_cast<double*>(base + L.r);
  sp.p0 = reinterpret_cast<double*>(base + L.p0);
  sp.p1 = reinterpret_cast<double*>(base + L.p1);
  sp.q = reinterpret_cast<double*>(base + L.q);
  sp.ctx_host = &d.ctx_host;
  sp.scal_host = &d.scal_host;
  sp.poll_host = d.poll_host;
  sp.poll_ev = nullptr;
  sp.grid = grid;
  sp.own = false;
  return run_cg_space(A, sp, b, x, tol, maxit, flags, info, stream);
}

}  // namespace
}  // namespace sla

extern "C" sla_status sla_cg_solve_noalloc(sla_csr A, const double* b, double* x, double tol,
                                           int64_t maxit, uint32_t flags, sla_cg_info* info_host,
                                           hipStream_t stream) {
  try {
    sla::clear_error();
    return sla::solve_noalloc(A, b, x, tol, maxit, flags, info_host, stream);
  } catch (const std::bad_alloc&) {
    sla::set_error("host out of memory");
    return SLA_ERR_OOM;
  } catch (...) {
    sla::set_error("internal error");
    return SLA_ERR_DEVICE;
  }
}
