// Internal definitions shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "sla.h"

namespace sla {

// ---------------------------------------------------------------------------
// Errors
// ---------------------------------------------------------------------------
void set_error(const char* fmt, ...);
void clear_error();

#define SLA_TRY_HIP(call)                                                      \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) {                                                    \
      ::sla::set_error("%s: %s (%s:%d)", #call, hipGetErrorString(e_),         \
                       __FILE__, __LINE__);                                    \
      return SLA_ERR_DEVICE;                                                   \
    }                                                                          \
  } while (0)

#define SLA_TRY(call)                                                          \
  do {                                                                         \
    sla_status s_ = (call);                                                    \
    if (s_ != SLA_OK) return s_;                                               \
  } while (0)

// Device allocation that reports SLA_ERR_OOM.
sla_status dev_alloc(void** p, size_t bytes, const char* what);
template <typename T>
inline sla_status dev_alloc(T** p, size_t count, const char* what) {
  return dev_alloc(reinterpret_cast<void**>(p), count * sizeof(T), what);
}
void dev_free(void* p);

// ---------------------------------------------------------------------------
// Launch geometry
// ---------------------------------------------------------------------------
constexpr int kBlock = 256;      // threads per workgroup (4 wave64)
constexpr int kTileRows = 256;   // rows per SpMV tile: one row per thread
constexpr int kWave = 64;
constexpr int kXcds = 8;         // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int64_t kLdsCapNnz = 4096;  // max staged slots per tile (48 KiB)

// Number of compute units of the current device (cached per device).
int device_cus();

// ---------------------------------------------------------------------------
// Device-side solver state
// ---------------------------------------------------------------------------
enum : int32_t {
  ST_RUNNING = 0,
  ST_CONVERGED = 1,
  ST_MAXIT = 2,
  ST_NOT_SPD = SLA_ERR_NOT_SPD,
  ST_NONFINITE = SLA_ERR_NONFINITE,
};

// Per-system CG scalars; they live on the device for the whole solve.
struct alignas(64) Scal {
  double rr;      // r_k . r_k (recursive residual)
  double bb;      // b . b
  double stop;    // (tol * tol) * bb
  double alpha;   // alpha of the last iteration whose SpMV phase finished
  double beta;    // beta used to form the next search direction
  int64_t it;     // completed iterations
  int64_t maxit;
  int32_t state;  // ST_*
  int32_t x_lag;  // 1: x still lacks alpha * p(lag_buf)
  int32_t lag_buf;
  int32_t pad;
};

// Everything the iteration kernels touch, resident in device memory so that
// a captured graph stays valid while the caller's x / b / values change.
struct Ctx {
  const void* rowptr;
  const int32_t* col;
  const double* vals;   // [batch][nnz]
  double* x;            // [batch][n] solution (lambda for the adjoint)
  const double* b;      // [batch][n] right-hand side
  double* r;            // [batch][n]
  double* p[2];         // [batch][n] search direction, double-buffered
  double* q;            // [batch][n] A p
  double* part_a;       // [batch][grid] partial p.q
  double* part_b;       // [batch][grid] partial r.r
  double* part_c;       // [batch][grid] partial b.b (set-up only)
  Scal* scal;           // [batch]
  double* hist;         // [batch][hist_cap][3] alpha, beta, rr or nullptr
  int* n_running;       // systems still iterating
  int64_t hist_cap;
  int64_t n;
  int64_t nnz;
  int64_t batch;
  int64_t tiles;        // ceil(n / kTileRows)
  int32_t grid;         // workgroups per system in the iteration kernels
  int32_t lds_cap;      // staged slots per tile (0: read slots from memory)
};

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double v) {
  // butterfly over the 64 lanes; every lane ends with the same total, and
  // the association order is fixed, so results are reproducible
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Sum over a workgroup of kBlock threads; valid in thread 0.  Fixed order.
__device__ __forceinline__ double block_sum(double v, double* lds4) {
  v = wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  if (lane == 0) lds4[w] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) t = (lds4[0] + lds4[1]) + (lds4[2] + lds4[3]);
  __syncthreads();
  return t;
}

// Tile range of workgroup `bid` of `grid`: the tiles are split into kXcds
// contiguous ranges, one per XCD (workgroup i runs on XCD i % 8), and the
// workgroups of one XCD interleave over its range, so that at any time the
// workgroups of an XCD work on neighbouring rows and share its L2.
struct TileWalk {
  int64_t first, stride, end;
};
__device__ __forceinline__ TileWalk tile_walk(int64_t tiles, int grid, int bid) {
  const int xcd = bid % kXcds;
  const int per_xcd = grid / kXcds;  // grid is a multiple of kXcds
  const int slot = bid / kXcds;
  const int64_t lo = tiles * xcd / kXcds;
  const int64_t hi = tiles * (xcd + 1) / kXcds;
  return TileWalk{lo + slot, per_xcd, hi};
}

}  // namespace sla

struct sla_csr_s;  // defined in handle.h
