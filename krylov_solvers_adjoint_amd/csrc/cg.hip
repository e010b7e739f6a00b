// CSR SpMV, the CG iteration and the adjoint pattern gradient on gfx950.
//
// Method: the torch-sla explainer (gist.science, arXiv 2601.13994),
// technical summary.  Methodology 1 names the sparse tensor's .matvec and
// .solve and the iterative CG backend; Methodology 2 (linear systems) gives
// the backward pass: solve A^T lambda = dL/dx, grad_b = lambda,
// grad_A = -lambda_i x_j on the stored pattern only.  CG is the textbook
// Hestenes-Stiefel iteration (x0 = 0, r0 = p0 = b):
//   q = A p;  alpha = rr / (p.q);  x += alpha p;  r -= alpha q;
//   rr' = r.r;  beta = rr' / rr;  p = r + beta p
//
// Layout and schedule (memory-bound: ~0.13 flop per byte, far below the fp64
// ridge, so no matrix cores):
//   * One iteration is four kernels, all reading the device-resident scalars
//     of each system; nothing comes back to the host inside the loop.
//       k_cg_spmv      p_k = r_k + beta p_{k-1}  (own rows, and recomputed at
//                      each gathered column), x += alpha_{k-1} p_{k-1} (the
//                      previous iteration's x update, deferred to this pass
//                      where p_{k-1} is read anyway), q = A p_k, partial p.q
//       k_cg_alpha     alpha = rr / sum(partials); breakdown checks
//       k_cg_residual  r -= alpha q, partial r.r
//       k_cg_beta      rr' = sum(partials); beta; stopping test; it++
//     p is double-buffered because the SpMV reads p_{k-1} at other
//     workgroups' rows while it writes p_k.  The arithmetic of every element
//     is the textbook one (each * and + rounded separately), so only the
//     order of the dot-product sums differs from a sequential CPU run.
//   * Rows are cut into tiles of 256 (one row per thread).  A tile's slots
//     [rowptr[r0], rowptr[r0+256]) are contiguous, so they are staged into LDS
//     with coalesced loads and each thread then walks its own row there.
//   * The iteration kernels run a fixed grid (8 workgroups per CU); each
//     workgroup walks tiles inside its XCD's contiguous share of the rows,
//     interleaved with the other workgroups of that XCD, so stencil
//     neighbours (rows i +- N) are read while still in that XCD's L2, and the
//     dot products have one partial per workgroup, summed in a fixed order:
//     results are bitwise reproducible.
//   * Blocks of iterations are captured once per handle as a HIP graph; each
//     kernel returns at once when its system has stopped, and the host only
//     polls the count of running systems between blocks.
#include <algorithm>
#include <cmath>

#include "handle.h"

namespace sla {
namespace {

#define LAUNCH_CHECK()                                                         \
  do {                                                                         \
    hipError_t e_ = hipGetLastError();                                         \
    if (e_ != hipSuccess) {                                                    \
      set_error("kernel launch failed: %s (%s:%d)", hipGetErrorString(e_),     \
                __FILE__, __LINE__);                                           \
      return SLA_ERR_DEVICE;                                                   \
    }                                                                          \
  } while (0)

// Row sum of one tile row: acc = sum_k vals[k] * g(col[k]) in ascending slot
// order, starting from 0.  `lv`/`lc` are LDS staging areas of lds_cap slots.
// Returns false for threads past the last row.  Contains workgroup barriers:
// every thread of the workgroup must call it for the same tile.
template <typename RP, typename G>
__device__ __forceinline__ bool tile_row(const RP* __restrict__ rowptr,
                                         const int32_t* __restrict__ col,
                                         const double* __restrict__ vals, int64_t n,
                                         int64_t tile, int lds_cap, double* lv, int32_t* lc,
                                         G g, int64_t& row, double& acc) {
  const int64_t r0 = tile * kTileRows;
  const int64_t r1 = r0 + kTileRows < n ? r0 + kTileRows : n;
  const int64_t s0 = rowptr[r0];
  const int64_t len = int64_t(rowptr[r1]) - s0;
  row = r0 + threadIdx.x;
  const bool ok = row < r1;
  int64_t a = 0, e = 0;
  if (ok) {
    a = rowptr[row];
    e = rowptr[row + 1];
  }
  acc = 0.0;
  if (len <= lds_cap) {
    for (int64_t k = threadIdx.x; k < len; k += kBlock) {
      lv[k] = vals[s0 + k];
      lc[k] = col[s0 + k];
    }
    __syncthreads();
    for (int64_t k = a - s0; k < e - s0; ++k) acc = acc + lv[k] * g(lc[k]);
    __syncthreads();
  } else {
    for (int64_t k = a; k < e; ++k) acc = acc + vals[k] * g(col[k]);
  }
  return ok;
}

// ---------------------------------------------------------------------------
// Standalone SpMV: y[s] = A_s x[s]
// ---------------------------------------------------------------------------
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_spmv(const RP* __restrict__ rowptr,
                                                 const int32_t* __restrict__ col,
                                                 const double* __restrict__ vals, int64_t n,
                                                 int64_t nnz, int64_t tiles, int lds_cap,
                                                 const double* __restrict__ x,
                                                 double* __restrict__ y) {
  extern __shared__ double lds_dyn[];
  double* lv = lds_dyn;
  int32_t* lc = reinterpret_cast<int32_t*>(lds_dyn + lds_cap);
  const int64_t s = blockIdx.y;
  const double* v = vals + s * nnz;
  const double* xs = x + s * n;
  double* ys = y + s * n;
  auto g = [&](int64_t j) { return xs[j]; };
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    int64_t i;
    double acc;
    if (tile_row<RP>(rowptr, col, v, n, t, lds_cap, lv, lc, g, i, acc)) ys[i] = acc;
  }
}

// ---------------------------------------------------------------------------
// CG kernels
// ---------------------------------------------------------------------------

// r = b (x = 0) or r = b - q with q = A x0; p_{-1} = 0; partial b.b and r.r.
__global__ __launch_bounds__(kBlock) void k_cg_init(const Ctx* __restrict__ c, int use_x0) {
  __shared__ double red[4];
  const int64_t s = blockIdx.y, n = c->n;
  const double* b = c->b + s * n;
  double* x = c->x + s * n;
  double* r = c->r + s * n;
  double* pm = c->p[1] + s * n;
  const double* q = c->q + s * n;
  const TileWalk w = tile_walk(c->tiles, c->grid, blockIdx.x);
  double bb = 0.0, rr = 0.0;
  for (int64_t t = w.first; t < w.end; t += w.stride) {
    const int64_t i = t * kTileRows + threadIdx.x;
    if (i < n) {
      const double bi = b[i];
      double ri;
      if (use_x0) {
        ri = bi - q[i];
      } else {
        ri = bi;
        x[i] = 0.0;
      }
      r[i] = ri;
      pm[i] = 0.0;
      bb = bb + bi * bi;
      rr = rr + ri * ri;
    }
  }
  bb = block_sum(bb, red);
  rr = block_sum(rr, red);
  if (threadIdx.x == 0) {
    c->part_c[s * c->grid + blockIdx.x] = bb;
    c->part_b[s * c->grid + blockIdx.x] = rr;
    if (blockIdx.x == 0 && s == 0) *c->n_running = 0;
  }
}

__device__ __forceinline__ double sum_partials(const double* __restrict__ part, int count,
                                               double* red) {
  double v = 0.0;
  for (int i = threadIdx.x; i < count; i += kBlock) v = v + part[i];
  return block_sum(v, red);
}

__global__ __launch_bounds__(kBlock) void k_cg_init_scalars(const Ctx* __restrict__ c,
                                                            double tol, int64_t maxit) {
  __shared__ double red[4];
  const int64_t s = blockIdx.x;
  const double bb = sum_partials(c->part_c + s * c->grid, c->grid, red);
  const double rr = sum_partials(c->part_b + s * c->grid, c->grid, red);
  if (threadIdx.x == 0) {
    Scal* sc = c->scal + s;
    sc->rr = rr;
    sc->bb = bb;
    sc->stop = (tol * tol) * bb;
    sc->alpha = 0.0;
    sc->beta = 0.0;
    sc->it = 0;
    sc->maxit = maxit;
    sc->x_lag = 0;
    sc->lag_buf = 0;
    int32_t st = ST_RUNNING;
    if (!isfinite(bb) || !isfinite(rr)) st = ST_NONFINITE;
    else if (rr <= sc->stop) st = ST_CONVERGED;
    else if (maxit <= 0) st = ST_MAXIT;
    sc->state = st;
    if (st == ST_RUNNING) atomicAdd(c->n_running, 1);
  }
}

template <typename RP>
__global__ __launch_bounds__(kBlock) void k_cg_spmv(const Ctx* __restrict__ c) {
  extern __shared__ double lds_dyn[];
  __shared__ double red[4];
  const int64_t s = blockIdx.y;
  const Scal* sc = c->scal + s;
  if (sc->state != ST_RUNNING) return;
  const int64_t n = c->n;
  const int64_t it = sc->it;
  const double beta = sc->beta;
  const double alpha = sc->alpha;
  const bool lag = sc->x_lag != 0;
  const RP* rowptr = static_cast<const RP*>(c->rowptr);
  const double* vals = c->vals + s * c->nnz;
  const double* r = c->r + s * n;
  const double* pold = c->p[(it + 1) & 1] + s * n;
  double* pnew = c->p[it & 1] + s * n;
  double* x = c->x + s * n;
  double* q = c->q + s * n;
  double* lv = lds_dyn;
  int32_t* lc = reinterpret_cast<int32_t*>(lds_dyn + c->lds_cap);
  auto g = [&](int64_t j) { return r[j] + beta * pold[j]; };
  const TileWalk w = tile_walk(c->tiles, c->grid, blockIdx.x);
  double pq = 0.0;
  for (int64_t t = w.first; t < w.end; t += w.stride) {
    int64_t i;
    double acc;
    if (tile_row<RP>(rowptr, c->col, vals, n, t, c->lds_cap, lv, lc, g, i, acc)) {
      const double po = pold[i];
      const double pn = r[i] + beta * po;
      if (lag) x[i] = x[i] + alpha * po;
      pnew[i] = pn;
      q[i] = acc;
      pq = pq + pn * acc;
    }
  }
  pq = block_sum(pq, red);
  if (threadIdx.x == 0) c->part_a[s * c->grid + blockIdx.x] = pq;
}

__global__ __launch_bounds__(kBlock) void k_cg_alpha(const Ctx* __restrict__ c) {
  __shared__ double red[4];
  const int64_t s = blockIdx.x;
  Scal* sc = c->scal + s;
  if (sc->state != ST_RUNNING) return;
  const double pq = sum_partials(c->part_a + s * c->grid, c->grid, red);
  if (threadIdx.x == 0) {
    if (!isfinite(pq)) {
      sc->state = ST_NONFINITE;
      sc->x_lag = 0;
      atomicSub(c->n_running, 1);
    } else if (!(pq > 0.0)) {
      sc->state = ST_NOT_SPD;
      sc->x_lag = 0;
      atomicSub(c->n_running, 1);
    } else {
      sc->alpha = sc->rr / pq;
      sc->x_lag = 1;
      sc->lag_buf = int32_t(sc->it & 1);
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_cg_residual(const Ctx* __restrict__ c) {
  __shared__ double red[4];
  const int64_t s = blockIdx.y;
  const Scal* sc = c->scal + s;
  if (sc->state != ST_RUNNING) return;
  const int64_t n = c->n;
  const double alpha = sc->alpha;
  double* r = c->r + s * n;
  const double* q = c->q + s * n;
  const TileWalk w = tile_walk(c->tiles, c->grid, blockIdx.x);
  double rr = 0.0;
  for (int64_t t = w.first; t < w.end; t += w.stride) {
    const int64_t i = t * kTileRows + threadIdx.x;
    if (i < n) {
      const double ri = r[i] - alpha * q[i];
      r[i] = ri;
      rr = rr + ri * ri;
    }
  }
  rr = block_sum(rr, red);
  if (threadIdx.x == 0) c->part_b[s * c->grid + blockIdx.x] = rr;
}

__global__ __launch_bounds__(kBlock) void k_cg_beta(const Ctx* __restrict__ c) {
  __shared__ double red[4];
  const int64_t s = blockIdx.x;
  Scal* sc = c->scal + s;
  if (sc->state != ST_RUNNING) return;
  const double rr_new = sum_partials(c->part_b + s * c->grid, c->grid, red);
  if (threadIdx.x == 0) {
    if (!isfinite(rr_new)) {
      sc->state = ST_NONFINITE;  // x still lacks alpha p: the finalize adds it
      atomicSub(c->n_running, 1);
      return;
    }
    const double beta = rr_new / sc->rr;
    const int64_t it = sc->it;
    if (c->hist != nullptr && it < c->hist_cap) {
      double* h = c->hist + (s * c->hist_cap + it) * 3;
      h[0] = sc->alpha;
      h[1] = beta;
      h[2] = rr_new;
    }
    sc->beta = beta;
    sc->rr = rr_new;
    sc->it = it + 1;
    if (rr_new <= sc->stop) {
      sc->state = ST_CONVERGED;
      atomicSub(c->n_running, 1);
    } else if (it + 1 >= sc->maxit) {
      sc->state = ST_MAXIT;
      atomicSub(c->n_running, 1);
    }
  }
}

// x += alpha p for the last iteration (deferred from the SpMV pass).
__global__ __launch_bounds__(kBlock) void k_cg_finalize(const Ctx* __restrict__ c) {
  const int64_t s = blockIdx.y;
  const Scal* sc = c->scal + s;
  if (sc->x_lag == 0) return;
  const int64_t n = c->n;
  const double alpha = sc->alpha;
  const double* p = c->p[sc->lag_buf] + s * n;
  double* x = c->x + s * n;
  const TileWalk w = tile_walk(c->tiles, c->grid, blockIdx.x);
  for (int64_t t = w.first; t < w.end; t += w.stride) {
    const int64_t i = t * kTileRows + threadIdx.x;
    if (i < n) x[i] = x[i] + alpha * p[i];
  }
}

// grad_vals[s][k] = -lambda[s][i] * x[s][col[k]] for every stored slot k of row i
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_pattern_grad(const RP* __restrict__ rowptr,
                                                         const int32_t* __restrict__ col,
                                                         int64_t n, int64_t nnz,
                                                         const double* __restrict__ lambda,
                                                         const double* __restrict__ x,
                                                         double* __restrict__ grad) {
  const int64_t s = blockIdx.y;
  const double* l = lambda + s * n;
  const double* xs = x + s * n;
  double* gs = grad + s * nnz;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x) {
    const double li = l[i];
    const int64_t a = rowptr[i], e = rowptr[i + 1];
    for (int64_t k = a; k < e; ++k) gs[k] = -(li * xs[col[k]]);
  }
}

size_t lds_bytes(const sla_csr A) { return size_t(A->lds_cap) * (sizeof(double) + sizeof(int32_t)); }

template <typename RP>
sla_status enqueue_iteration(sla_csr A, int64_t batch, hipStream_t st) {
  const dim3 grid2(unsigned(A->grid), unsigned(batch));
  k_cg_spmv<RP><<<grid2, kBlock, lds_bytes(A), st>>>(A->ctx_dev);
  k_cg_alpha<<<unsigned(batch), kBlock, 0, st>>>(A->ctx_dev);
  k_cg_residual<<<grid2, kBlock, 0, st>>>(A->ctx_dev);
  k_cg_beta<<<unsigned(batch), kBlock, 0, st>>>(A->ctx_dev);
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status enqueue_block(sla_csr A, int64_t batch, int64_t iters, hipStream_t st) {
  for (int64_t k = 0; k < iters; ++k) {
    if (A->rp_idx == SLA_I32) SLA_TRY(enqueue_iteration<int32_t>(A, batch, st));
    else SLA_TRY(enqueue_iteration<int64_t>(A, batch, st));
  }
  return SLA_OK;
}

sla_status get_graph(sla_csr A, int64_t batch, hipGraphExec_t* exec) {
  auto it = A->graphs.find(batch);
  if (it != A->graphs.end()) {
    *exec = it->second.second;
    return SLA_OK;
  }
  if (A->capture_stream == nullptr) SLA_TRY_HIP(hipStreamCreateWithFlags(&A->capture_stream,
                                                                         hipStreamNonBlocking));
  hipGraph_t g = nullptr;
  hipGraphExec_t e = nullptr;
  SLA_TRY_HIP(hipStreamBeginCapture(A->capture_stream, hipStreamCaptureModeThreadLocal));
  sla_status s = enqueue_block(A, batch, A->graph_block, A->capture_stream);
  hipError_t he = hipStreamEndCapture(A->capture_stream, &g);
  if (s != SLA_OK) {
    if (g) (void)hipGraphDestroy(g);
    return s;
  }
  if (he != hipSuccess) {
    set_error("graph capture failed: %s", hipGetErrorString(he));
    return SLA_ERR_DEVICE;
  }
  he = hipGraphInstantiate(&e, g, nullptr, nullptr, 0);
  if (he != hipSuccess) {
    (void)hipGraphDestroy(g);
    set_error("graph instantiation failed: %s", hipGetErrorString(he));
    return SLA_ERR_DEVICE;
  }
  A->graphs[batch] = {g, e};
  *exec = e;
  return SLA_OK;
}

void drop_graphs(sla_csr A) {
  for (auto& kv : A->graphs) {
    (void)hipGraphExecDestroy(kv.second.second);
    (void)hipGraphDestroy(kv.second.first);
  }
  A->graphs.clear();
}

}  // namespace

// ---------------------------------------------------------------------------
// Workspace
// ---------------------------------------------------------------------------
void release_workspace(sla_csr A) {
  drop_graphs(A);
  dev_free(A->r);
  dev_free(A->p0);
  dev_free(A->p1);
  dev_free(A->q);
  dev_free(A->part);
  dev_free(A->scal);
  dev_free(A->n_running);
  dev_free(A->ctx_dev);
  dev_free(A->hist);
  if (A->ctx_host) (void)hipHostFree(A->ctx_host);
  if (A->scal_host) (void)hipHostFree(A->scal_host);
  if (A->poll_host) (void)hipHostFree(A->poll_host);
  for (auto& e : A->poll_ev)
    if (e) (void)hipEventDestroy(e);
  if (A->capture_stream) (void)hipStreamDestroy(A->capture_stream);
  A->r = A->p0 = A->p1 = A->q = A->part = A->hist = nullptr;
  A->scal = nullptr;
  A->scal_host = nullptr;
  A->n_running = nullptr;
  A->ctx_dev = nullptr;
  A->ctx_host = nullptr;
  A->poll_host = nullptr;
  A->poll_ev[0] = A->poll_ev[1] = nullptr;
  A->capture_stream = nullptr;
  A->ws_batch = 0;
  A->hist_cap = A->hist_batch = 0;
}

sla_status ensure_workspace(sla_csr A, int64_t batch) {
  if (A->ws_batch == batch && A->r != nullptr) return SLA_OK;
  release_workspace(A);
  const int64_t n = A->n;
  // iteration grid: about 8 workgroups per CU in total, a multiple of the
  // XCD count per system, never more than the tiles need (rounded up)
  const int64_t target = std::max<int64_t>(kXcds, int64_t(device_cus()) * 8 / batch);
  int64_t g = std::min<int64_t>(A->tiles, target);
  g = (g + kXcds - 1) / kXcds * kXcds;
  A->grid = int32_t(std::max<int64_t>(g, kXcds));
  const size_t vec = size_t(batch) * size_t(n);
  SLA_TRY(dev_alloc(&A->r, vec, "r"));
  SLA_TRY(dev_alloc(&A->p0, vec, "p"));
  SLA_TRY(dev_alloc(&A->p1, vec, "p"));
  SLA_TRY(dev_alloc(&A->q, vec, "q"));
  SLA_TRY(dev_alloc(&A->part, size_t(3) * batch * A->grid, "partials"));
  SLA_TRY(dev_alloc(&A->scal, batch, "scalars"));
  SLA_TRY(dev_alloc(&A->n_running, 1, "running count"));
  SLA_TRY(dev_alloc(&A->ctx_dev, 1, "context"));
  SLA_TRY_HIP(hipHostMalloc(reinterpret_cast<void**>(&A->ctx_host), sizeof(Ctx)));
  SLA_TRY_HIP(hipHostMalloc(reinterpret_cast<void**>(&A->scal_host), sizeof(Scal) * batch));
  SLA_TRY_HIP(hipHostMalloc(reinterpret_cast<void**>(&A->poll_host), sizeof(int) * 2));
  for (auto& e : A->poll_ev) SLA_TRY_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  A->ws_batch = batch;
  return SLA_OK;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
sla_status launch_spmv(sla_csr A, const double* vals, int64_t batch, const double* x, double* y,
                       hipStream_t st) {
  if (A->n == 0) return SLA_OK;
  const int64_t target = std::max<int64_t>(1, int64_t(device_cus()) * 8 / batch);
  const dim3 grid(unsigned(std::min<int64_t>(A->tiles, std::max<int64_t>(target, 1))),
                  unsigned(batch));
  if (A->rp_idx == SLA_I32)
    k_spmv<int32_t><<<grid, kBlock, lds_bytes(A), st>>>(
        (const int32_t*)A->rowptr, A->col, vals, A->n, A->nnz, A->tiles, A->lds_cap, x, y);
  else
    k_spmv<int64_t><<<grid, kBlock, lds_bytes(A), st>>>(
        (const int64_t*)A->rowptr, A->col, vals, A->n, A->nnz, A->tiles, A->lds_cap, x, y);
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status launch_pattern_grad(sla_csr A, int64_t batch, const double* lambda, const double* x,
                               double* grad_vals, hipStream_t st) {
  if (A->n == 0) return SLA_OK;
  const dim3 grid(unsigned(std::min<int64_t>((A->n + kBlock - 1) / kBlock, 1 << 20)),
                  unsigned(batch));
  if (A->rp_idx == SLA_I32)
    k_pattern_grad<int32_t><<<grid, kBlock, 0, st>>>((const int32_t*)A->rowptr, A->col, A->n,
                                                     A->nnz, lambda, x, grad_vals);
  else
    k_pattern_grad<int64_t><<<grid, kBlock, 0, st>>>((const int64_t*)A->rowptr, A->col, A->n,
                                                     A->nnz, lambda, x, grad_vals);
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status run_cg(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                  uint32_t flags, sla_cg_info* info, hipStream_t st) {
  const int64_t batch = A->batch;
  SLA_TRY(ensure_workspace(A, batch));
  const bool want_hist = (flags & SLA_FLAG_HISTORY) != 0;
  if (want_hist) {
    const int64_t cap = std::max<int64_t>(1, maxit);
    if (A->hist == nullptr || A->hist_cap < cap || A->hist_batch < batch) {
      dev_free(A->hist);
      A->hist = nullptr;
      SLA_TRY(dev_alloc(&A->hist, size_t(batch) * cap * 3, "history"));
      A->hist_cap = cap;
      A->hist_batch = batch;
    }
  }
  Ctx& c = *A->ctx_host;
  c.rowptr = A->rowptr;
  c.col = A->col;
  c.vals = A->vals;
  c.x = x;
  c.b = b;
  c.r = A->r;
  c.p[0] = A->p0;
  c.p[1] = A->p1;
  c.q = A->q;
  c.part_a = A->part;
  c.part_b = A->part + size_t(batch) * A->grid;
  c.part_c = A->part + size_t(2) * batch * A->grid;
  c.scal = A->scal;
  c.hist = want_hist ? A->hist : nullptr;
  c.hist_cap = want_hist ? A->hist_cap : 0;
  c.n_running = A->n_running;
  c.n = A->n;
  c.nnz = A->nnz;
  c.batch = batch;
  c.tiles = A->tiles;
  c.grid = A->grid;
  c.lds_cap = A->lds_cap;
  SLA_TRY_HIP(hipMemcpyAsync(A->ctx_dev, A->ctx_host, sizeof(Ctx), hipMemcpyHostToDevice, st));

  const bool x0 = (flags & SLA_FLAG_X0) != 0;
  if (x0) SLA_TRY(launch_spmv(A, A->vals, batch, x, A->q, st));  // q = A x0
  const dim3 grid2(unsigned(A->grid), unsigned(batch));
  k_cg_init<<<grid2, kBlock, 0, st>>>(A->ctx_dev, x0 ? 1 : 0);
  k_cg_init_scalars<<<unsigned(batch), kBlock, 0, st>>>(A->ctx_dev, tol, maxit);
  LAUNCH_CHECK();
  SLA_TRY_HIP(hipMemcpyAsync(A->poll_host, A->n_running, sizeof(int), hipMemcpyDeviceToHost,
                             st));
  SLA_TRY_HIP(hipStreamSynchronize(st));

  if (A->poll_host[0] > 0) {
    const int64_t K = A->graph_block > 0 ? A->graph_block : 16;
    const int64_t nblocks = (maxit + K - 1) / K;
    hipGraphExec_t exec = nullptr;
    if (A->graph_block > 0) SLA_TRY(get_graph(A, batch, &exec));
    for (int64_t j = 0; j < nblocks; ++j) {
      if (exec) SLA_TRY_HIP(hipGraphLaunch(exec, st));
      else SLA_TRY(enqueue_block(A, batch, K, st));
      SLA_TRY_HIP(hipMemcpyAsync(A->poll_host + (j & 1), A->n_running, sizeof(int),
                                 hipMemcpyDeviceToHost, st));
      SLA_TRY_HIP(hipEventRecord(A->poll_ev[j & 1], st));
      if (j >= 1) {
        // wait for the previous block only, so one block is always queued
        SLA_TRY_HIP(hipEventSynchronize(A->poll_ev[(j - 1) & 1]));
        if (A->poll_host[(j - 1) & 1] == 0) break;
      }
    }
  }
  k_cg_finalize<<<grid2, kBlock, 0, st>>>(A->ctx_dev);
  LAUNCH_CHECK();
  SLA_TRY_HIP(hipMemcpyAsync(A->scal_host, A->scal, sizeof(Scal) * batch,
                             hipMemcpyDeviceToHost, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));

  sla_status first = SLA_OK;
  for (int64_t s = 0; s < batch; ++s) {
    const Scal& sc = A->scal_host[s];
    const sla_status ss = sc.state >= SLA_ERR_NOT_SPD ? sla_status(sc.state) : SLA_OK;
    if (info) {
      info[s].iterations = sc.it;
      info[s].rel_residual = sc.bb > 0 ? std::sqrt(sc.rr / sc.bb) : 0.0;
      info[s].converged = (ss == SLA_OK && sc.rr <= sc.stop) ? 1 : 0;
      info[s].status = ss;
    }
    if (ss != SLA_OK && first == SLA_OK) first = ss;
  }
  if (first != SLA_OK)
    set_error("CG stopped: %s", first == SLA_ERR_NOT_SPD ? "p.Ap <= 0 (matrix not SPD)"
                                                         : "non-finite value");
  return first;
}

}  // namespace sla
