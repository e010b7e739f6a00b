// BiCGStab for non-symmetric systems (a CPU backend solver named by the
// torch-sla summary, Methodology 1) and its adjoint (Methodology 2, linear
// systems: A^T lambda = dL/dx, gradient -lambda_i x_j on the pattern).
//
// The method, without preconditioner:
//   r = b - A x0, rhat = r, p = v = 0, rho_prev = alpha = omega = 1;
//   each iteration j:
//     rho = rhat.r; beta = (rho / rho_prev)(alpha / omega)
//     p = r + beta (p - omega v)                      k_bs_direction
//     v = A p and the rhat.v partials                  the library's SpMV
//     alpha = rho / rhat.v; s = r - alpha v, s.s       k_bs_s
//     t = A s and the t.s, t.t partials                the library's SpMV
//     s.s <= tol^2 b.b: x += alpha p, done; else
//     omega = t.s / t.t; x = (x + alpha p) + omega s; r = s - omega t;
//     rhat.r and r.r partials                          k_bs_update
// Every kernel's workgroups first sum the previous kernel's partials (one
// per workgroup) themselves, in one fixed order, so all of them take the
// same decisions from the same bits, and no reduction kernel or
// cross-workgroup signal is needed.
//
// Iteration index and stopping live in device memory, so a block of
// iterations can be captured once as a HIP graph and replayed.
// k_bs_direction reads the next iteration's index jn (written only by
// k_bs_update) and publishes it as jc for the other kernels of the
// iteration.  A kernel that ends the solve stores its position 8 jc + phase;
// a later kernel of the same iteration sees a smaller position and returns,
// while the workgroups of the stopping launch itself see their own position
// and still finish its work (the x update of a half-step finish, the update
// before an omega = 0 breakdown).  The next k_bs_direction that finds a stop
// raises `halted`, which every later kernel checks first.
#include <cmath>
#include <vector>

#include "handle.h"

namespace sla {

namespace {

constexpr int kBsBlock = kIterBlock;  // 16 waves
enum : int { P_RHR = 0, P_RR, P_RV, P_SS, P_TT, P_TS, P_BB, kBsSets };
enum : int { PH_DIR = 0, PH_S = 1, PH_UPD = 2 };
constexpr int64_t kNoStop = INT64_MAX;

struct alignas(64) BsScal {
  double rho;       // rhat.r of the current iteration        (k_bs_direction)
  double rho_prev;  //                                          (k_bs_update)
  double alpha;     //                                          (k_bs_s)
  double omega;     //                                          (k_bs_update)
  double bb;        // b.b                                      (set-up)
  double stop;      // tol^2 b.b                                (set-up)
  double rr;        // residual norm squared, last known        (k_bs_direction, k_bs_update)
  int64_t it;       // completed iterations                     (k_bs_update)
  int64_t stop_pos; // 8 jc + phase of the stopping kernel, or kNoStop
  int64_t jn;       // index of the next iteration              (k_bs_update)
  int64_t jc;       // index of the current iteration           (k_bs_direction)
  int64_t maxit;    //                                          (set-up)
  int32_t status;   // ST_* of the stop
  int32_t halted;   // a stop was seen by a later iteration     (k_bs_direction)
};

struct BsArgs {
  int64_t n, G;
  const double* b;
  double* x;
  double* r;
  double* rh;
  double* p;
  double* v;
  double* s;
  double* t;
  double* part;     // [batch][kBsSets][G]
  BsScal* scal;     // [batch]
  double* hist;     // [batch][hist_cap][4] rho, alpha, omega, rr, or nullptr
  int64_t hist_cap;
};

__device__ __forceinline__ int64_t stop_pos_of(const BsScal* sc) {
  return __hip_atomic_load(&sc->stop_pos, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Kernels after the head of an iteration: return when the solve has halted
// or stopped at an earlier position of this iteration.
__device__ __forceinline__ bool skip(const BsScal* sc, int phase, int64_t* j) {
  if (sc->halted) return true;
  *j = sc->jc;
  return stop_pos_of(sc) < 8 * *j + phase;
}

// Workgroup stop: one thread records the position and status.
__device__ __forceinline__ void set_stop(BsScal* sc, int64_t pos, int32_t status) {
  sc->status = status;
  __hip_atomic_store(&sc->stop_pos, pos, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The G partials of one set, summed in the same order by every workgroup.
__device__ __forceinline__ double sum_set(const double* part, int64_t G, double* red) {
  double a = 0.0;
  for (int64_t g = threadIdx.x; g < G; g += kBsBlock) a = a + part[g];
  return block_sum_all<kBsBlock>(a, red);
}

__device__ __forceinline__ void put_partial(double* part, double v, double* red) {
  v = block_sum_all<kBsBlock>(v, red);
  if (threadIdx.x == 0) part[blockIdx.x] = v;
}

// One-shot forms for an LDS area that the launch uses for no other sum: no
// closing barrier (see block_sum_once).
__device__ __forceinline__ double sum_set_once(const double* part, int64_t G, double* red) {
  double a = 0.0;
  for (int64_t g = threadIdx.x; g < G; g += kBsBlock) a = a + part[g];
  return block_sum_once<kBsBlock>(a, red);
}

__device__ __forceinline__ void put_partial_once(double* part, double v, double* red) {
  v = block_sum_once<kBsBlock>(v, red);
  if (threadIdx.x == 0) part[blockIdx.x] = v;
}

constexpr int kBsWaves = kBsBlock / kWave;

// K sets of G partials summed in one pass: the same order as K calls of
// sum_set (each thread's strided terms, a wave butterfly, the waves in
// order).  Thread k adds set k's wave sums and broadcasts the total through
// LDS.  red holds K * (kBsWaves + 1) doubles, an area that the launch uses
// for no other sum (there is no closing barrier).
template <int K>
__device__ __forceinline__ void sum_sets(const double* const (&p)[K], int64_t G, double* red,
                                         double (&out)[K]) {
  double a[K];
#pragma unroll
  for (int k = 0; k < K; ++k) a[k] = 0.0;
  for (int64_t g = threadIdx.x; g < G; g += kBsBlock) {
#pragma unroll
    for (int k = 0; k < K; ++k) a[k] = a[k] + p[k][g];
  }
  const int wave = int(threadIdx.x) / kWave;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    a[k] = wave_sum(a[k]);
    if ((threadIdx.x & (kWave - 1)) == 0) red[k * kBsWaves + wave] = a[k];
  }
  __syncthreads();
  if (threadIdx.x < K) {
    const int k = int(threadIdx.x);
    double t = 0.0;
    for (int q = 0; q < kBsWaves; ++q) t = t + red[k * kBsWaves + q];
    red[K * kBsWaves + k] = t;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) out[k] = red[K * kBsWaves + k];
}

// K per-workgroup partials written in one pass (same order as put_partial).
template <int K>
__device__ __forceinline__ void put_partials(double* const (&part)[K], const double (&v)[K],
                                             double* red) {
  const int wave = int(threadIdx.x) / kWave;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const double a = wave_sum(v[k]);
    if ((threadIdx.x & (kWave - 1)) == 0) red[k * kBsWaves + wave] = a;
  }
  __syncthreads();
  if (threadIdx.x < K) {
    const int k = int(threadIdx.x);
    double t = 0.0;
    for (int q = 0; q < kBsWaves; ++q) t = t + red[k * kBsWaves + q];
    part[k][blockIdx.x] = t;
  }
}

__device__ __forceinline__ double* hist_of(const BsArgs& a, int64_t sys) {
  return a.hist ? a.hist + sys * a.hist_cap * 4 : nullptr;
}

// r = b - A x0 (q holds A x0) or r = b with x = 0; rhat = r; p = v = 0;
// partials of b.b, rhat.r, r.r.
__global__ __launch_bounds__(kBsBlock) __attribute__((amdgpu_waves_per_eu(kWavesPerEu))) void k_bs_init(BsArgs a, const double* __restrict__ q,
                                                      int use_x0) {
  __shared__ double red[kBsBlock / kWave];
  const int64_t sys = blockIdx.y, n = a.n, o = sys * n;
  double bb = 0.0, rr = 0.0;
  for (int64_t i = int64_t(blockIdx.x) * kBsBlock + threadIdx.x; i < n;
       i += a.G * kBsBlock) {
    const double bi = a.b[o + i];
    double ri;
    if (use_x0) {
      ri = bi - q[o + i];
    } else {
      ri = bi;
      a.x[o + i] = 0.0;
    }
    a.r[o + i] = ri;
    a.rh[o + i] = ri;
    a.p[o + i] = 0.0;
    a.v[o + i] = 0.0;
    bb = bb + bi * bi;
    rr = rr + ri * ri;
  }
  double* part = a.part + sys * kBsSets * a.G;
  put_partial(part + P_BB * a.G, bb, red);
  put_partial(part + P_RR * a.G, rr, red);
  put_partial(part + P_RHR * a.G, rr, red);
}

__global__ __launch_bounds__(kBsBlock) void k_bs_init_scalars(BsArgs a, double tol, int64_t maxit) {
  __shared__ double red[kBsBlock / kWave];
  const int64_t sys = blockIdx.x;
  const double* part = a.part + sys * kBsSets * a.G;
  const double bb = sum_set(part + P_BB * a.G, a.G, red);
  const double rr = sum_set(part + P_RR * a.G, a.G, red);
  if (threadIdx.x == 0) {
    BsScal* sc = a.scal + sys;
    sc->rho = 0.0;
    sc->rho_prev = 1.0;
    sc->alpha = 1.0;
    sc->omega = 1.0;
    sc->bb = bb;
    sc->stop = (tol * tol) * bb;
    sc->rr = rr;
    sc->it = 0;
    sc->jn = 0;
    sc->jc = 0;
    sc->maxit = maxit;
    sc->halted = 0;
    sc->status = ST_RUNNING;
    sc->stop_pos = kNoStop;
    if (!isfinite(bb) || !isfinite(rr)) set_stop(sc, -1, ST_NONFINITE);
  }
}

// Head of iteration j = jn: the stopping tests on r.r, rho = rhat.r, beta
// and p = r + beta (p - omega v).  Launched once more after the last
// iteration to close the solve (it then only tests).
__global__ __launch_bounds__(kBsBlock) __attribute__((amdgpu_waves_per_eu(kWavesPerEu))) void k_bs_direction(BsArgs a) {
  const int64_t sys = blockIdx.y, n = a.n, o = sys * n;
  BsScal* sc = a.scal + sys;
  if (sc->halted) return;
  if (stop_pos_of(sc) != kNoStop) {
    // stopped in an earlier iteration (or by workgroup 0 of this launch,
    // after the same tests this workgroup would make)
    if (blockIdx.x == 0 && threadIdx.x == 0) sc->halted = 1;
    return;
  }
  const int64_t j = sc->jn, maxit = sc->maxit;
  const int64_t pos = 8 * j + PH_DIR;
  const double* part = a.part + sys * kBsSets * a.G;
  __shared__ double red2[2 * (kBsWaves + 1)];
  double sums[2];
  sum_sets<2>({part + P_RHR * a.G, part + P_RR * a.G}, a.G, red2, sums);
  const double rho = sums[0], rr = sums[1];
  int32_t st = ST_RUNNING;
  if (!isfinite(rr)) st = ST_NONFINITE;
  else if (rr <= sc->stop) st = ST_CONVERGED;
  else if (j >= maxit) st = ST_MAXIT;
  else if (!isfinite(rho)) st = ST_NONFINITE;
  else if (rho == 0.0) st = ST_BREAKDOWN;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    sc->rr = rr;
    sc->jc = j;
    double* h = hist_of(a, sys);
    if (h && j >= 1 && j - 1 < a.hist_cap) h[(j - 1) * 4 + 3] = rr;
    if (st != ST_RUNNING) set_stop(sc, pos, st);
    else sc->rho = rho;
  }
  if (st != ST_RUNNING) return;
  const double beta = (rho / sc->rho_prev) * (sc->alpha / sc->omega);
  const double om = sc->omega;
  for (int64_t i = int64_t(blockIdx.x) * kBsBlock + threadIdx.x; i < n;
       i += a.G * kBsBlock)
    a.p[o + i] = a.r[o + i] + beta * (a.p[o + i] - om * a.v[o + i]);
}

// alpha = rho / rhat.v; s = r - alpha v and the s.s partials.
__global__ __launch_bounds__(kBsBlock) __attribute__((amdgpu_waves_per_eu(kWavesPerEu))) void k_bs_s(BsArgs a) {
  __shared__ double red[2 * kBsWaves];  // the rhat.v sum, the s.s partial
  const int64_t sys = blockIdx.y, n = a.n, o = sys * n;
  BsScal* sc = a.scal + sys;
  int64_t j;
  if (skip(sc, PH_S, &j)) return;
  const int64_t pos = 8 * j + PH_S;
  const double* part = a.part + sys * kBsSets * a.G;
  const double rv = sum_set_once(part + P_RV * a.G, a.G, red);
  int32_t st = ST_RUNNING;
  if (!isfinite(rv)) st = ST_NONFINITE;
  else if (rv == 0.0) st = ST_BREAKDOWN;
  const double alpha = sc->rho / rv;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    if (st != ST_RUNNING) {
      set_stop(sc, pos, st);
    } else {
      sc->alpha = alpha;
      double* h = hist_of(a, sys);
      if (h && j < a.hist_cap) {
        h[j * 4 + 0] = sc->rho;
        h[j * 4 + 1] = alpha;
      }
    }
  }
  if (st != ST_RUNNING) return;
  double ss = 0.0;
  for (int64_t i = int64_t(blockIdx.x) * kBsBlock + threadIdx.x; i < n;
       i += a.G * kBsBlock) {
    const double si = a.r[o + i] - alpha * a.v[o + i];
    a.s[o + i] = si;
    ss = ss + si * si;
  }
  put_partial_once(a.part + (sys * kBsSets + P_SS) * a.G, ss, red + kBsWaves);
}

// After t = A s: the half-step finish (s.s <= tol^2 b.b: x += alpha p), else
// omega = t.s / t.t; x = (x + alpha p) + omega s; r = s - omega t; the
// rhat.r and r.r partials of the next iteration.
__global__ __launch_bounds__(kBsBlock) __attribute__((amdgpu_waves_per_eu(kWavesPerEu))) void k_bs_update(BsArgs a) {
  const int64_t sys = blockIdx.y, n = a.n, o = sys * n;
  BsScal* sc = a.scal + sys;
  int64_t j;
  if (skip(sc, PH_UPD, &j)) return;
  const int64_t pos = 8 * j + PH_UPD;
  const double* part = a.part + sys * kBsSets * a.G;
  __shared__ double red3[3 * (kBsWaves + 1)], redp[2 * kBsWaves];
  double sums[3];
  sum_sets<3>({part + P_SS * a.G, part + P_TT * a.G, part + P_TS * a.G}, a.G, red3, sums);
  const double ss = sums[0];
  if (!isfinite(ss)) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_stop(sc, pos, ST_NONFINITE);
    return;
  }
  if (ss <= sc->stop) {
    const double alpha = sc->alpha;
    for (int64_t i = int64_t(blockIdx.x) * kBsBlock + threadIdx.x; i < n;
         i += a.G * kBsBlock)
      a.x[o + i] = a.x[o + i] + alpha * a.p[o + i];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      sc->rr = ss;
      sc->it = j + 1;
      double* h = hist_of(a, sys);
      if (h && j < a.hist_cap) {
        h[j * 4 + 2] = 0.0;
        h[j * 4 + 3] = ss;
      }
      set_stop(sc, pos, ST_CONVERGED);
    }
    return;
  }
  const double tt = sums[1], ts = sums[2];
  int32_t st = ST_RUNNING;
  if (!isfinite(tt) || !isfinite(ts)) st = ST_NONFINITE;
  else if (tt == 0.0) st = ST_BREAKDOWN;
  if (st != ST_RUNNING) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_stop(sc, pos, st);
    return;
  }
  const double omega = ts / tt;
  const double alpha = sc->alpha;
  double rhr = 0.0, rr = 0.0;
  for (int64_t i = int64_t(blockIdx.x) * kBsBlock + threadIdx.x; i < n;
       i += a.G * kBsBlock) {
    const double si = a.s[o + i];
    a.x[o + i] = (a.x[o + i] + alpha * a.p[o + i]) + omega * si;
    const double ri = si - omega * a.t[o + i];
    a.r[o + i] = ri;
    rhr = rhr + a.rh[o + i] * ri;
    rr = rr + ri * ri;
  }
  double* wpart = a.part + sys * kBsSets * a.G;
  put_partials<2>({wpart + P_RHR * a.G, wpart + P_RR * a.G}, {rhr, rr}, redp);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    sc->it = j + 1;
    double* h = hist_of(a, sys);
    if (h && j < a.hist_cap) h[j * 4 + 2] = omega;
    if (omega == 0.0) {
      set_stop(sc, pos, ST_BREAKDOWN);
    } else {
      sc->omega = omega;
      sc->rho_prev = sc->rho;
      sc->jn = j + 1;
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// iterations per captured graph
constexpr int64_t kBsGraphIters = 16;

struct BsWork {
  int64_t cap_n = 0, cap_batch = 0, cap_g = 0;
  double* vec = nullptr;    // [6][batch][n]: r, rhat, p, v, s, t
  double* part = nullptr;   // [batch][kBsSets][G]
  BsScal* scal = nullptr;   // [batch]
  BsScal* scal_host = nullptr;  // pinned [3][batch]: final copy, two poll copies
  hipEvent_t poll_ev[2] = {nullptr, nullptr};
  // the captured block of iterations and what its kernel arguments bake in
  hipStream_t capture_stream = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  const void* key_pattern = nullptr;
  const void* key_vals = nullptr;
  const void* key_x = nullptr;
  const void* key_hist = nullptr;
  int64_t key_batch = 0, key_g = 0, key_hcap = 0;
  double* hist = nullptr;   // [batch][hist_cap][4]
  int64_t hist_cap = 0, hist_batch = 0;
  double* tvals = nullptr;  // [batch][nnz] values of A^T (adjoint)
  int64_t tvals_batch = 0;
};

void release_bs_work(sla_csr A) {
  BsWork* w = A->bs;
  if (!w) return;
  dev_free(w->vec);
  dev_free(w->part);
  dev_free(w->scal);
  dev_free(w->hist);
  dev_free(w->tvals);
  if (w->scal_host) (void)hipHostFree(w->scal_host);
  for (auto& e : w->poll_ev)
    if (e) (void)hipEventDestroy(e);
  if (w->exec) (void)hipGraphExecDestroy(w->exec);
  if (w->graph) (void)hipGraphDestroy(w->graph);
  if (w->capture_stream) (void)hipStreamDestroy(w->capture_stream);
  delete w;
  A->bs = nullptr;
}

// Workgroups per system of the vector kernels: the SpMV's, so that the
// partial sums the SpMV leaves line up with the vector kernels' own.
static int64_t bs_groups(sla_csr P, int64_t batch) { return spmv_groups(P, batch); }

static sla_status ensure_bs_work(sla_csr A, int64_t batch) {
  const int64_t n = A->n, G = bs_groups(A, 1);
  BsWork* w = A->bs;
  if (w && w->cap_n == n && w->cap_batch >= batch && w->cap_g >= G) return SLA_OK;
  release_bs_work(A);
  w = new BsWork();
  A->bs = w;
  w->cap_n = n;
  w->cap_batch = batch;
  w->cap_g = G;
  SLA_TRY(dev_alloc(&w->vec, size_t(6) * size_t(batch) * size_t(n), "BiCGStab vectors"));
  SLA_TRY(dev_alloc(&w->part, size_t(batch) * kBsSets * size_t(G), "BiCGStab partials"));
  SLA_TRY(dev_alloc(&w->scal, size_t(batch), "BiCGStab scalars"));
  SLA_TRY_HIP(hipHostMalloc((void**)&w->scal_host, sizeof(BsScal) * 3 * size_t(batch),
                            hipHostMallocDefault));
  for (auto& e : w->poll_ev) SLA_TRY_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  return SLA_OK;
}

// One iteration: three vector kernels around the two SpMVs, which leave the
// rhat.v and the t.s, t.t partials (their grid is the vector kernels').
static sla_status bs_enqueue_iteration(const BsArgs& a, sla_csr P, const double* vals,
                                       int64_t batch, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.G), static_cast<unsigned>(batch));
  const int64_t ps = kBsSets * a.G;
  k_bs_direction<<<grid, kBsBlock, 0, st>>>(a);
  SLA_TRY(launch_spmv_dots(P, vals, batch, a.p, a.v, a.rh, 1, a.part, ps, P_RV, 0, st));
  k_bs_s<<<grid, kBsBlock, 0, st>>>(a);
  SLA_TRY(launch_spmv_dots(P, vals, batch, a.s, a.t, a.s, 2, a.part, ps, P_TS, P_TT, st));
  k_bs_update<<<grid, kBsBlock, 0, st>>>(a);
  LAUNCH_CHECK();
  return SLA_OK;
}

// The graph of kBsGraphIters iterations for these arguments: reused while
// the pointers it bakes in are unchanged, else captured anew.
static sla_status bs_graph(BsWork* w, const BsArgs& a, sla_csr P, const double* vals,
                           int64_t batch, hipGraphExec_t* exec) {
  if (w->exec && w->key_pattern == P && w->key_vals == vals && w->key_x == a.x &&
      w->key_hist == a.hist && w->key_batch == batch && w->key_g == a.G &&
      w->key_hcap == a.hist_cap) {
    *exec = w->exec;
    return SLA_OK;
  }
  if (w->exec) (void)hipGraphExecDestroy(w->exec);
  if (w->graph) (void)hipGraphDestroy(w->graph);
  w->exec = nullptr;
  w->graph = nullptr;
  if (w->capture_stream == nullptr)
    SLA_TRY_HIP(hipStreamCreateWithFlags(&w->capture_stream, hipStreamNonBlocking));
  hipGraph_t g = nullptr;
  SLA_TRY_HIP(hipStreamBeginCapture(w->capture_stream, hipStreamCaptureModeThreadLocal));
  sla_status s = SLA_OK;
  for (int64_t k = 0; k < kBsGraphIters && s == SLA_OK; ++k)
    s = bs_enqueue_iteration(a, P, vals, batch, w->capture_stream);
  hipError_t he = hipStreamEndCapture(w->capture_stream, &g);
  if (s != SLA_OK) {
    if (g) (void)hipGraphDestroy(g);
    return s;
  }
  if (he != hipSuccess) {
    set_error("BiCGStab graph capture failed: %s", hipGetErrorString(he));
    return SLA_ERR_DEVICE;
  }
  hipGraphExec_t e = nullptr;
  he = hipGraphInstantiate(&e, g, nullptr, nullptr, 0);
  if (he != hipSuccess) {
    (void)hipGraphDestroy(g);
    set_error("BiCGStab graph instantiation failed: %s", hipGetErrorString(he));
    return SLA_ERR_DEVICE;
  }
  w->graph = g;
  w->exec = e;
  w->key_pattern = P;
  w->key_vals = vals;
  w->key_x = a.x;
  w->key_hist = a.hist;
  w->key_batch = batch;
  w->key_g = a.G;
  w->key_hcap = a.hist_cap;
  *exec = e;
  return SLA_OK;
}

// The engine: BiCGStab on the pattern P with values `vals` [batch][P->nnz],
// workspace and scalars from A's BiCGStab work area.
static sla_status bs_run(sla_csr A, sla_csr P, const double* vals, int64_t batch,
                         const double* b, double* x, double tol, int64_t maxit, uint32_t flags,
                         sla_cg_info* info, hipStream_t st) {
  SLA_TRY(ensure_bs_work(A, batch));
  BsWork* w = A->bs;
  const int64_t n = A->n;
  const int64_t G = bs_groups(P, batch);
  const bool want_hist = (flags & SLA_FLAG_HISTORY) != 0;
  if (want_hist) {
    const int64_t cap = maxit > 0 ? maxit : 1;
    if (w->hist == nullptr || w->hist_cap < cap || w->hist_batch < batch) {
      dev_free(w->hist);
      w->hist = nullptr;
      SLA_TRY(dev_alloc(&w->hist, size_t(batch) * size_t(cap) * 4, "BiCGStab history"));
      w->hist_cap = cap;
      w->hist_batch = batch;
    }
  }
  A->bs_hist_valid = want_hist;
  const size_t bn = size_t(batch) * size_t(n);
  BsArgs a{};
  a.n = n;
  a.G = G;
  a.b = b;
  a.x = x;
  a.r = w->vec;
  a.rh = a.r + bn;
  a.p = a.rh + bn;
  a.v = a.p + bn;
  a.s = a.v + bn;
  a.t = a.s + bn;
  a.part = w->part;
  a.scal = w->scal;
  a.hist = want_hist ? w->hist : nullptr;
  a.hist_cap = want_hist ? w->hist_cap : 0;
  const dim3 grid(static_cast<unsigned>(G), static_cast<unsigned>(batch));
  const bool x0 = (flags & SLA_FLAG_X0) != 0;
  if (x0) SLA_TRY(launch_spmv(P, vals, batch, x, a.v, st));  // v = A x0, read by k_bs_init
  k_bs_init<<<grid, kBsBlock, 0, st>>>(a, a.v, x0 ? 1 : 0);
  k_bs_init_scalars<<<unsigned(batch), kBsBlock, 0, st>>>(a, tol, maxit);
  LAUNCH_CHECK();
  if (maxit < 2 * kBsGraphIters) {
    // short runs: every iteration launched directly (kernels of a stopped
    // system return at once)
    for (int64_t j = 0; j < maxit; ++j) SLA_TRY(bs_enqueue_iteration(a, P, vals, batch, st));
  } else {
    // blocks of kBsGraphIters iterations replayed from one captured graph;
    // after each block the scalars are copied to pinned memory, and before
    // block k is launched the host waits for the copy behind block k - 2,
    // so one block is always queued while the host can still stop early
    hipGraphExec_t exec = nullptr;
    SLA_TRY(bs_graph(w, a, P, vals, batch, &exec));
    const int64_t blocks = (maxit + kBsGraphIters - 1) / kBsGraphIters;
    for (int64_t k = 0; k < blocks; ++k) {
      if (k >= 2) {
        const int q = int(k & 1);
        SLA_TRY_HIP(hipEventSynchronize(w->poll_ev[q]));
        const BsScal* h = w->scal_host + (1 + q) * batch;
        int64_t running = 0;
        for (int64_t s = 0; s < batch; ++s) running += h[s].stop_pos == kNoStop;
        if (running == 0) break;
      }
      SLA_TRY_HIP(hipGraphLaunch(exec, st));
      const int q = int(k & 1);
      SLA_TRY_HIP(hipMemcpyAsync(w->scal_host + (1 + q) * batch, w->scal,
                                 sizeof(BsScal) * size_t(batch), hipMemcpyDeviceToHost, st));
      SLA_TRY_HIP(hipEventRecord(w->poll_ev[q], st));
    }
  }
  // close: the stopping tests of the state after the last iteration
  k_bs_direction<<<grid, kBsBlock, 0, st>>>(a);
  LAUNCH_CHECK();
  SLA_TRY_HIP(hipMemcpyAsync(w->scal_host, w->scal, sizeof(BsScal) * size_t(batch),
                             hipMemcpyDeviceToHost, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));
  sla_status first = SLA_OK;
  for (int64_t s = 0; s < batch; ++s) {
    const BsScal& sc = w->scal_host[s];
    sla_cg_info in{};
    in.iterations = sc.it;
    in.rel_residual = sc.bb > 0.0 ? std::sqrt(sc.rr / sc.bb) : 0.0;
    in.converged = (sc.status == ST_CONVERGED) ? 1 : 0;
    in.status = (sc.status == ST_CONVERGED || sc.status == ST_MAXIT) ? SLA_OK : sc.status;
    if (info) info[s] = in;
    if (first == SLA_OK && in.status != SLA_OK) first = sla_status(in.status);
  }
  if (first != SLA_OK)
    set_error("BiCGStab: %s", first == SLA_ERR_BREAKDOWN ? "breakdown (rhat.r, rhat.v or t.t is 0)"
                                                         : "non-finite value");
  return first;
}

sla_status run_bicgstab(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                        uint32_t flags, sla_cg_info* info, hipStream_t st) {
  return bs_run(A, A, A->vals, A->batch, b, x, tol, maxit, flags, info, st);
}

sla_status run_bicgstab_adjoint(sla_csr A, const double* x, const double* grad_x,
                                double* grad_b, double* grad_vals, double tol, int64_t maxit,
                                uint32_t flags, sla_cg_info* info, hipStream_t st) {
  SLA_TRY(build_transpose(A, st));
  sla_csr T = A->trans;
  const int64_t batch = A->batch;
  SLA_TRY(ensure_bs_work(A, batch));
  BsWork* w = A->bs;
  if (w->tvals == nullptr || w->tvals_batch < batch) {
    dev_free(w->tvals);
    w->tvals = nullptr;
    SLA_TRY(dev_alloc(&w->tvals, size_t(batch) * size_t(A->nnz > 0 ? A->nnz : 1),
                      "transposed values"));
    w->tvals_batch = batch;
  }
  // A^T's values in its slot order, once per adjoint solve
  if (A->nnz > 0) SLA_TRY(launch_values_from_coo(T, A->vals, w->tvals, batch, st));
  const sla_status s = bs_run(A, T, w->tvals, batch, grad_x, grad_b, tol, maxit,
                              flags & ~uint32_t(SLA_FLAG_X0), info, st);
  if (s != SLA_OK && s != SLA_ERR_BREAKDOWN && s != SLA_ERR_NONFINITE) return s;
  if (grad_vals != nullptr && A->nnz > 0)
    SLA_TRY(launch_slot_products(A, batch, grad_b, x, grad_vals, true, st));
  return s;
}

sla_status bicgstab_history(sla_csr A, int64_t system, double* rho, double* alpha,
                            double* omega, double* rr, int64_t cap, int64_t* count) {
  BsWork* w = A->bs;
  if (w == nullptr || !A->bs_hist_valid || w->hist == nullptr) {
    set_error("sla_bicgstab_history: the last BiCGStab solve kept no history");
    return SLA_ERR_ARG;
  }
  if (system < 0 || system >= w->hist_batch) {
    set_error("sla_bicgstab_history: system %lld out of range", (long long)system);
    return SLA_ERR_ARG;
  }
  const int64_t k = w->scal_host[system].it < w->hist_cap ? w->scal_host[system].it : w->hist_cap;
  if (count) *count = k;
  const int64_t m = k < cap ? k : cap;
  if (m <= 0) return SLA_OK;
  std::vector<double> h(size_t(m) * 4);
  SLA_TRY_HIP(hipMemcpy(h.data(), w->hist + system * w->hist_cap * 4,
                        sizeof(double) * size_t(m) * 4, hipMemcpyDeviceToHost));
  for (int64_t i = 0; i < m; ++i) {
    if (rho) rho[i] = h[i * 4 + 0];
    if (alpha) alpha[i] = h[i * 4 + 1];
    if (omega) omega[i] = h[i * 4 + 2];
    if (rr) rr[i] = h[i * 4 + 3];
  }
  return SLA_OK;
}

}  // namespace sla
