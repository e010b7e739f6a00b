// The .eigsh of the torch-sla summary (Methodology 1): a few extreme
// eigenpairs of a sparse symmetric matrix by the Lanczos process, and their
// gradient by the Hellmann-Feynman relation d lambda / d A_ij = v_i v_j on the
// stored slots (Methodology 2, eigenvalue problems).
//
// A step j of the process, on one system:
//   w = A v_j                                   (the library's SpMV)
//   h  = V_j^T w  (+ w.w)   ; w -= V_j h        (Gram-Schmidt, first pass)
//   h' = V_j^T w            ; w -= V_j h'       (second pass, + w.w partials)
//   alpha_j = h_j + h'_j, beta_j = |w|, stop when beta_j <= 1e-10 |A v_j|
//   v_{j+1} = w / beta_j
// Every pass over the basis V reads it once from HBM; the dot passes keep
// their rows of w in registers and emit one partial per workgroup and basis
// vector, summed in a fixed order by a second kernel, so the results do not
// depend on timing.  A stop flag in device memory makes the kernels of later
// steps return at once; the host looks at it every few steps without waiting
// and stops launching.
//
// The tridiagonal eigenproblem T y = theta y is solved on the device by one
// wave: Sturm-count bisection for the wanted eigenvalues, then inverse
// iteration with a pivoted tridiagonal LU for their vectors, orthogonalised
// inside clusters of close eigenvalues.  Ritz vectors are X = V Y.
#include <cfloat>
#include <cmath>

#include "handle.h"

namespace sla {

constexpr int kLzBlock = 256;   // workgroup of the Lanczos kernels (4 waves)
constexpr int kLzDotVecs = 8;   // basis vectors per workgroup of the dot pass
constexpr int64_t kLzChunk = 2048;  // rows per workgroup of the dot pass
constexpr int kLzDotRows = 4;   // rows per thread and loop trip of the dot pass
constexpr int kLzRitz = 8;      // Ritz vectors accumulated per pass over V
constexpr int kInvIters = 3;    // inverse-iteration solves per eigenvector
constexpr int64_t kTriLdsMax = 960;  // largest m whose tridiagonal work fits in LDS
constexpr double kBreakdown = 1e-10;

struct alignas(64) LzState {
  double norm0;    // |v0|
  int64_t steps;   // completed Lanczos steps
  int32_t stop;    // no further step: breakdown, m steps done, or an error
  int32_t status;  // SLA_OK or the error of this system
};

struct EigWork {
  int64_t cap_n = 0, cap_m = 0, cap_k = 0, cap_g = 0;
  double* V = nullptr;      // [m+1][n] Lanczos basis
  double* w = nullptr;      // [n]
  double* part = nullptr;   // [m+2][G] dot partials, basis-vector major
  double* pww = nullptr;    // [G] w.w partials after the second pass
  double* h1 = nullptr;     // [m+2] first-pass coefficients, then w.w
  double* h2 = nullptr;     // [m+2]
  double* alpha = nullptr;  // [m]
  double* beta = nullptr;   // [m]
  double* Y = nullptr;      // [k][m] eigenvectors of T
  double* tri = nullptr;    // [6][m] inverse-iteration scratch
  LzState* st = nullptr;
  LzState* st_host = nullptr;  // pinned
  int32_t* poll_host = nullptr;  // pinned
  hipEvent_t poll_ev = nullptr;
};

// ---------------------------------------------------------------------------
// Gram-Schmidt passes
// ---------------------------------------------------------------------------

// part[l][g] = sum over the rows of chunk g of src_l[i] w[i], where src_l is
// basis vector l for l < nvec and w itself for l == nvec (when with_ww).
// A workgroup takes one chunk of kLzChunk rows and a block of kLzDotVecs
// vectors and reduces its sums once, at the end.  Workgroups are numbered so
// that those sharing a chunk run on one XCD one after another (workgroup i
// runs on XCD i % 8): the chunk of w they all read then comes from that
// XCD's L2 after the first.
__global__ __launch_bounds__(kLzBlock) void k_lz_dot(const double* __restrict__ V, int64_t n,
                                                     int64_t nvec, const double* __restrict__ w,
                                                     int with_ww, double* __restrict__ part,
                                                     int64_t G, int64_t nblk,
                                                     const LzState* __restrict__ st) {
  if (st->stop) return;
  __shared__ double red[kLzBlock / kWave][kLzDotVecs];
  const int64_t xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int64_t g = (slot / nblk) * kXcds + xcd;
  const int64_t l0 = (slot % nblk) * kLzDotVecs;
  if (g >= G) return;
  const int64_t total = nvec + (with_ww ? 1 : 0);
  double acc[kLzDotVecs];
#pragma unroll
  for (int q = 0; q < kLzDotVecs; ++q) acc[q] = 0.0;
  const int64_t r1 = (g + 1) * kLzChunk < n ? (g + 1) * kLzChunk : n;
  for (int64_t i0 = g * kLzChunk + threadIdx.x; i0 < r1; i0 += kLzBlock * kLzDotRows) {
    double wi[kLzDotRows];
#pragma unroll
    for (int r = 0; r < kLzDotRows; ++r) {
      const int64_t i = i0 + r * kLzBlock;
      wi[r] = i < r1 ? w[i] : 0.0;
    }
#pragma unroll
    for (int q = 0; q < kLzDotVecs; ++q) {
      const int64_t l = l0 + q;
      if (l < total) {
        const double* src = l < nvec ? V + l * n : w;
#pragma unroll
        for (int r = 0; r < kLzDotRows; ++r) {
          const int64_t i = i0 + r * kLzBlock;
          if (i < r1) acc[q] = fma(src[i], wi[r], acc[q]);
        }
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kLzDotVecs; ++q) acc[q] = wave_sum(acc[q]);
  const int wave = wave_index();
  if (lane_id() == 0) {
#pragma unroll
    for (int q = 0; q < kLzDotVecs; ++q) red[wave][q] = acc[q];
  }
  __syncthreads();
  if (threadIdx.x < kLzDotVecs && l0 + threadIdx.x < total) {
    double s = 0.0;
#pragma unroll
    for (int v = 0; v < kLzBlock / kWave; ++v) s = s + red[v][threadIdx.x];
    part[(l0 + threadIdx.x) * G + g] = s;
  }
}

// out[l] = sum_g part[l][g] for l < count (one workgroup per l, fixed order).
__global__ __launch_bounds__(kLzBlock) void k_lz_reduce(const double* __restrict__ part,
                                                        int64_t G, double* __restrict__ out,
                                                        const LzState* __restrict__ st) {
  if (st->stop) return;
  __shared__ double lds[kLzBlock / kWave];
  const double* p = part + int64_t(blockIdx.x) * G;
  double s = 0.0;
  for (int64_t g = threadIdx.x; g < G; g += kLzBlock) s = s + p[g];
  s = block_sum_all<kLzBlock>(s, lds);
  if (threadIdx.x == 0) out[blockIdx.x] = s;
}

// w -= V_nvec h over this workgroup's rows (basis vectors in index order);
// with pww, also the workgroup's partial of w.w after the update.
template <int R>
__global__ __launch_bounds__(kLzBlock) void k_lz_update(const double* __restrict__ V, int64_t n,
                                                        int64_t nvec,
                                                        const double* __restrict__ h,
                                                        double* __restrict__ w,
                                                        double* __restrict__ pww,
                                                        const LzState* __restrict__ st) {
  if (st->stop) return;
  __shared__ double lds[kLzBlock / kWave];
  const int64_t base = int64_t(blockIdx.x) * (kLzBlock * R) + threadIdx.x;
  double wv[R];
  bool in[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = base + int64_t(r) * kLzBlock;
    in[r] = i < n;
    wv[r] = in[r] ? w[i] : 0.0;
  }
  int64_t l = 0;
  for (; l + 4 <= nvec; l += 4) {
    const double h0 = h[l], h1 = h[l + 1], h2 = h[l + 2], h3 = h[l + 3];
    const double* v0 = V + l * n;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!in[r]) continue;
      const int64_t i = base + int64_t(r) * kLzBlock;
      const double a0 = v0[i], a1 = v0[n + i], a2 = v0[2 * n + i], a3 = v0[3 * n + i];
      wv[r] = fma(-a0, h0, wv[r]);
      wv[r] = fma(-a1, h1, wv[r]);
      wv[r] = fma(-a2, h2, wv[r]);
      wv[r] = fma(-a3, h3, wv[r]);
    }
  }
  for (; l < nvec; ++l) {
    const double hl = h[l];
    const double* v = V + l * n;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t i = base + int64_t(r) * kLzBlock;
      if (in[r]) wv[r] = fma(-v[i], hl, wv[r]);
    }
  }
  double ss = 0.0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = base + int64_t(r) * kLzBlock;
    if (in[r]) w[i] = wv[r];
    ss = fma(wv[r], wv[r], ss);
  }
  if (pww != nullptr) {
    ss = block_sum_all<kLzBlock>(ss, lds);
    if (threadIdx.x == 0) pww[blockIdx.x] = ss;
  }
}

// |v0| and the start of a system's process.
__global__ __launch_bounds__(kLzBlock) void k_lz_begin(const double* __restrict__ part, int64_t G,
                                                       LzState* __restrict__ st) {
  __shared__ double lds[kLzBlock / kWave];
  double s = 0.0;
  for (int64_t g = threadIdx.x; g < G; g += kLzBlock) s = s + part[g];
  s = block_sum_all<kLzBlock>(s, lds);
  if (threadIdx.x == 0) {
    const double nv = sqrt(s);
    st->norm0 = nv;
    st->steps = 0;
    if (!(nv > 0.0) || !isfinite(nv)) {
      st->stop = 1;
      st->status = isfinite(nv) ? SLA_ERR_ARG : SLA_ERR_NONFINITE;
    }
  }
}

__global__ void k_lz_reset(LzState* st) {
  st->norm0 = 0.0;
  st->steps = 0;
  st->stop = 0;
  st->status = SLA_OK;
}

// alpha_j, beta_j and the stopping test of step j.  h1[j + 1] holds w.w
// before the Gram-Schmidt passes.
__global__ __launch_bounds__(kLzBlock) void k_lz_finish(const double* __restrict__ pww,
                                                        int64_t G, const double* __restrict__ h1,
                                                        const double* __restrict__ h2, int64_t j,
                                                        int64_t m, double* __restrict__ alpha,
                                                        double* __restrict__ beta,
                                                        LzState* __restrict__ st) {
  if (st->stop) return;
  __shared__ double lds[kLzBlock / kWave];
  double s = 0.0;
  for (int64_t g = threadIdx.x; g < G; g += kLzBlock) s = s + pww[g];
  s = block_sum_all<kLzBlock>(s, lds);
  if (threadIdx.x == 0) {
    const double a = h1[j] + h2[j];
    const double b = sqrt(s);
    const double wn = sqrt(h1[j + 1]);
    alpha[j] = a;
    beta[j] = b;
    st->steps = j + 1;
    if (!isfinite(a) || !isfinite(b)) {
      st->status = SLA_ERR_NONFINITE;
      st->stop = 1;
    } else if (!(b > kBreakdown * wn) || j + 1 == m) {
      st->stop = 1;
    }
  }
}

// dst = src / *d (a correctly rounded division per element).
__global__ __launch_bounds__(kLzBlock) void k_lz_scale(const double* __restrict__ src,
                                                       double* __restrict__ dst, int64_t n,
                                                       const double* __restrict__ d,
                                                       const LzState* __restrict__ st) {
  if (st->stop) return;
  const double dv = *d;
  for (int64_t i = int64_t(blockIdx.x) * kLzBlock + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * kLzBlock)
    dst[i] = src[i] / dv;
}

// ---------------------------------------------------------------------------
// The tridiagonal eigenproblem
// ---------------------------------------------------------------------------

// Number of eigenvalues of T (diagonal a, off-diagonal b, size m) below x, by
// the signs of the pivots of T - x I (Sturm sequence); pivots of magnitude
// at most pivmin are replaced by -pivmin.
__device__ int64_t sturm_count(const double* a, const double* b, int64_t m, double x,
                               double pivmin) {
  double q = a[0] - x;
  if (fabs(q) <= pivmin) q = -pivmin;
  int64_t c = q < 0.0 ? 1 : 0;
  for (int64_t i = 1; i < m; ++i) {
    q = (a[i] - x) - (b[i - 1] * b[i - 1]) / q;
    if (fabs(q) <= pivmin) q = -pivmin;
    c += q < 0.0 ? 1 : 0;
  }
  return c;
}

// Solve (T - x I) y = y in place by LU with partial pivoting; pivots smaller
// than `tiny` in magnitude are replaced by +-tiny (the solve then amplifies
// the eigenvector direction, which is what inverse iteration needs).
// scratch: d, du, du2, dl [m] each, and a pivot flag array.
__device__ void tri_shifted_solve(const double* a, const double* b, int64_t m, double x,
                                  double tiny, double* d, double* du, double* du2, double* dl,
                                  double* piv, double* y) {
  for (int64_t i = 0; i < m; ++i) {
    d[i] = a[i] - x;
    if (i + 1 < m) {
      du[i] = b[i];
      dl[i] = b[i];
    }
    du2[i] = 0.0;
  }
  for (int64_t i = 0; i + 1 < m; ++i) {
    if (fabs(d[i]) >= fabs(dl[i])) {
      // no interchange: eliminate the sub-diagonal entry of row i+1
      if (fabs(d[i]) <= tiny) d[i] = d[i] < 0.0 ? -tiny : tiny;
      const double f = dl[i] / d[i];
      dl[i] = f;
      d[i + 1] = d[i + 1] - f * du[i];
      piv[i] = 0.0;
    } else {
      // rows i and i+1 swap; row i+1 (now the pivot row) gains a fill-in two
      // columns to the right of the diagonal
      const double f = d[i] / dl[i];
      d[i] = dl[i];
      dl[i] = f;
      const double t = du[i];
      du[i] = d[i + 1];
      d[i + 1] = t - f * d[i + 1];
      if (i + 2 < m) {
        du2[i] = du[i + 1];
        du[i + 1] = -f * du[i + 1];
      }
      piv[i] = 1.0;
    }
  }
  if (fabs(d[m - 1]) <= tiny) d[m - 1] = d[m - 1] < 0.0 ? -tiny : tiny;
  // L solve
  for (int64_t i = 0; i + 1 < m; ++i) {
    if (piv[i] == 0.0) {
      y[i + 1] = y[i + 1] - dl[i] * y[i];
    } else {
      const double t = y[i];
      y[i] = y[i + 1];
      y[i + 1] = t - dl[i] * y[i + 1];
    }
  }
  // U solve (upper triangular with two super-diagonals)
  y[m - 1] = y[m - 1] / d[m - 1];
  if (m >= 2) y[m - 2] = (y[m - 2] - du[m - 2] * y[m - 1]) / d[m - 2];
  for (int64_t i = m - 3; i >= 0; --i)
    y[i] = (y[i] - du[i] * y[i + 1] - du2[i] * y[i + 2]) / d[i];
}

// One wave: the k wanted eigenpairs of the steps x steps tridiagonal T
// (which = SLA_EIG_LARGEST: the k largest, else the k smallest), ascending;
// Y[t][0 .. steps) their unit eigenvectors (largest component positive),
// resid[t] = |beta_{steps-1} Y[t][steps-1]|, the residual norm of the Ritz pair.
// With use_lds, T and the inverse-iteration arrays live in LDS (8 ldy
// doubles of dynamic LDS): the LU recurrences then wait on LDS, not on
// global memory, at every step.
__global__ __launch_bounds__(kWave) void k_tri_eig(const double* __restrict__ alpha_g,
                                                   const double* __restrict__ beta_g, int64_t k,
                                                   int which, double* __restrict__ theta,
                                                   double* __restrict__ Y, int64_t ldy,
                                                   double* __restrict__ resid,
                                                   double* __restrict__ scratch_g, int use_lds,
                                                   LzState* __restrict__ st) {
  __shared__ double bounds[4];
  extern __shared__ double tri_lds[];
  if (st->status != SLA_OK) return;
  const int64_t m = st->steps;
  if (m < k) {
    if (threadIdx.x == 0) st->status = SLA_ERR_KRYLOV;
    return;
  }
  const double* alpha = alpha_g;
  const double* beta = beta_g;
  double* scratch = scratch_g;
  if (use_lds) {
    double* a_s = tri_lds;
    double* b_s = tri_lds + ldy;
    for (int64_t i = threadIdx.x; i < m; i += kWave) {
      a_s[i] = alpha_g[i];
      b_s[i] = beta_g[i];
    }
    __syncthreads();
    alpha = a_s;
    beta = b_s;
    scratch = tri_lds + 2 * ldy;
  }
  if (threadIdx.x == 0) {
    double lo = INFINITY, hi = -INFINITY, nrm = 0.0, bmax = 0.0;
    for (int64_t i = 0; i < m; ++i) {
      const double off = (i > 0 ? fabs(beta[i - 1]) : 0.0) + (i + 1 < m ? fabs(beta[i]) : 0.0);
      lo = fmin(lo, alpha[i] - off);
      hi = fmax(hi, alpha[i] + off);
      nrm = fmax(nrm, fabs(alpha[i]) + off);
      if (i + 1 < m) bmax = fmax(bmax, beta[i] * beta[i]);
    }
    const double pad = 2.0 * DBL_EPSILON * nrm * double(m) + DBL_MIN;
    bounds[0] = lo - pad;
    bounds[1] = hi + pad;
    bounds[2] = nrm;
    bounds[3] = DBL_MIN * fmax(1.0, bmax);
  }
  __syncthreads();
  const double nrm = bounds[2], pivmin = bounds[3];
  // bisection: eigenvalue number idx (0-based, ascending) lies in (lo, hi]
  for (int64_t t = threadIdx.x; t < k; t += kWave) {
    const int64_t idx = which == SLA_EIG_LARGEST ? m - k + t : t;
    double lo = bounds[0], hi = bounds[1];
    for (int it = 0; it < 4096; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (!(mid > lo && mid < hi)) break;
      if (hi - lo <= 2.0 * DBL_EPSILON * fmax(fabs(lo), fabs(hi)) + DBL_EPSILON * nrm) break;
      if (sturm_count(alpha, beta, m, mid, pivmin) > idx) hi = mid;
      else lo = mid;
    }
    theta[t] = 0.5 * (lo + hi);
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  // inverse iteration, eigenvalues in ascending order; eigenvalues closer
  // than 1e-3 |T| to their predecessor form a cluster whose vectors are kept
  // orthogonal to each other
  double* d = scratch;
  double* du = d + ldy;
  double* du2 = du + ldy;
  double* dl = du2 + ldy;
  double* piv = dl + ldy;
  double* y = piv + ldy;
  const double ortol = 1e-3 * nrm;
  const double tiny = DBL_EPSILON * nrm > DBL_MIN ? DBL_EPSILON * nrm : DBL_MIN;
  int64_t first = 0;  // first eigenvector of the current cluster
  double xprev = 0.0;
  for (int64_t t = 0; t < k; ++t) {
    double x = theta[t];
    if (t > 0) {
      if (x - theta[t - 1] > ortol) first = t;
      // equal shifts would give equal vectors: move the shift a little
      const double pert = 10.0 * DBL_EPSILON * fabs(x) + tiny;
      if (x - xprev < pert) x = xprev + pert;
    }
    xprev = x;
    // a fixed start vector with no special structure
    uint64_t seed = 0x9E3779B97F4A7C15ull * uint64_t(t + 1);
    for (int64_t i = 0; i < m; ++i) {
      seed = seed * 6364136223846793005ull + 1442695040888963407ull;
      y[i] = double(int64_t(seed >> 11) - (int64_t(1) << 52)) * (1.0 / 4503599627370496.0);
    }
    for (int it = 0; it < kInvIters; ++it) {
      tri_shifted_solve(alpha, beta, m, x, tiny, d, du, du2, dl, piv, y);
      for (int64_t u = first; u < t; ++u) {
        const double* yu = Y + u * ldy;
        double c = 0.0;
        for (int64_t i = 0; i < m; ++i) c = fma(yu[i], y[i], c);
        for (int64_t i = 0; i < m; ++i) y[i] = fma(-c, yu[i], y[i]);
      }
      double s = 0.0;
      for (int64_t i = 0; i < m; ++i) s = fma(y[i], y[i], s);
      const double inv = 1.0 / sqrt(s);
      for (int64_t i = 0; i < m; ++i) y[i] = y[i] * inv;
    }
    int64_t imax = 0;
    for (int64_t i = 1; i < m; ++i)
      if (fabs(y[i]) > fabs(y[imax])) imax = i;
    const double sg = y[imax] < 0.0 ? -1.0 : 1.0;
    double* yt = Y + t * ldy;
    for (int64_t i = 0; i < m; ++i) yt[i] = sg * y[i];
    resid[t] = fabs(beta[m - 1] * yt[m - 1]);
  }
}

// X[t][i] = sum_{j < steps} V[j][i] Y[t][j] for t in [t0, t0 + KB).
template <int KB>
__global__ __launch_bounds__(kLzBlock) void k_lz_ritz(const double* __restrict__ V, int64_t n,
                                                      const double* __restrict__ Y, int64_t ldy,
                                                      int64_t t0, int64_t k,
                                                      double* __restrict__ X,
                                                      const LzState* __restrict__ st) {
  if (st->status != SLA_OK) return;
  const int64_t m = st->steps;
  const int64_t i = int64_t(blockIdx.x) * kLzBlock + threadIdx.x;
  if (i >= n) return;
  double acc[KB];
#pragma unroll
  for (int q = 0; q < KB; ++q) acc[q] = 0.0;
  for (int64_t j = 0; j < m; ++j) {
    const double v = V[j * n + i];
#pragma unroll
    for (int q = 0; q < KB; ++q)
      if (t0 + q < k) acc[q] = fma(v, Y[(t0 + q) * ldy + j], acc[q]);
  }
#pragma unroll
  for (int q = 0; q < KB; ++q)
    if (t0 + q < k) X[(t0 + q) * n + i] = acc[q];
}

// grad[s][slot (i, j)] = sum_t g[s][t] X[s][t][i] X[s][t][j] on every stored
// slot: the Hellmann-Feynman gradient of sum_t g_t theta_t.  One wave per
// 64-row tile; its lanes take consecutive slots (coalesced column reads and
// gradient writes), each slot's row read from a map of the tile's slots to
// their rows, built in LDS `cap` slots at a time.
template <typename RP>
__global__ __launch_bounds__(kIterBlock) void k_eig_grad(const RP* __restrict__ rowptr,
                                                         const int32_t* __restrict__ col,
                                                         int64_t n, int64_t nnz, int64_t tiles,
                                                         int cap, int64_t k,
                                                         const double* __restrict__ X,
                                                         const double* __restrict__ g,
                                                         double* __restrict__ grad) {
  extern __shared__ uint8_t slot_rows[];
  const int wv = wave_index();
  const int lane = int(lane_id());
  uint8_t* rowmap = slot_rows + int64_t(wv) * cap;
  const int64_t s = blockIdx.y;
  const double* Xs = X + s * k * n;
  const double* gs = g + s * k;
  double* out = grad + s * nnz;
  // contiguous tile ranges per XCD: the tiles that gather the same entries
  // of X run close together on one L2
  const TileWalk walk = wave_walk(tiles, int(gridDim.x), int(blockIdx.x), kWaves, wv);
  for (int64_t t = walk.first; t < walk.end; t += walk.stride) {
    const int64_t r0 = t * kTileRows;
    const int64_t r1 = r0 + kTileRows < n ? r0 + kTileRows : n;
    const int64_t s0 = rowptr[r0];
    const int64_t len = int64_t(rowptr[r1]) - s0;
    const int64_t i = r0 + lane;
    int64_t a = 0, e = 0;
    if (i < r1) {
      a = int64_t(rowptr[i]) - s0;
      e = int64_t(rowptr[i + 1]) - s0;
    }
    for (int64_t c0 = 0; c0 < len; c0 += cap) {
      const int64_t clen = len - c0 < cap ? len - c0 : cap;
      const int64_t qa = a > c0 ? a : c0, qe = e < c0 + clen ? e : c0 + clen;
      for (int64_t q = qa; q < qe; ++q) rowmap[q - c0] = uint8_t(lane);
      wave_sync();
      for (int64_t q = lane; q < clen; q += kWave) {
        const int64_t row = r0 + rowmap[q];
        const int64_t slot = s0 + c0 + q;
        const int64_t j = col[slot];
        double acc = 0.0;
        for (int64_t u = 0; u < k; ++u) acc = acc + gs[u] * (Xs[u * n + row] * Xs[u * n + j]);
        out[slot] = acc;
      }
      wave_sync();
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// 4 rows per thread once that still leaves about 2 workgroups per CU
static int lz_rows_per_thread(int64_t n) { return n >= (int64_t(1) << 19) ? 4 : 1; }

static int64_t lz_groups(int64_t n) {
  const int64_t rows = int64_t(kLzBlock) * lz_rows_per_thread(n);
  return (n + rows - 1) / rows;
}

static int64_t lz_dot_chunks(int64_t n);

void release_eig_work(sla_csr A) {
  EigWork* e = A->eig;
  if (!e) return;
  dev_free(e->V);
  dev_free(e->w);
  dev_free(e->part);
  dev_free(e->pww);
  dev_free(e->h1);
  dev_free(e->h2);
  dev_free(e->alpha);
  dev_free(e->beta);
  dev_free(e->Y);
  dev_free(e->tri);
  dev_free(e->st);
  if (e->st_host) (void)hipHostFree(e->st_host);
  if (e->poll_host) (void)hipHostFree(e->poll_host);
  if (e->poll_ev) (void)hipEventDestroy(e->poll_ev);
  delete e;
  A->eig = nullptr;
}

static sla_status ensure_eig_work(sla_csr A, int64_t m, int64_t k) {
  const int64_t n = A->n;
  const int64_t G = lz_groups(n) > lz_dot_chunks(n) ? lz_groups(n) : lz_dot_chunks(n);
  EigWork* e = A->eig;
  if (e && e->cap_n == n && e->cap_m >= m && e->cap_k >= k && e->cap_g >= G) return SLA_OK;
  release_eig_work(A);
  e = new EigWork();
  A->eig = e;
  e->cap_n = n;
  e->cap_m = m;
  e->cap_k = k;
  e->cap_g = G;
  SLA_TRY(dev_alloc(&e->V, size_t(m + 1) * size_t(n), "Lanczos basis"));
  SLA_TRY(dev_alloc(&e->w, size_t(n), "Lanczos vector"));
  SLA_TRY(dev_alloc(&e->part, size_t(m + 2) * size_t(G), "Lanczos partials"));
  SLA_TRY(dev_alloc(&e->pww, size_t(G), "Lanczos partials"));
  SLA_TRY(dev_alloc(&e->h1, size_t(m + 2), "Lanczos coefficients"));
  SLA_TRY(dev_alloc(&e->h2, size_t(m + 2), "Lanczos coefficients"));
  SLA_TRY(dev_alloc(&e->alpha, size_t(m), "Lanczos alpha"));
  SLA_TRY(dev_alloc(&e->beta, size_t(m), "Lanczos beta"));
  SLA_TRY(dev_alloc(&e->Y, size_t(k) * size_t(m), "tridiagonal eigenvectors"));
  SLA_TRY(dev_alloc(&e->tri, size_t(6) * size_t(m), "tridiagonal scratch"));
  SLA_TRY(dev_alloc(&e->st, 1, "Lanczos state"));
  SLA_TRY_HIP(hipHostMalloc((void**)&e->st_host, sizeof(LzState), hipHostMallocDefault));
  SLA_TRY_HIP(hipHostMalloc((void**)&e->poll_host, sizeof(int32_t), hipHostMallocDefault));
  SLA_TRY_HIP(hipEventCreateWithFlags(&e->poll_ev, hipEventDisableTiming));
  return SLA_OK;
}

static int64_t lz_dot_chunks(int64_t n) { return (n + kLzChunk - 1) / kLzChunk; }

static void lz_launch_dot(EigWork* e, int64_t n, int64_t nvec, const double* w, int with_ww,
                          hipStream_t st) {
  const int64_t G = lz_dot_chunks(n);
  const int64_t nblk = (nvec + (with_ww ? 1 : 0) + kLzDotVecs - 1) / kLzDotVecs;
  const int64_t groups = (G + kXcds - 1) / kXcds * kXcds * nblk;
  k_lz_dot<<<unsigned(groups), kLzBlock, 0, st>>>(e->V, n, nvec, w, with_ww, e->part, G, nblk,
                                                  e->st);
}

template <int R>
static void lz_launch_update(EigWork* e, int64_t n, int64_t nvec, const double* h, double* pww,
                             int64_t G, hipStream_t st) {
  k_lz_update<R><<<unsigned(G), kLzBlock, 0, st>>>(e->V, n, nvec, h, e->w, pww, e->st);
}

// One system: m Lanczos steps from v0 with the values `vals`, then the k
// wanted Ritz pairs.
template <int R>
static sla_status lanczos_system(sla_csr A, const double* vals, const double* v0, int64_t m,
                                 int64_t k, int which, double* theta, double* X, double* resid,
                                 sla_eig_info* info, hipStream_t st) {
  EigWork* e = A->eig;
  const int64_t n = A->n, G = lz_groups(n);
  const unsigned G2 = unsigned((n + kLzBlock - 1) / kLzBlock);
  const unsigned Gs = G2 < 4096u ? G2 : 4096u;
  k_lz_reset<<<1, 1, 0, st>>>(e->st);
  const int64_t Gd = lz_dot_chunks(n);
  lz_launch_dot(e, n, 0, v0, 1, st);
  k_lz_begin<<<1, kLzBlock, 0, st>>>(e->part, Gd, e->st);
  k_lz_scale<<<Gs, kLzBlock, 0, st>>>(v0, e->V, n, &e->st->norm0, e->st);
  LAUNCH_CHECK();
  constexpr int64_t kPoll = 8;
  bool polled = false;
  for (int64_t j = 0; j < m; ++j) {
    if (polled && hipEventQuery(e->poll_ev) == hipSuccess) {
      polled = false;
      if (*e->poll_host) break;
    }
    SLA_TRY(launch_spmv(A, vals, 1, e->V + j * n, e->w, st));
    lz_launch_dot(e, n, j + 1, e->w, 1, st);
    k_lz_reduce<<<unsigned(j + 2), kLzBlock, 0, st>>>(e->part, Gd, e->h1, e->st);
    lz_launch_update<R>(e, n, j + 1, e->h1, nullptr, G, st);
    lz_launch_dot(e, n, j + 1, e->w, 0, st);
    k_lz_reduce<<<unsigned(j + 1), kLzBlock, 0, st>>>(e->part, Gd, e->h2, e->st);
    lz_launch_update<R>(e, n, j + 1, e->h2, e->pww, G, st);
    k_lz_finish<<<1, kLzBlock, 0, st>>>(e->pww, G, e->h1, e->h2, j, m, e->alpha, e->beta,
                                         e->st);
    k_lz_scale<<<Gs, kLzBlock, 0, st>>>(e->w, e->V + (j + 1) * n, n, e->beta + j, e->st);
    LAUNCH_CHECK();
    if (!polled && (j + 1) % kPoll == 0) {
      SLA_TRY_HIP(hipMemcpyAsync(e->poll_host, &e->st->stop, sizeof(int32_t),
                                 hipMemcpyDeviceToHost, st));
      SLA_TRY_HIP(hipEventRecord(e->poll_ev, st));
      polled = true;
    }
  }
  const int tri_lds = m <= kTriLdsMax ? 1 : 0;
  k_tri_eig<<<1, kWave, tri_lds ? size_t(8) * size_t(m) * sizeof(double) : 0, st>>>(
      e->alpha, e->beta, k, which, theta, e->Y, m, resid, e->tri, tri_lds, e->st);
  for (int64_t t0 = 0; t0 < k; t0 += kLzRitz)
    k_lz_ritz<kLzRitz><<<G2, kLzBlock, 0, st>>>(e->V, n, e->Y, m, t0, k, X, e->st);
  LAUNCH_CHECK();
  SLA_TRY_HIP(hipMemcpyAsync(e->st_host, e->st, sizeof(LzState), hipMemcpyDeviceToHost, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));
  info->steps = e->st_host->steps;
  info->status = e->st_host->status;
  return SLA_OK;
}

sla_status run_eigsh(sla_csr A, int64_t k, int which, int64_t m, const double* v0,
                     double* theta, double* X, double* resid, sla_eig_info* info,
                     hipStream_t st) {
  SLA_TRY(ensure_eig_work(A, m, k));
  const int64_t n = A->n;
  sla_status first = SLA_OK;
  for (int64_t s = 0; s < A->batch; ++s) {
    const double* vals = A->vals + s * A->nnz;
    sla_eig_info inf{};
    const sla_status rc =
        lz_rows_per_thread(n) == 4
            ? lanczos_system<4>(A, vals, v0 + s * n, m, k, which, theta + s * k,
                                X + s * k * n, resid + s * k, &inf, st)
            : lanczos_system<1>(A, vals, v0 + s * n, m, k, which, theta + s * k,
                                X + s * k * n, resid + s * k, &inf, st);
    SLA_TRY(rc);
    if (info) info[s] = inf;
    if (first == SLA_OK && inf.status != SLA_OK) {
      first = sla_status(inf.status);
      set_error("sla_eigsh: system %lld: %s", (long long)s,
                inf.status == SLA_ERR_KRYLOV
                    ? "the Krylov space of v0 has fewer than k dimensions"
                    : inf.status == SLA_ERR_NONFINITE ? "non-finite value in the process"
                                                      : "v0 is zero");
    }
  }
  return first;
}

sla_status profile_lanczos_kernels(sla_csr A, int64_t nvec, int64_t reps, double* avg_ms,
                                   hipStream_t st) {
  EigWork* e = A->eig;
  if (e == nullptr || nvec < 1 || nvec > e->cap_m) {
    set_error("sla_profile_lanczos_kernels: needs an earlier sla_eigsh with m >= nvec = %lld",
              (long long)nvec);
    return SLA_ERR_ARG;
  }
  const int64_t n = A->n, G = lz_groups(n);
  // the kernels return at once once the process has stopped: clear the flag
  k_lz_reset<<<1, 1, 0, st>>>(e->st);
  LAUNCH_CHECK();
  hipEvent_t ev[4];
  for (auto& x : ev) SLA_TRY_HIP(hipEventCreate(&x));
  SLA_TRY_HIP(hipEventRecord(ev[0], st));
  for (int64_t r = 0; r < reps; ++r) lz_launch_dot(e, n, nvec, e->w, 1, st);
  SLA_TRY_HIP(hipEventRecord(ev[1], st));
  for (int64_t r = 0; r < reps; ++r) {
    if (lz_rows_per_thread(n) == 4) lz_launch_update<4>(e, n, nvec, e->h1, nullptr, G, st);
    else lz_launch_update<1>(e, n, nvec, e->h1, nullptr, G, st);
  }
  SLA_TRY_HIP(hipEventRecord(ev[2], st));
  LAUNCH_CHECK();
  SLA_TRY_HIP(hipEventSynchronize(ev[2]));
  float t0 = 0.f, t1 = 0.f;
  SLA_TRY_HIP(hipEventElapsedTime(&t0, ev[0], ev[1]));
  SLA_TRY_HIP(hipEventElapsedTime(&t1, ev[1], ev[2]));
  for (auto& x : ev) (void)hipEventDestroy(x);
  avg_ms[0] = double(t0) / double(reps);
  avg_ms[1] = double(t1) / double(reps);
  return SLA_OK;
}

sla_status launch_eig_grad(sla_csr A, int64_t k, const double* X, const double* g,
                           double* grad, hipStream_t st) {
  // a multiple of kXcds workgroups (the tile walk splits the tiles by XCD)
  int64_t per_xcd = (A->tiles + int64_t(kWaves) * kXcds - 1) / (int64_t(kWaves) * kXcds);
  per_xcd = per_xcd < 1 ? 1 : (per_xcd > 8191 ? 8191 : per_xcd);
  const int64_t blocks = per_xcd * kXcds;
  const int cap = A->wave_cap;  // >= 1 once the pattern is analysed
  const dim3 grid(unsigned(blocks), unsigned(A->batch));
  const size_t lds = size_t(kWaves) * size_t(cap);
  if (A->rp_idx == SLA_I32)
    k_eig_grad<int32_t><<<grid, kIterBlock, lds, st>>>((const int32_t*)A->rowptr, A->col, A->n,
                                                        A->nnz, A->tiles, cap, k, X, g, grad);
  else
    k_eig_grad<int64_t><<<grid, kIterBlock, lds, st>>>((const int64_t*)A->rowptr, A->col, A->n,
                                                        A->nnz, A->tiles, cap, k, X, g, grad);
  LAUNCH_CHECK();
  return SLA_OK;
}

}  // namespace sla
