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
//   * One iteration k is two kernels; nothing returns to the host inside the
//     loop.
//       SpMV step k     rr_k = sum of the r.r partials; beta = rr_k / rr_{k-1};
//                       stopping test; p_k = r_k + beta p_{k-1} (own rows, and
//                       recomputed at each gathered column); the deferred
//                       x += alpha_{k-1} p_{k-1}; q = A p_k; p.q partials
//       residual step k alpha_k = rr_k / sum of the p.q partials; breakdown
//                       test; r -= alpha_k q; r.r partials
//     Each workgroup sums the (at most a few hundred) partials of the previous
//     step itself, in one fixed order, so every workgroup obtains the same
//     bits; no one-workgroup reduction kernel and no cross-workgroup signal
//     inside a kernel is needed.  The x update is deferred by one step to the
//     pass that reads p_{k-1} anyway; when the stopping test fires, that pass
//     only applies it.  p is double-buffered because the SpMV reads p_{k-1}
//     at other waves' rows while it writes p_k.  Each element's arithmetic is
//     the textbook one (every * and + rounded on its own), so only the order
//     of the dot-product sums differs from a sequential CPU run.
//   * Rows are cut into 64-row wave tiles (one row per lane).  A tile's slots
//     [rowptr[r0], rowptr[r0+64]) are contiguous: the wave stages them into
//     its own LDS area with coalesced loads, then each lane walks its row.
//     Only wave-level synchronisation is needed, so the 16 waves of a
//     workgroup progress independently.
//   * Fixed grid of two 1024-thread workgroups per CU; each wave walks tiles
//     inside its XCD's contiguous share of the rows, interleaved with the
//     other waves of that XCD, so stencil neighbours (rows i +- N) are read
//     while still in that XCD's L2.
//   * Blocks of iterations are captured once per handle as a HIP graph; a
//     kernel returns at once when its system has stopped, and the host only
//     polls the count of running systems between blocks.
#include <algorithm>
#include <cmath>
#include <vector>

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

// Row sum of one lane's row in a wave tile: acc = sum_k vals[k] * g(col[k])
// in ascending slot order, starting from 0.  The tile's slots
// [rowptr[r0], rowptr[r1]) are contiguous: the wave stages them into its LDS
// areas `lv`/`lc` (`cap` slots) with coalesced loads, in as many chunks as
// the tile needs, and each lane adds the slots of its row that fall into the
// chunk; the ascending order of every row's sum is kept across chunks.
// Returns false for lanes past the last row.  Every lane of the wave must
// call it for the same tile.
template <typename RP, typename G>
__device__ __forceinline__ bool wave_tile_row(const RP* rowptr_, const int32_t* col_,
                                              const double* vals_, int64_t n, int64_t tile,
                                              int cap, double* lv, int32_t* lc, G g, int64_t& row,
                                              double& acc) {
  const SLA_GLOBAL RP* __restrict__ rowptr = gmem(rowptr_);
  const SLA_GLOBAL int32_t* __restrict__ col = gmem(col_);
  const SLA_GLOBAL double* __restrict__ vals = gmem(vals_);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r0 = tile * kTileRows;
  const int64_t r1 = r0 + kTileRows < n ? r0 + kTileRows : n;
  const int64_t s0 = rowptr[r0];
  const int64_t len = int64_t(rowptr[r1]) - s0;
  row = r0 + lane;
  const bool ok = row < r1;
  int64_t a = 0, e = 0;
  if (ok) {
    a = rowptr[row] - s0;
    e = rowptr[row + 1] - s0;
  }
  acc = 0.0;
  for (int64_t c0 = 0; c0 < len; c0 += cap) {
    const int clen = int(len - c0 < cap ? len - c0 : cap);
    // a lane stages at most kStageLoads slots, in rounds of kStageRound
    // whose loads are all issued before their LDS writes
#pragma unroll
    for (int j0 = 0; j0 < kStageLoads; j0 += kStageRound) {
      double v[kStageRound];
      int32_t cc[kStageRound];
#pragma unroll
      for (int j = 0; j < kStageRound; ++j) {
        const int k = lane + (j0 + j) * kWave;
        if (k < clen) {
          v[j] = vals[s0 + c0 + k];
          cc[j] = col[s0 + c0 + k];
        }
      }
#pragma unroll
      for (int j = 0; j < kStageRound; ++j) {
        const int k = lane + (j0 + j) * kWave;
        if (k < clen) {
          lv[k] = v[j];
          lc[k] = cc[j];
        }
      }
    }
    wave_sync();
    const int k0 = int(a > c0 ? a - c0 : 0);
    const int k1 = int(e - c0 < clen ? e - c0 : clen);
    for (int k = k0; k < k1; ++k) acc = acc + lv[k] * g(lc[k]);
    wave_sync();
  }
  return ok;
}

// Exclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_exclusive_sum(int v) {
  const int lane = threadIdx.x & (kWave - 1);
  int inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  return inc - v;
}

// The same row sum for a banded pattern: row i's slots are the columns
// i + band.off[t] for the bits t of mask[i], in ascending t (= ascending
// column, the CSR order).  The wave reads one row pointer per tile and one
// mask byte per row instead of the column array and per-row row pointers;
// slot positions come from a prefix sum of the rows' bit counts.  Only the
// values are staged (8 bytes per slot), chunked like the CSR form.
template <typename RP, typename G>
__device__ __forceinline__ bool wave_tile_row_band(const RP* rowptr_, const uint8_t* mask_,
                                                   const BandOffsets& band, const double* vals_,
                                                   int64_t n, int64_t tile, int cap, double* lv,
                                                   G g, int64_t& row, double& acc) {
  const SLA_GLOBAL RP* __restrict__ rowptr = gmem(rowptr_);
  const SLA_GLOBAL uint8_t* __restrict__ mask = gmem(mask_);
  const SLA_GLOBAL double* __restrict__ vals = gmem(vals_);
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t r0 = tile * kTileRows;
  const int64_t r1 = r0 + kTileRows < n ? r0 + kTileRows : n;
  const int64_t s0 = rowptr[r0];
  const int64_t len = int64_t(rowptr[r1]) - s0;
  row = r0 + lane;
  const bool ok = row < r1;
  const unsigned m = ok ? unsigned(mask[row]) : 0u;
  const int pre = wave_exclusive_sum(__builtin_popcount(m));
  acc = 0.0;
  int t = 0;     // next offset index of this lane's row
  int k = pre;   // its slot, relative to s0
  for (int64_t c0 = 0; c0 < len; c0 += cap) {
    const int clen = int(len - c0 < cap ? len - c0 : cap);
#pragma unroll
    for (int j0 = 0; j0 < kStageLoads; j0 += kStageRound) {
      double v[kStageRound];
#pragma unroll
      for (int j = 0; j < kStageRound; ++j) {
        const int kk = lane + (j0 + j) * kWave;
        if (kk < clen) v[j] = vals[s0 + c0 + kk];
      }
#pragma unroll
      for (int j = 0; j < kStageRound; ++j) {
        const int kk = lane + (j0 + j) * kWave;
        if (kk < clen) lv[kk] = v[j];
      }
    }
    wave_sync();
    for (; t < band.count && k - c0 < clen; ++t)
      if ((m >> t) & 1u) {
        acc = acc + lv[k - c0] * g(row + band.off[t]);
        ++k;
      }
    wave_sync();
  }
  return ok;
}

// This wave's LDS staging areas: 12 bytes per slot (value and column), or 8
// for a banded pattern (values only).
__device__ __forceinline__ void wave_areas(double* lds_dyn, int cap, bool banded, double*& lv,
                                           int32_t*& lc) {
  const int w = threadIdx.x / kWave;
  lv = lds_dyn + int64_t(w) * (banded ? cap : cap + (cap + 1) / 2);
  lc = reinterpret_cast<int32_t*>(lv + cap);
}

size_t solver_lds_bytes(int cap, int waves, bool banded) {
  return size_t(waves) * size_t(banded ? cap : cap + (cap + 1) / 2) * sizeof(double);
}

// Sum of `count` partials, the same fixed order in every workgroup: thread t
// adds part[t], part[t + 1024], ..., then the workgroup tree.  The result is
// in every thread.
__device__ __forceinline__ double sum_partials_all(const SLA_GLOBAL double* __restrict__ part,
                                                   int count, double* red) {
  double v = 0.0;
  for (int i = threadIdx.x; i < count; i += kIterBlock) v = v + part[i];
  return block_sum_all<kIterBlock>(v, red);
}

// ---------------------------------------------------------------------------
// Standalone SpMV: y[s] = A_s x[s]
// ---------------------------------------------------------------------------
template <typename RP, bool BANDED>
__global__ __launch_bounds__(kIterBlock) __attribute__((amdgpu_waves_per_eu(kWavesPerEu)))
void k_spmv(const RP* __restrict__ rowptr,
                                                     const int32_t* __restrict__ col,
                                                     const uint8_t* __restrict__ mask,
                                                     BandOffsets band,
                                                     const double* __restrict__ vals, int64_t n,
                                                     int64_t nnz, int64_t tiles, int cap,
                                                     const double* __restrict__ x,
                                                     double* __restrict__ y) {
  extern __shared__ double lds_dyn[];
  double* lv;
  int32_t* lc;
  wave_areas(lds_dyn, cap, BANDED, lv, lc);
  const int64_t s = blockIdx.y;
  const double* v = vals + s * nnz;
  const SLA_GLOBAL double* xs = gmem(x + s * n);
  SLA_GLOBAL double* ys = gmem(y + s * n);
  auto g = [&](int64_t j) { return xs[j]; };
  const int w = threadIdx.x / kWave;
  for (int64_t t = int64_t(blockIdx.x) * kWaves + w; t < tiles; t += int64_t(gridDim.x) * kWaves) {
    int64_t i;
    double acc;
    const bool ok = BANDED ? wave_tile_row_band<RP>(rowptr, mask, band, v, n, t, cap, lv, g, i, acc)
                           : wave_tile_row<RP>(rowptr, col, v, n, t, cap, lv, lc, g, i, acc);
    if (ok) ys[i] = acc;
  }
}

// ---------------------------------------------------------------------------
// CG kernels
// ---------------------------------------------------------------------------

// r = b (x = 0) or r = b - q with q = A x0; p_{-1} = 0; partials of b.b and
// of r_0.r_0.
__global__ __launch_bounds__(kIterBlock) void k_cg_init(const Ctx* __restrict__ c, int use_x0) {
  __shared__ double red[kWaves];
  const int64_t s = blockIdx.y, n = c->n;
  const SLA_GLOBAL double* b = gmem(c->b + s * n);
  SLA_GLOBAL double* x = gmem(c->x + s * n);
  SLA_GLOBAL double* r = gmem(c->r + s * n);
  SLA_GLOBAL double* pm = gmem(c->p[1] + s * n);
  const SLA_GLOBAL double* q = gmem(c->q + s * n);
  const int lane = threadIdx.x & (kWave - 1);
  const TileWalk w = wave_walk(c->tiles, c->grid, blockIdx.x, kWaves, threadIdx.x / kWave);
  double bb = 0.0, rr = 0.0;
  for (int64_t t = w.first; t < w.end; t += w.stride) {
    const int64_t i = t * kTileRows + lane;
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
  bb = block_sum_all<kIterBlock>(bb, red);
  rr = block_sum_all<kIterBlock>(rr, red);
  if (threadIdx.x == 0) {
    SLA_GLOBAL double* part = gmem(c->part + s * kPartSets * c->grid);
    part[4 * c->grid + blockIdx.x] = bb;
    part[0 * c->grid + blockIdx.x] = rr;
    if (blockIdx.x == 0 && s == 0) *c->n_running = 0;
  }
}

__global__ __launch_bounds__(kIterBlock) void k_cg_init_scalars(const Ctx* __restrict__ c,
                                                                double tol, int64_t maxit) {
  __shared__ double red[kWaves];
  const int64_t s = blockIdx.x;
  const SLA_GLOBAL double* part = gmem(c->part + s * kPartSets * c->grid);
  const double bb = sum_partials_all(part + 4 * c->grid, c->grid, red);
  const double rr = sum_partials_all(part + 0 * c->grid, c->grid, red);
  if (threadIdx.x == 0) {
    Scal* sc = c->scal + s;
    sc->rr[0] = rr;
    sc->rr[1] = rr;
    sc->alpha = 0.0;
    sc->bb = bb;
    sc->stop = (tol * tol) * bb;
    sc->rr_final = rr;
    sc->ka = 0;
    sc->kr = 0;
    sc->it = 0;
    sc->maxit = maxit;
    const int32_t st = (!isfinite(bb) || !isfinite(rr)) ? ST_NONFINITE : ST_RUNNING;
    sc->state_a = st;
    sc->state_r = st;
    if (st == ST_RUNNING) atomicAdd(c->n_running, 1);
  }
}

// The scalar part of SpMV step k, in every workgroup: rr_k from the r.r
// partials (the same bits everywhere), beta, the stopping test; workgroup 0
// records the history, rr_k, the step index for the residual step and, when
// the system stops, its final state.
struct StepHead {
  int64_t k;
  double alpha, beta;
  bool lag;      // x still lacks alpha_{k-1} p_{k-1}
  int32_t stop;  // ST_RUNNING or the final state
};

__device__ __forceinline__ StepHead step_head(const Ctx* __restrict__ c, int64_t s,
                                              double* red) {
  Scal* sc = c->scal + s;
  const bool lead = blockIdx.x == 0 && threadIdx.x == 0;
  const int G = c->grid;
  const SLA_GLOBAL double* part = gmem(c->part + s * kPartSets * G);
  StepHead h;
  h.k = sc->ka;
  const int64_t k = h.k;
  const double rr = sum_partials_all(part + (k & 1) * G, G, red);
  h.lag = k > 0;
  h.alpha = 0.0;
  h.beta = 0.0;
  h.stop = ST_RUNNING;
  int64_t it_stop = k;
  double rr_stop = rr;
  if (h.lag) {
    const double rr_prev = sc->rr[(k - 1) & 1];
    h.alpha = sc->alpha;
    if (!isfinite(rr)) {
      h.stop = ST_NONFINITE;  // iteration k-1 did not complete
      it_stop = k - 1;
      rr_stop = rr_prev;
    } else {
      h.beta = rr / rr_prev;
    }
  }
  if (h.stop == ST_RUNNING) {
    if (rr <= sc->stop) h.stop = ST_CONVERGED;
    else if (k >= sc->maxit) h.stop = ST_MAXIT;
  }
  if (lead) {
    if (h.lag && h.stop != ST_NONFINITE && c->hist != nullptr && k - 1 < c->hist_cap) {
      SLA_GLOBAL double* hh = gmem(c->hist + (s * c->hist_cap + (k - 1)) * 3);
      hh[0] = h.alpha;
      hh[1] = h.beta;
      hh[2] = rr;
    }
    sc->rr[k & 1] = rr;
    sc->kr = k;
    if (h.stop != ST_RUNNING) {
      sc->it = it_stop;
      sc->rr_final = rr_stop;
      sc->state_a = h.stop;
      atomicSub(c->n_running, 1);
    }
  }
  return h;
}

// SpMV step k (see the file comment): direction update, deferred x update,
// q = A p_k with p_k recomputed at each gathered column, p.Ap partials.
template <typename RP, bool BANDED>
__global__ __launch_bounds__(kIterBlock) __attribute__((amdgpu_waves_per_eu(kWavesPerEu)))
void k_cg_spmv(const Ctx* __restrict__ c) {
  extern __shared__ double lds_dyn[];
  __shared__ double red[kWaves];
  const int64_t s = blockIdx.y;
  Scal* sc = c->scal + s;
  const int32_t st_in = sc->state_r;
  if (st_in != ST_RUNNING) {
    if (blockIdx.x == 0 && threadIdx.x == 0) sc->state_a = st_in;
    return;
  }
  const StepHead h = step_head(c, s, red);
  const int64_t k = h.k;
  const double alpha = h.alpha, beta = h.beta;
  const bool lag = h.lag;
  const int G = c->grid;
  const int64_t n = c->n;
  const SLA_GLOBAL double* pold = gmem(c->p[(k + 1) & 1] + s * n);
  SLA_GLOBAL double* x = gmem(c->x + s * n);
  const int w = threadIdx.x / kWave;
  const TileWalk wk = wave_walk(c->tiles, G, blockIdx.x, kWaves, w);
  if (h.stop != ST_RUNNING) {
    // last pass: only the deferred x update
    if (lag) {
      const int lane = threadIdx.x & (kWave - 1);
      for (int64_t t = wk.first; t < wk.end; t += wk.stride) {
        const int64_t i = t * kTileRows + lane;
        if (i < n) x[i] = x[i] + alpha * pold[i];
      }
    }
    return;
  }
  const RP* rowptr = static_cast<const RP*>(c->rowptr);
  const double* vals = c->vals + s * c->nnz;
  const SLA_GLOBAL double* r = gmem(c->r + s * n);
  SLA_GLOBAL double* pnew = gmem(c->p[k & 1] + s * n);
  SLA_GLOBAL double* q = gmem(c->q + s * n);
  double* lv;
  int32_t* lc;
  wave_areas(lds_dyn, c->wave_cap, BANDED, lv, lc);
  auto g = [&](int64_t j) { return r[j] + beta * pold[j]; };
  const BandOffsets band = c->band;
  // plain row order, or the panel order for wide bands (see panel_tile)
  const bool panels = c->panel > 0;
  const int xcd = blockIdx.x % kXcds;
  const int64_t lo = c->tiles * xcd / kXcds, hi = c->tiles * (xcd + 1) / kXcds;
  const int64_t pend = panels ? panel_positions(hi - lo, c->panel, c->pblock) : wk.end - lo;
  double pq = 0.0;
  for (int64_t pos = wk.first - lo; pos < pend; pos += wk.stride) {
    const int64_t t = panels ? panel_tile(pos, lo, hi, c->panel, c->pblock) : lo + pos;
    if (t < 0) continue;
    int64_t i;
    double acc;
    const bool ok =
        BANDED ? wave_tile_row_band<RP>(rowptr, c->mask, band, vals, n, t, c->wave_cap, lv, g, i,
                                        acc)
               : wave_tile_row<RP>(rowptr, c->col, vals, n, t, c->wave_cap, lv, lc, g, i, acc);
    if (ok) {
      const double po = pold[i];
      const double pn = r[i] + beta * po;
      if (lag) x[i] = x[i] + alpha * po;
      pnew[i] = pn;
      q[i] = acc;
      pq = pq + pn * acc;
    }
  }
  pq = block_sum_all<kIterBlock>(pq, red);
  if (threadIdx.x == 0) gmem(c->part)[s * kPartSets * G + (2 + (k & 1)) * G + blockIdx.x] = pq;
}

// For patterns whose rows reach all over the matrix (no locality to reuse
// r and p_{k-1} at gathered columns), SpMV step k is split in two passes so
// that the SpMV gathers one vector instead of two:
//   direction pass:  scalars as above, p_k = r_k + beta p_{k-1}, deferred
//                    x update (own rows only, streaming);
//   product pass:    q = A p_k, p.Ap partials.
// The product pass reads the step index and state the direction pass
// recorded and writes no scalar.
__global__ __launch_bounds__(kIterBlock) __attribute__((amdgpu_waves_per_eu(kWavesPerEu)))
void k_cg_direction(const Ctx* __restrict__ c) {
  __shared__ double red[kWaves];
  const int64_t s = blockIdx.y;
  Scal* sc = c->scal + s;
  const int32_t st_in = sc->state_r;
  if (st_in != ST_RUNNING) {
    if (blockIdx.x == 0 && threadIdx.x == 0) sc->state_a = st_in;
    return;
  }
  const StepHead h = step_head(c, s, red);
  const int64_t k = h.k, n = c->n;
  const SLA_GLOBAL double* pold = gmem(c->p[(k + 1) & 1] + s * n);
  const SLA_GLOBAL double* r = gmem(c->r + s * n);
  SLA_GLOBAL double* pnew = gmem(c->p[k & 1] + s * n);
  SLA_GLOBAL double* x = gmem(c->x + s * n);
  const int lane = threadIdx.x & (kWave - 1);
  const TileWalk wk = wave_walk(c->tiles, c->grid, blockIdx.x, kWaves, threadIdx.x / kWave);
  const bool run = h.stop == ST_RUNNING;
  for (int64_t t = wk.first; t < wk.end; t += wk.stride) {
    const int64_t i = t * kTileRows + lane;
    if (i < n) {
      const double po = pold[i];
      if (h.lag) x[i] = x[i] + h.alpha * po;
      if (run) pnew[i] = r[i] + h.beta * po;
    }
  }
}

template <typename RP>
__global__ __launch_bounds__(kIterBlock) __attribute__((amdgpu_waves_per_eu(kWavesPerEu)))
void k_cg_product(const Ctx* __restrict__ c) {
  extern __shared__ double lds_dyn[];
  __shared__ double red[kWaves];
  const int64_t s = blockIdx.y;
  const Scal* sc = c->scal + s;
  if (sc->state_a != ST_RUNNING) return;
  const int64_t k = sc->kr, n = c->n;
  const int G = c->grid;
  const RP* rowptr = static_cast<const RP*>(c->rowptr);
  const double* vals = c->vals + s * c->nnz;
  const SLA_GLOBAL double* p = gmem(c->p[k & 1] + s * n);
  SLA_GLOBAL double* q = gmem(c->q + s * n);
  double* lv;
  int32_t* lc;
  wave_areas(lds_dyn, c->wave_cap, false, lv, lc);
  auto g = [&](int64_t j) { return p[j]; };
  const TileWalk wk = wave_walk(c->tiles, G, blockIdx.x, kWaves, threadIdx.x / kWave);
  double pq = 0.0;
  for (int64_t t = wk.first; t < wk.end; t += wk.stride) {
    int64_t i;
    double acc;
    if (wave_tile_row<RP>(rowptr, c->col, vals, n, t, c->wave_cap, lv, lc, g, i, acc)) {
      q[i] = acc;
      pq = pq + p[i] * acc;
    }
  }
  pq = block_sum_all<kIterBlock>(pq, red);
  if (threadIdx.x == 0) gmem(c->part)[s * kPartSets * G + (2 + (k & 1)) * G + blockIdx.x] = pq;
}

// Residual step k (see the file comment).
__global__ __launch_bounds__(kIterBlock) __attribute__((amdgpu_waves_per_eu(kWavesPerEu)))
void k_cg_residual(const Ctx* __restrict__ c) {
  __shared__ double red[kWaves];
  const int64_t s = blockIdx.y;
  Scal* sc = c->scal + s;
  const bool lead = blockIdx.x == 0 && threadIdx.x == 0;
  const int32_t st_in = sc->state_a;
  if (st_in != ST_RUNNING) {
    if (lead) sc->state_r = st_in;
    return;
  }
  const int G = c->grid;
  SLA_GLOBAL double* part = gmem(c->part + s * kPartSets * G);
  const int64_t k = sc->kr;
  const double pq = sum_partials_all(part + (2 + (k & 1)) * G, G, red);
  const double rr = sc->rr[k & 1];
  int32_t stop = ST_RUNNING;
  if (!isfinite(pq)) stop = ST_NONFINITE;
  else if (!(pq > 0.0)) stop = ST_NOT_SPD;
  if (stop != ST_RUNNING) {
    // breakdown: x already holds x_k (the SpMV step applied the lagged update)
    if (lead) {
      sc->it = k;
      sc->rr_final = rr;
      sc->state_r = stop;
      atomicSub(c->n_running, 1);
    }
    return;
  }
  const double alpha = rr / pq;
  if (lead) {
    sc->alpha = alpha;
    sc->ka = k + 1;
  }
  const int64_t n = c->n;
  SLA_GLOBAL double* r = gmem(c->r + s * n);
  const SLA_GLOBAL double* q = gmem(c->q + s * n);
  const int lane = threadIdx.x & (kWave - 1);
  const TileWalk wk = wave_walk(c->tiles, G, blockIdx.x, kWaves, threadIdx.x / kWave);
  double rn = 0.0;
  for (int64_t t = wk.first; t < wk.end; t += wk.stride) {
    const int64_t i = t * kTileRows + lane;
    if (i < n) {
      const double ri = r[i] - alpha * q[i];
      r[i] = ri;
      rn = rn + ri * ri;
    }
  }
  rn = block_sum_all<kIterBlock>(rn, red);
  if (threadIdx.x == 0) part[((k + 1) & 1) * G + blockIdx.x] = rn;
}

// grad_vals[s][k] = -lambda[s][i] * x[s][col[k]] for every stored slot k of
// row i.  The lanes of a wave walk the tile's slots in order (coalesced
// column loads and gradient stores); each slot's row comes from an LDS map
// the lanes fill for their own rows.
template <typename RP>
__global__ __launch_bounds__(kIterBlock) void k_pattern_grad(const RP* __restrict__ rowptr,
                                                             const int32_t* __restrict__ col,
                                                             int64_t n, int64_t nnz, int64_t tiles,
                                                             int cap,
                                                             const double* __restrict__ lambda,
                                                             const double* __restrict__ x,
                                                             double* __restrict__ grad) {
  extern __shared__ double lds_dyn[];
  const int w = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  uint8_t* rowmap = reinterpret_cast<uint8_t*>(lds_dyn) + int64_t(w) * cap;
  const int64_t s = blockIdx.y;
  const SLA_GLOBAL double* l = gmem(lambda + s * n);
  const SLA_GLOBAL double* xs = gmem(x + s * n);
  SLA_GLOBAL double* gs = gmem(grad + s * nnz);
  for (int64_t t = int64_t(blockIdx.x) * kWaves + w; t < tiles; t += int64_t(gridDim.x) * kWaves) {
    const int64_t r0 = t * kTileRows;
    const int64_t r1 = r0 + kTileRows < n ? r0 + kTileRows : n;
    const int64_t s0 = rowptr[r0];
    const int64_t len = int64_t(rowptr[r1]) - s0;
    const int64_t i = r0 + lane;
    int64_t a = 0, e = 0;
    if (i < r1) {
      a = rowptr[i] - s0;
      e = rowptr[i + 1] - s0;
    }
    for (int64_t c0 = 0; c0 < len; c0 += cap) {
      const int64_t clen = len - c0 < cap ? len - c0 : cap;
      for (int64_t k = (a > c0 ? a : c0); k < (e < c0 + clen ? e : c0 + clen); ++k)
        rowmap[k - c0] = uint8_t(lane);
      wave_sync();
      for (int64_t k = lane; k < clen; k += kWave)
        gs[s0 + c0 + k] = -(l[r0 + rowmap[k]] * xs[col[s0 + c0 + k]]);
      wave_sync();
    }
  }
}

size_t lds_bytes(const sla_csr A) { return solver_lds_bytes(A->wave_cap, kWaves, use_band(A)); }

template <typename RP>
sla_status enqueue_iteration(sla_csr A, int64_t batch, hipStream_t st) {
  const dim3 grid2(unsigned(A->grid), unsigned(batch));
  if (use_split(A)) {
    k_cg_direction<<<grid2, kIterBlock, 0, st>>>(A->ctx_dev);
    k_cg_product<RP><<<grid2, kIterBlock, lds_bytes(A), st>>>(A->ctx_dev);
  } else if (use_band(A)) {
    k_cg_spmv<RP, true><<<grid2, kIterBlock, lds_bytes(A), st>>>(A->ctx_dev);
  } else {
    k_cg_spmv<RP, false><<<grid2, kIterBlock, lds_bytes(A), st>>>(A->ctx_dev);
  }
  k_cg_residual<<<grid2, kIterBlock, 0, st>>>(A->ctx_dev);
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
  if (A->capture_stream == nullptr)
    SLA_TRY_HIP(hipStreamCreateWithFlags(&A->capture_stream, hipStreamNonBlocking));
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

void fill_ctx(sla_csr A, Ctx& c, const double* b, double* x, int64_t batch, bool hist) {
  c = Ctx{};
  c.rowptr = A->rowptr;
  c.col = A->col;
  c.vals = A->vals;
  c.x = x;
  c.b = b;
  c.r = A->r;
  c.p[0] = A->p0;
  c.p[1] = A->p1;
  c.q = A->q;
  c.part = A->part;
  c.scal = A->scal;
  c.hist = hist ? A->hist : nullptr;
  c.hist_cap = hist ? A->hist_cap : 0;
  c.n_running = A->n_running;
  c.n = A->n;
  c.nnz = A->nnz;
  c.batch = batch;
  c.tiles = A->tiles;
  c.grid = A->grid;
  c.wave_cap = A->wave_cap;
  c.mask = use_band(A) ? A->band_mask : nullptr;
  c.band = A->band;
  c.panel = A->panel;
  c.pblock = A->pblock;
}

// Workgroups for a one-pass kernel over `tiles` wave tiles and `batch` systems.
unsigned plain_grid(int64_t tiles, int64_t batch) {
  const int64_t need = (tiles + kWaves - 1) / kWaves;
  const int64_t target = std::max<int64_t>(1, int64_t(device_cus()) * 2 / batch);
  return unsigned(std::max<int64_t>(1, std::min(need, target)));
}

}  // namespace

bool use_split(const sla_csr A) {
  if (A->spmv_variant == SLA_SPMV_SPLIT) return true;
  return A->spmv_variant == SLA_SPMV_AUTO && !use_band(A) && A->wide_cols;
}

bool use_band(const sla_csr A) {
  if (A->band_mask == nullptr || A->spmv_variant == SLA_SPMV_CSR ||
      A->spmv_variant == SLA_SPMV_SPLIT)
    return false;
  if (A->spmv_variant == SLA_SPMV_BANDED) return true;
  // automatic: only when the CSR arrays stream from HBM rather than staying
  // in the Infinity Cache, i.e. when the bytes saved are HBM bytes
  return double(A->nnz) * 12.0 > double(kInfinityCacheBytes);
}

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
  // solver grid: two workgroups per CU in total, a multiple of the XCD count
  // per system, never more than the wave tiles need (rounded up)
  const int64_t target = std::max<int64_t>(kXcds, int64_t(device_cus()) * 2 / batch);
  int64_t g = std::min<int64_t>((A->tiles + kWaves - 1) / kWaves, target);
  g = (g + kXcds - 1) / kXcds * kXcds;
  A->grid = int32_t(std::max<int64_t>(g, kXcds));
  const size_t vec = size_t(batch) * size_t(n);
  SLA_TRY(dev_alloc(&A->r, vec, "r"));
  SLA_TRY(dev_alloc(&A->p0, vec, "p"));
  SLA_TRY(dev_alloc(&A->p1, vec, "p"));
  SLA_TRY(dev_alloc(&A->q, vec, "q"));
  SLA_TRY(dev_alloc(&A->part, size_t(kPartSets) * batch * A->grid, "partials"));
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
  const dim3 grid(plain_grid(A->tiles, batch), unsigned(batch));
  const size_t lds = lds_bytes(A);
  const bool bd = use_band(A);
  if (A->rp_idx == SLA_I32) {
    auto k = bd ? k_spmv<int32_t, true> : k_spmv<int32_t, false>;
    k<<<grid, kIterBlock, lds, st>>>((const int32_t*)A->rowptr, A->col, A->band_mask, A->band,
                                     vals, A->n, A->nnz, A->tiles, A->wave_cap, x, y);
  } else {
    auto k = bd ? k_spmv<int64_t, true> : k_spmv<int64_t, false>;
    k<<<grid, kIterBlock, lds, st>>>((const int64_t*)A->rowptr, A->col, A->band_mask, A->band,
                                     vals, A->n, A->nnz, A->tiles, A->wave_cap, x, y);
  }
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status launch_pattern_grad(sla_csr A, int64_t batch, const double* lambda, const double* x,
                               double* grad_vals, hipStream_t st) {
  const dim3 grid(plain_grid(A->tiles, batch), unsigned(batch));
  const int cap = A->wave_cap;
  const size_t lds = size_t(kWaves) * size_t(cap);
  if (A->rp_idx == SLA_I32)
    k_pattern_grad<int32_t><<<grid, kIterBlock, lds, st>>>(
        (const int32_t*)A->rowptr, A->col, A->n, A->nnz, A->tiles, cap, lambda, x, grad_vals);
  else
    k_pattern_grad<int64_t><<<grid, kIterBlock, lds, st>>>(
        (const int64_t*)A->rowptr, A->col, A->n, A->nnz, A->tiles, cap, lambda, x, grad_vals);
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
  fill_ctx(A, *A->ctx_host, b, x, batch, want_hist);
  SLA_TRY_HIP(hipMemcpyAsync(A->ctx_dev, A->ctx_host, sizeof(Ctx), hipMemcpyHostToDevice, st));

  const bool x0 = (flags & SLA_FLAG_X0) != 0;
  if (x0) SLA_TRY(launch_spmv(A, A->vals, batch, x, A->q, st));  // q = A x0
  const dim3 grid2(unsigned(A->grid), unsigned(batch));
  k_cg_init<<<grid2, kIterBlock, 0, st>>>(A->ctx_dev, x0 ? 1 : 0);
  k_cg_init_scalars<<<unsigned(batch), kIterBlock, 0, st>>>(A->ctx_dev, tol, maxit);
  LAUNCH_CHECK();
  SLA_TRY_HIP(hipMemcpyAsync(A->poll_host, A->n_running, sizeof(int), hipMemcpyDeviceToHost,
                             st));
  SLA_TRY_HIP(hipStreamSynchronize(st));

  if (A->poll_host[0] > 0) {
    // at most maxit + 1 SpMV steps: the last one only applies the x update
    const int64_t K = A->graph_block > 0 ? A->graph_block : 16;
    const int64_t nblocks = (maxit + 1 + K - 1) / K;
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
  SLA_TRY_HIP(hipMemcpyAsync(A->scal_host, A->scal, sizeof(Scal) * batch,
                             hipMemcpyDeviceToHost, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));

  sla_status first = SLA_OK;
  for (int64_t s = 0; s < batch; ++s) {
    const Scal& sc = A->scal_host[s];
    const int32_t state = sc.state_a != ST_RUNNING ? sc.state_a : sc.state_r;
    const sla_status ss = state >= SLA_ERR_NOT_SPD ? sla_status(state) : SLA_OK;
    if (info) {
      info[s].iterations = sc.it;
      info[s].rel_residual = sc.bb > 0 ? std::sqrt(sc.rr_final / sc.bb) : 0.0;
      info[s].converged = (ss == SLA_OK && sc.rr_final <= sc.stop) ? 1 : 0;
      info[s].status = ss;
    }
    if (state == ST_RUNNING && first == SLA_OK) {
      set_error("CG loop ended with a system still running (internal error)");
      first = SLA_ERR_DEVICE;
    }
    if (ss != SLA_OK && first == SLA_OK) first = ss;
  }
  if (first == SLA_ERR_NOT_SPD || first == SLA_ERR_NONFINITE)
    set_error("CG stopped: %s", first == SLA_ERR_NOT_SPD ? "p.Ap <= 0 (matrix not SPD)"
                                                         : "non-finite value");
  return first;
}

// ---------------------------------------------------------------------------
// Instrumentation: time each iteration kernel on its own
// ---------------------------------------------------------------------------
namespace {
template <typename RP>
sla_status time_kernels(sla_csr A, int64_t reps, double* avg_ms, hipStream_t st) {
  const dim3 grid2(unsigned(A->grid), 1u);
  const dim3 block(kIterBlock, 1u);
  // the SpMV step is one kernel, or the direction and product passes
  const bool split = use_split(A);
  const void* fns[3];
  size_t ldss[3];
  int nk = 0;
  if (split) {
    fns[nk] = reinterpret_cast<const void*>(&k_cg_direction);
    ldss[nk++] = 0;
    fns[nk] = reinterpret_cast<const void*>(&k_cg_product<RP>);
    ldss[nk++] = lds_bytes(A);
  } else {
    fns[nk] = use_band(A) ? reinterpret_cast<const void*>(&k_cg_spmv<RP, true>)
                          : reinterpret_cast<const void*>(&k_cg_spmv<RP, false>);
    ldss[nk++] = lds_bytes(A);
  }
  fns[nk] = reinterpret_cast<const void*>(&k_cg_residual);
  ldss[nk++] = 0;
  std::vector<hipEvent_t> ev(size_t(2 * reps), nullptr);
  for (auto& e : ev) SLA_TRY_HIP(hipEventCreate(&e));
  sla_status status = SLA_OK;
  avg_ms[0] = avg_ms[1] = 0.0;
  for (int k = 0; k < nk && status == SLA_OK; ++k) {
    void* args[1] = {&A->ctx_dev};
    for (int64_t r = 0; r < reps; ++r) {
      hipError_t e = hipExtLaunchKernel(fns[k], grid2, block, args, ldss[k], st, ev[2 * r],
                                        ev[2 * r + 1], 0);
      if (e != hipSuccess) {
        set_error("timed launch failed: %s", hipGetErrorString(e));
        status = SLA_ERR_DEVICE;
        break;
      }
    }
    if (status != SLA_OK) break;
    if (hipStreamSynchronize(st) != hipSuccess) {
      set_error("timed launch: synchronisation failed");
      status = SLA_ERR_DEVICE;
      break;
    }
    double total = 0.0;
    for (int64_t r = 0; r < reps; ++r) {
      float ms = 0.f;
      (void)hipEventElapsedTime(&ms, ev[2 * r], ev[2 * r + 1]);
      total += ms;
    }
    avg_ms[k == nk - 1 ? 1 : 0] += total / double(reps);
  }
  for (auto& e : ev)
    if (e) (void)hipEventDestroy(e);
  return status;
}
}  // namespace

sla_status profile_kernels(sla_csr A, const double* b, double* x, int64_t reps, double* avg_ms,
                           hipStream_t st) {
  // a running solve (tol 0, no iteration limit in reach) advanced by one
  // iteration, so that the timed SpMV steps include the deferred x update
  const int64_t huge = int64_t(1) << 40;
  SLA_TRY(ensure_workspace(A, 1));
  fill_ctx(A, *A->ctx_host, b, x, 1, false);
  SLA_TRY_HIP(hipMemcpyAsync(A->ctx_dev, A->ctx_host, sizeof(Ctx), hipMemcpyHostToDevice, st));
  const dim3 grid2(unsigned(A->grid), 1u);
  k_cg_init<<<grid2, kIterBlock, 0, st>>>(A->ctx_dev, 0);
  k_cg_init_scalars<<<1u, kIterBlock, 0, st>>>(A->ctx_dev, 0.0, huge);
  LAUNCH_CHECK();
  if (A->rp_idx == SLA_I32) SLA_TRY(enqueue_iteration<int32_t>(A, 1, st));
  else SLA_TRY(enqueue_iteration<int64_t>(A, 1, st));
  if (A->rp_idx == SLA_I32) return time_kernels<int32_t>(A, reps, avg_ms, st);
  return time_kernels<int64_t>(A, reps, avg_ms, st);
}

}  // namespace sla
