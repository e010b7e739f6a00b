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
//     Only wave-level synchronisation is needed, so the waves of a
//     workgroup progress independently.
//   * A fixed grid per handle, one or two workgroups per CU (solver_grid);
//     workgroups of 1024 threads, or 512 for the line walk, for the residual
//     step unless 16 waves finish it in one round of loads
//     (residual_block), and for bands in panel order (spmv_step_block).
//     Each wave walks tiles inside its XCD's contiguous share of the rows,
//     interleaved with the other waves of that XCD, so stencil neighbours
//     (rows i +- N) are read while still in that XCD's L2.
//   * Blocks of iterations are captured once per handle as a HIP graph; a
//     kernel returns at once when its system has stopped, and the host only
//     polls the count of running systems between blocks.
#include <algorithm>
#include <cmath>
#include <type_traits>
#include <vector>

#include "handle.h"

namespace sla {
CgSpace own_space(sla_csr A);  // the handle's own workspace as a space

namespace {

// Slots a lane gathers at a time in a plain CSR tile (two rounds cover the
// kStageLoads slots per lane of a full chunk).
constexpr int kSlotGather = 3;
static_assert(kStageLoads % kSlotGather == 0, "whole rounds per chunk");
// Tiles a wave keeps in flight in the streaming passes.
constexpr int kStreamTiles = 4;

// The vector a row sum gathers: v[j] = a[j] (one vector), or, with TWO,
// v[j] = a[j] + beta * b[j] (the new search direction, recomputed at each
// gathered column from r and p_{k-1}).  Loads and arithmetic are separate so
// that a row sum issues all its loads before it uses the first one.  WIDE
// selects 64-bit addresses for columns of vectors of 4 GiB or more.
template <bool TWO, bool WIDE>
struct Gather {
  const SLA_GLOBAL double* a;
  const SLA_GLOBAL double* b;
  double beta;
  // column j of the whole vector
  __device__ __forceinline__ void load(int32_t j, double& u, double& w) const {
    if constexpr (WIDE) {
      u = a[int64_t(j)];
      if constexpr (TWO) w = b[int64_t(j)];
    } else {
      u = ld(a, uint32_t(j));
      if constexpr (TWO) w = ld(b, uint32_t(j));
    }
  }
  // column base + o: `base` wave-uniform, o below 2^28
  __device__ __forceinline__ void load_at(int64_t base, uint32_t o, double& u, double& w) const {
    u = ld(a + base, o);
    if constexpr (TWO) w = ld(b + base, o);
  }
  __device__ __forceinline__ double value(double u, double w) const {
    if constexpr (TWO) return u + beta * w;
    else return u;
  }
};

// The index data of a tile that the row sum's loads depend on.  The tile
// loops load it one tile ahead, so that a tile's gathers and value loads
// are all issued in one round trip.  Raw row pointers; differences are taken
// at use.
template <typename RP>
struct TileIndex {
  // row pointers in their stored type: widening them where they are loaded
  // would wait for the load
  RP s0;       // rowptr[r0]: the tile's first slot
  RP s1;       // rowptr[r1]: one past its last slot (plain CSR)
  RP a;        // rowptr of the lane's row (plain CSR)
  RP e;        // rowptr of the next row (plain CSR)
  unsigned m;  // mask byte of the lane's row (banded)
};

// Lane `lane`'s row in the tile starting at r0, clamped to the tile's last
// row (lanes past the end compute that row again; see band_row).
__device__ __forceinline__ uint32_t tile_lane(int64_t r0, int64_t n, uint32_t lane) {
  const int64_t last = (r0 + kTileRows < n ? r0 + kTileRows : n) - 1 - r0;
  return int64_t(lane) <= last ? lane : uint32_t(last);
}

template <int NB, typename RP>
__device__ __forceinline__ TileIndex<RP> tile_index(const RP* rowptr_, const uint8_t* mask_,
                                                    int64_t n, int64_t r0, uint32_t lr) {
  const SLA_GLOBAL RP* rowptr = gmem(rowptr_);
  TileIndex<RP> x{};
  x.s0 = rowptr[r0];
  if constexpr (NB > 0) {
    x.m = unsigned(ld(gmem(mask_) + r0, lr));
  } else {
    x.s1 = rowptr[r0 + kTileRows < n ? r0 + kTileRows : n];
    x.a = ld(rowptr + r0, lr);
    x.e = ld(rowptr + r0 + 1, lr);
  }
  return x;
}

// Row sum of one lane's row in a wave tile: acc = sum_k vals[k] * v[col[k]]
// in ascending slot order, starting from 0.  The tile's slots
// [rowptr[r0], rowptr[r1]) are contiguous; the wave takes them in chunks of
// `cap`, lane l handling slots l, l + 64, ... of a chunk: it loads their
// values and columns (coalesced), gathers v at those columns (every lane
// busy, whatever the row lengths) and stores each product into the wave's
// LDS area `lv`.  Each lane then adds the products of its own row in slot
// order.  Every product and sum is rounded on its own, so the row sum has
// the bits of the sequential sum of vals[k] * v[col[k]].  Slots past the
// chunk are clamped to its last slot (those lanes store that slot's product
// again), so no load or store needs a branch.  The lane computes the row
// `ix` was loaded for; lanes past the last row of the tile compute the
// tile's last row (see band_row).  Every lane of the wave must call it for
// the same tile.
template <typename RP, typename GT>
__device__ __forceinline__ double wave_tile_row(const int32_t* col_, const double* vals_,
                                                const TileIndex<RP>& ix, int cap, double* lv,
                                                int32_t* lc, const GT& g) {
  (void)lc;
  const SLA_GLOBAL int32_t* __restrict__ col = gmem(col_);
  const SLA_GLOBAL double* __restrict__ vals = gmem(vals_);
  const uint32_t lane = lane_id();
  const int64_t s0 = uniform(int64_t(ix.s0));
  const int64_t len = uniform(int64_t(ix.s1)) - s0;
  const int64_t a = int64_t(ix.a) - s0, e = int64_t(ix.e) - s0;
  double acc = 0.0;
  for (int64_t c0 = 0; c0 < len; c0 += cap) {
    const int clen = int(len - c0 < cap ? len - c0 : cap);
    const SLA_GLOBAL double* vb = vals + s0 + c0;
    const SLA_GLOBAL int32_t* cb = col + s0 + c0;
    // kSlotGather slots per lane at a time: values and columns, then the
    // gathers, then the products into LDS
    for (int j0 = 0; j0 < kStageLoads; j0 += kSlotGather) {
      double v[kSlotGather], gu[kSlotGather], gw[kSlotGather];
      int32_t cc[kSlotGather];
#pragma unroll
      for (int j = 0; j < kSlotGather; ++j) {
        const int k = int(lane) + (j0 + j) * kWave;
        const uint32_t kc = uint32_t(k < clen ? k : clen - 1);
        v[j] = ld(vb, kc);
        cc[j] = ld(cb, kc);
      }
#pragma unroll
      for (int j = 0; j < kSlotGather; ++j) g.load(cc[j], gu[j], gw[j]);
#pragma unroll
      for (int j = 0; j < kSlotGather; ++j) {
        const int k = int(lane) + (j0 + j) * kWave;
        const int kc = k < clen ? k : clen - 1;
        lv[kc] = v[j] * g.value(gu[j], gw[j]);
      }
      if ((j0 + kSlotGather) * kWave >= clen) break;
    }
    wave_sync();
    const int k0 = int(a > c0 ? a - c0 : 0);
    const int k1 = int(e - c0 < clen ? e - c0 : clen);
    // the row's products in slot order; four LDS reads in flight at a time
    // (one round trip per four slots instead of one per slot)
    int k = k0;
    for (; k + 4 <= k1; k += 4) {
      const double p0 = lv[k], p1 = lv[k + 1], p2 = lv[k + 2], p3 = lv[k + 3];
      acc = acc + p0;
      acc = acc + p1;
      acc = acc + p2;
      acc = acc + p3;
    }
    for (; k < k1; ++k) acc = acc + lv[k];
    wave_sync();
  }
  return acc;
}

// Exclusive prefix sum over the 64 lanes of a wave, by data-parallel
// primitives (DPP) instead of lane permutes through the LDS crossbar: shifts
// by 1, 2, 4 and 8 lanes within each 16-lane row, then lane 15's total
// broadcast into rows 1 and 3 and lane 31's into rows 2 and 3.  Lanes with no
// source lane add 0.  Integer sums: exact in any order.
__device__ __forceinline__ int wave_exclusive_sum(int v) {
  int inc = v;
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x111, 0xF, 0xF, false);  // row_shr:1
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x112, 0xF, 0xF, false);  // row_shr:2
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x114, 0xF, 0xF, false);  // row_shr:4
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x118, 0xF, 0xF, false);  // row_shr:8
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x142, 0xA, 0xF, false);  // row_bcast:15
  inc += __builtin_amdgcn_update_dpp(0, inc, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return inc - v;
}

// The same row sum for a banded pattern: row i's slots are the columns
// i + band.off[t] for the bits t of mask[i], in ascending t (= ascending
// column, the CSR order).  Every load of the tile is issued before the first
// one is used, at indices clamped into range so that no load needs a branch:
// the gathered vector at all NB offsets of the band (columns clamped into
// [0, n), addressed from a wave-uniform base row), the row's mask byte, one
// row pointer per tile, and the row's values, read from the CSR array at the
// positions a prefix sum of the rows' bit counts gives.  Terms of slots the
// row does not have are dropped by a select.  No LDS and no per-row row
// pointers or column indices.  band.count <= NB.
//
// Lanes past the last row of the tile compute the tile's last row again
// (`lr`, the same bits as its own lane), so that the caller's stores need no
// branch: a branch would let the compiler sink the loads into it.
template <int NB, typename RP, typename GT>
__device__ __forceinline__ double band_row(const BandOffsets& band, const double* vals_,
                                           int64_t n, int64_t nnz, int64_t r0, uint32_t lr,
                                           bool ok, const TileIndex<RP>& ix, const GT& g) {
  const int64_t s0 = uniform(int64_t(ix.s0));
  const unsigned m = ix.m;
  // gathered columns relative to a wave-uniform base row; 32-bit arithmetic
  const int64_t lo = r0 + (band.off[0] < 0 ? band.off[0] : 0);
  const int64_t base = lo > 0 ? lo : 0;
  const int32_t d = int32_t(r0 - base) + int32_t(lr);
  const int32_t top = int32_t(n - 1 - base);
  double gu[NB], gw[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    int32_t j = t < band.count ? d + band.off[t] : d;
    j = j < 0 ? 0 : (j > top ? top : j);
    g.load_at(base, uint32_t(j), gu[t], gw[t]);
  }
  // slot of the row's first value: prefix sum over the tile's own rows, read
  // from lane lr
  const int kx = wave_exclusive_sum(ok ? __builtin_popcount(m) : 0);
  uint32_t k = uint32_t(__shfl(kx, int(lr), kWave));
  // a tile without slots starts at nnz (> 0 for a banded pattern): its
  // unused loads read the last slot instead
  const SLA_GLOBAL double* v = gmem(vals_) + (s0 < nnz ? s0 : nnz - 1);
  double a[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const bool use = t < band.count && ((m >> t) & 1u);
    a[t] = ld(v, use ? k : 0u);
    k += use ? 1u : 0u;
  }
  double acc = 0.0;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const bool use = t < band.count && ((m >> t) & 1u);
    const double sum = acc + a[t] * g.value(gu[t], gw[t]);
    acc = use ? sum : acc;
  }
  return acc;
}

// This wave's LDS staging area for plain CSR rows: 12 bytes per slot (value
// and column).
__device__ __forceinline__ void wave_areas(double* lds_dyn, int cap, double*& lv, int32_t*& lc) {
  const int w = wave_index();
  lv = lds_dyn + int64_t(w) * (cap + (cap + 1) / 2);
  lc = reinterpret_cast<int32_t*>(lv + cap);
}

size_t solver_lds_bytes(int cap, int waves) {
  return size_t(waves) * size_t(cap + (cap + 1) / 2) * sizeof(double);
}

// Sum of `count` partials, the same fixed order in every workgroup of NT
// threads: thread t adds part[t], part[t + NT], ..., then the workgroup tree.
// The result is in every thread.
template <int NT = kIterBlock>
__device__ __forceinline__ double sum_partials_all(const SLA_GLOBAL double* __restrict__ part,
                                                   int count, double* red) {
  double v = 0.0;
  for (int i = threadIdx.x; i < count; i += NT) v = v + part[i];
  return block_sum_all<NT>(v, red);
}

// The same sum into an LDS area of its own (see block_sum_once).
template <int NT = kIterBlock>
__device__ __forceinline__ double sum_partials_once(const SLA_GLOBAL double* __restrict__ part,
                                                    int count, double* red) {
  double v = 0.0;
  for (int i = threadIdx.x; i < count; i += NT) v = v + part[i];
  return block_sum_once<NT>(v, red);
}

// ---------------------------------------------------------------------------
// Standalone SpMV: y[s] = A_s x[s]
// ---------------------------------------------------------------------------
// NB > 0: banded rows with at most NB offsets; NB = 0: plain CSR rows
// (staged through LDS) with vectors below 4 GiB, gathered with 32-bit
// offsets; NB = -1: plain CSR rows with 64-bit gather addresses.
//
// ND > 0 also leaves per-workgroup partial dot products for a caller's
// iteration (BiCGStab): ND = 1 the partial of wdot.y at part[set0], ND = 2 in
// addition that of y.y at part[set1] (part[set][blockIdx.x] for system
// blockIdx.y, `pstride` doubles per system).
template <typename RP, int NB, int ND = 0, int NT = kIterBlock>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2 * (NT / kWave) / 4)))
void k_spmv(const RP* __restrict__ rowptr, const int32_t* __restrict__ col,
            const uint8_t* __restrict__ mask, BandOffsets band, const double* __restrict__ vals,
            int64_t n, int64_t nnz, int64_t tiles, int cap, const double* __restrict__ x,
            double* __restrict__ y, const double* __restrict__ wdot,
            double* __restrict__ part, int64_t pstride, int set0, int set1) {
  extern __shared__ double lds_dyn[];
  double* lv;
  int32_t* lc;
  wave_areas(lds_dyn, cap, lv, lc);
  const int64_t s = blockIdx.y;
  const double* v = vals + s * nnz;
  const SLA_GLOBAL double* xs = gmem(x + s * n);
  SLA_GLOBAL double* ys = gmem(y + s * n);
  const SLA_GLOBAL double* wd = gmem(wdot + s * n);
  const Gather<false, (NB < 0)> g{xs, nullptr, 0.0};
  const int w = wave_index();
  const uint32_t lane = lane_id();
  // each XCD walks a contiguous eighth of the tiles (the grid is a multiple
  // of kXcds), so a tile and the tiles its band reaches share one L2
  const TileWalk walk = wave_walk(tiles, int(gridDim.x), int(blockIdx.x), NT / kWave, w);
  int64_t t = walk.first;
  double d0 = 0.0, d1 = 0.0;
  // each tile's index data is loaded one tile ahead
  TileIndex<RP> ix{};
  if (t < walk.end) ix = tile_index<NB, RP>(rowptr, mask, n, t * kTileRows, tile_lane(t * kTileRows, n, lane));
  for (; t < walk.end; t += walk.stride) {
    const int64_t r0 = t * kTileRows;
    const bool ok = r0 + lane < n;
    const uint32_t lr = tile_lane(r0, n, lane);
    const TileIndex<RP> cur = ix;
    const int64_t tn = t + walk.stride;
    const int64_t tp = tn < walk.end ? tn : t;  // unconditional load (see k_cg_spmv_lines)
    ix = tile_index<NB, RP>(rowptr, mask, n, tp * kTileRows, tile_lane(tp * kTileRows, n, lane));
    double acc;
    if constexpr (NB > 0) acc = band_row<NB, RP>(band, v, n, nnz, r0, lr, ok, cur, g);
    else acc = wave_tile_row<RP>(col, v, cur, cap, lv, lc, g);
    st(ys + r0, lr, acc);
    if constexpr (ND > 0) {
      // lanes past the last row repeat the tile's last row: counted once
      const double wi = ld(wd + r0, lr);
      d0 = d0 + (ok ? wi * acc : 0.0);
      if constexpr (ND > 1) d1 = d1 + (ok ? acc * acc : 0.0);
    }
  }
  if constexpr (ND > 0) {
    // both sums in one pass: a wave sum each, one barrier, then thread 0
    // adds the waves' sums in wave order
    __shared__ double red[2][NT / kWave];
    d0 = wave_sum(d0);
    if constexpr (ND > 1) d1 = wave_sum(d1);
    if (lane == 0) {
      red[0][w] = d0;
      if constexpr (ND > 1) red[1][w] = d1;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double a = 0.0, b = 0.0;
      for (int q = 0; q < NT / kWave; ++q) {
        a = a + red[0][q];
        if constexpr (ND > 1) b = b + red[1][q];
      }
      part[s * pstride + int64_t(set0) * gridDim.x + blockIdx.x] = a;
      if constexpr (ND > 1) part[s * pstride + int64_t(set1) * gridDim.x + blockIdx.x] = b;
    }
  }
}

// ---------------------------------------------------------------------------
// CG kernels
// ---------------------------------------------------------------------------

// r = b (x = 0) or r = b - q with q = A x0; p_{-1} = 0; partials of b.b and
// of r_0.r_0.
template <typename RP>
__global__ __launch_bounds__(kIterBlock) void k_cg_init(const Ctx* __restrict__ c, int use_x0) {
  __shared__ double red[kWaves];
  const int64_t s = blockIdx.y, n = c->n;
  const SLA_GLOBAL double* b = gmem(c->b + s * n);
  SLA_GLOBAL double* x = gmem(c->x + s * n);
  SLA_GLOBAL double* r = gmem(c->r + s * n);
  SLA_GLOBAL double* pm = gmem(c->p[1] + s * n);
  const SLA_GLOBAL double* q = gmem(c->q + s * n);
  const bool jac = c->jacobi != 0;
  const SLA_GLOBAL RP* rowptr = gmem(static_cast<const RP*>(c->rowptr));
  const SLA_GLOBAL int32_t* col = gmem(c->col);
  const SLA_GLOBAL double* vals = gmem(c->vals + s * c->nnz);
  const int lane = threadIdx.x & (kWave - 1);
  const TileWalk w = wave_walk(c->tiles, c->grid, blockIdx.x, kWaves, wave_index());
  double bb = 0.0, rr = 0.0, rz = 0.0;
  bool bad = false;
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
      if (jac) {
        // the stored diagonal entry of row i (0 when the row has none)
        double d = 0.0;
        for (int64_t k = rowptr[i]; k < int64_t(rowptr[i + 1]); ++k)
          if (col[k] == i) d = vals[k];
        bad = bad || !(d > 0.0);
        const double zi = ri / d;
        gmem(const_cast<double*>(c->diag) + s * n)[i] = d;
        gmem(c->z + s * n)[i] = zi;
        rz = rz + ri * zi;
      }
    }
  }
  if (bad) c->bad[s] = 1;  // every writer stores the same value
  bb = block_sum_all<kIterBlock>(bb, red);
  rr = block_sum_all<kIterBlock>(rr, red);
  if (jac) rz = block_sum_all<kIterBlock>(rz, red);
  if (threadIdx.x == 0) {
    SLA_GLOBAL double* part = gmem(c->part + s * kPartSets * c->grid);
    part[4 * c->grid + blockIdx.x] = bb;
    part[0 * c->grid + blockIdx.x] = rr;
    if (jac) part[5 * c->grid + blockIdx.x] = rz;
    if (blockIdx.x == 0 && s == 0) *c->n_running = 0;
  }
}

__global__ __launch_bounds__(kIterBlock) void k_cg_init_scalars(const Ctx* __restrict__ c,
                                                                double tol, int64_t maxit) {
  __shared__ double red[kWaves];
  const int64_t s = blockIdx.x;
  const bool jac = c->jacobi != 0;
  const SLA_GLOBAL double* part = gmem(c->part + s * kPartSets * c->grid);
  const double bb = sum_partials_all(part + 4 * c->grid, c->grid, red);
  const double rr = sum_partials_all(part + 0 * c->grid, c->grid, red);
  const double rz = jac ? sum_partials_all(part + 5 * c->grid, c->grid, red) : 0.0;
  if (threadIdx.x == 0) {
    Scal* sc = scal_of(c, s);
    sc->rr[0] = rr;
    sc->rr[1] = rr;
    sc->rz[0] = rz;
    sc->rz[1] = rz;
    sc->alpha[0] = 0.0;
    sc->alpha[1] = 0.0;
    sc->bb = bb;
    sc->stop = (tol * tol) * bb;
    sc->rr_final = rr;
    sc->ka = 0;
    sc->kr = 0;
    sc->it = 0;
    sc->maxit = maxit;
    int32_t st = (!isfinite(bb) || !isfinite(rr) || !isfinite(rz)) ? ST_NONFINITE : ST_RUNNING;
    if (jac && c->bad[s] != 0) {
      st = ST_NOT_SPD;  // a diagonal entry is not > 0: before any iteration
      c->bad[s] = 0;    // cleared for the next solve
    }
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
  double alpha, beta;  // alpha_{k-1}, beta_k
  double alpha2;       // alpha_{k-2} (k >= 2)
  bool lag;      // x still lacks alpha_{k-1} p_{k-1}
  int32_t stop;  // ST_RUNNING or the final state
};

// What an SpMV step reads of its system's record and of the context's
// scalars, loaded at the top of the kernel and pinned (with the kernel's
// own context fields) before its first branch.  The record's fields are
// written by earlier launches only (this one writes rr[k & 1], rz[k & 1] and
// the fields after alpha); both parities are loaded, since an index from k
// would wait for k.
struct StepIn {
  int64_t k;      // index of this SpMV step (ka)
  int32_t state;  // state_r
  int32_t jacobi, grid;
  double rr0, rr1, rz0, rz1, alpha0, alpha1, stop;
  int64_t maxit;
};

// step_in from the words of load_ctx
__device__ __forceinline__ StepIn step_in_words(const CtxWords& cw) {
  StepIn in;
  in.k = SLA_REC(cw, int64_t, ka);
  in.state = SLA_REC(cw, int32_t, state_r);
  in.jacobi = SLA_CTX(cw, int32_t, jacobi);
  in.grid = SLA_CTX(cw, int32_t, grid);
  in.rr0 = SLA_REC(cw, double, rr[0]);
  in.rr1 = SLA_REC(cw, double, rr[1]);
  in.rz0 = SLA_REC(cw, double, rz[0]);
  in.rz1 = SLA_REC(cw, double, rz[1]);
  in.alpha0 = SLA_REC(cw, double, alpha[0]);
  in.alpha1 = SLA_REC(cw, double, alpha[1]);
  in.stop = SLA_REC(cw, double, stop);
  in.maxit = SLA_REC(cw, int64_t, maxit);
  return in;
}

__device__ __forceinline__ StepIn step_in(const Ctx* __restrict__ c, int64_t s) {
  const SLA_GLOBAL Scal* scg = gmem(static_cast<const Scal*>(scal_of(c, s)));
  StepIn in;
  in.k = scg->ka;
  in.state = scg->state_r;
  in.jacobi = c->jacobi;
  in.grid = c->grid;
  in.rr0 = scg->rr[0];
  in.rr1 = scg->rr[1];
  in.rz0 = scg->rz[0];
  in.rz1 = scg->rz[1];
  in.alpha0 = scg->alpha[0];
  in.alpha1 = scg->alpha[1];
  in.stop = scg->stop;
  in.maxit = scg->maxit;
  pin(in.k, in.state, in.jacobi, in.grid, in.rr0, in.rr1, in.rz0, in.rz1, in.alpha0, in.alpha1,
      in.stop, in.maxit);
  return in;
}

// `red`: two LDS areas of NT / 64 doubles that the launch uses for no
// other sum.
template <int NT = kIterBlock>
__device__ __forceinline__ StepHead step_head(const Ctx* __restrict__ c, int64_t s,
                                              const StepIn& in, double* red) {
  Scal* sc = scal_of(c, s);
  const int64_t k = in.k;
  const double rr_prev = (k & 1) ? in.rr0 : in.rr1, rz_prev = (k & 1) ? in.rz0 : in.rz1;
  // alpha_{k-1} and alpha_{k-2}, by parity
  const double alpha_in = (k & 1) ? in.alpha0 : in.alpha1, stop_at = in.stop;
  const double alpha2_in = (k & 1) ? in.alpha1 : in.alpha0;
  const int64_t maxit = in.maxit;
  const bool lead = blockIdx.x == 0 && threadIdx.x == 0;
  const int G = in.grid;
  const SLA_GLOBAL double* part = gmem(c->part + s * kPartSets * G);
  StepHead h;
  h.k = k;
  const double rr = sum_partials_once<NT>(part + (k & 1) * G, G, red);
  // Jacobi: beta from r.z, the stopping test still on r.r
  const bool jac = in.jacobi != 0;
  const double rz =
      jac ? sum_partials_once<NT>(part + (5 + (k & 1)) * G, G, red + NT / kWave) : 0.0;
  h.lag = k > 0;
  h.alpha = 0.0;
  h.alpha2 = k >= 2 ? alpha2_in : 0.0;
  h.beta = 0.0;
  h.stop = ST_RUNNING;
  int64_t it_stop = k;
  double rr_stop = rr;
  if (h.lag) {
    h.alpha = alpha_in;
    if (!isfinite(rr) || !isfinite(rz)) {
      h.stop = ST_NONFINITE;  // iteration k-1 did not complete
      it_stop = k - 1;
      rr_stop = rr_prev;
    } else {
      h.beta = jac ? rz / rz_prev : rr / rr_prev;
    }
  }
  if (h.stop == ST_RUNNING) {
    if (rr <= stop_at) h.stop = ST_CONVERGED;
    else if (k >= maxit) h.stop = ST_MAXIT;
  }
  if (lead) {
    if (h.lag && h.stop != ST_NONFINITE && c->hist != nullptr && k - 1 < c->hist_cap) {
      SLA_GLOBAL double* hh = gmem(c->hist + (s * c->hist_cap + (k - 1)) * 3);
      hh[0] = h.alpha;
      hh[1] = h.beta;
      hh[2] = rr;
    }
    sc->rr[k & 1] = rr;
    sc->rz[k & 1] = rz;
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
template <typename RP, int NB, int NT = kIterBlock>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2 * (NT / kWave) / 4)))
void k_cg_spmv(const Ctx* __restrict__ c) {
  constexpr int W = NT / kWave;
  extern __shared__ double lds_dyn[];
  __shared__ double red[3 * W];  // step head (2 areas), the p.Ap partial
  const int64_t s = blockIdx.y;
  // context fields first: read before the kernel's first store, they come
  // in through scalar loads
  const int64_t n = c->n, nnz = c->nnz, tiles = c->tiles;
  const int G = c->grid, cap = c->wave_cap, panel = c->panel, pblock = c->pblock;
  const RP* rowptr = static_cast<const RP*>(c->rowptr);
  const int32_t* col = c->col;
  const uint8_t* mask = c->mask;
  const BandOffsets band = c->band;
  const double* vals = c->vals + s * nnz;
  double* const p0 = c->p[0] + s * n;
  double* const p1 = c->p[1] + s * n;
  SLA_GLOBAL double* x = gmem(c->x + s * n);
  const SLA_GLOBAL double* r = gmem(c->rd + s * n);  // r, or z with Jacobi
  SLA_GLOBAL double* q = gmem(c->q + s * n);
  SLA_GLOBAL double* part = gmem(c->part + s * kPartSets * G);
  Scal* sc = scal_of(c, s);
  const StepIn in = step_in(c, s);
  const int32_t st_in = in.state;
  if (st_in != ST_RUNNING) {
    if (blockIdx.x == 0 && threadIdx.x == 0) sc->state_a = st_in;
    return;
  }
  const StepHead h = step_head<NT>(c, s, in, red);
  const int64_t k = uniform(h.k);
  const double alpha = uniform(h.alpha), beta = uniform(h.beta);
  const bool lag = h.lag;
  // p_{k-1} and p_k
  const SLA_GLOBAL double* pold = gmem((k & 1) ? p0 : p1);
  SLA_GLOBAL double* pnew = gmem((k & 1) ? p1 : p0);
  const TileWalk wk = wave_walk(tiles, G, blockIdx.x, W, wave_index());
  if (h.stop != ST_RUNNING) {
    // last pass: only the deferred x update
    if (lag) {
      const uint32_t lane = lane_id();
      for (int64_t t = wk.first; t < wk.end; t += wk.stride) {
        const int64_t i0 = t * kTileRows;
        if (i0 + lane < n) st(x + i0, lane, ld(x + i0, lane) + alpha * ld(pold + i0, lane));
      }
    }
    return;
  }
  double* lv;
  int32_t* lc;
  wave_areas(lds_dyn, cap, lv, lc);
  const Gather<true, (NB < 0)> g{r, pold, beta};
  const uint32_t lane = lane_id();
  // plain row order, or the panel order for wide bands (see panel_tile)
  const bool panels = panel > 0;
  const int xcd = blockIdx.x % kXcds;
  const int64_t lo = tiles * xcd / kXcds, hi = tiles * (xcd + 1) / kXcds;
  const int64_t pend = panels ? panel_positions(hi - lo, panel, pblock) : wk.end - lo;
  // the wave's next tile at or after position p (p moves to it), or -1
  auto next_tile = [&](int64_t& p) -> int64_t {
    for (; p < pend; p += wk.stride) {
      const int64_t tt = panels ? panel_tile(p, lo, hi, panel, pblock) : lo + p;
      if (tt >= 0) return tt;
    }
    return -1;
  };
  double pq = 0.0;
  int64_t pos = wk.first - lo;
  int64_t t = next_tile(pos);
  // each tile's index data is loaded one tile ahead
  TileIndex<RP> ix{};
  if (t >= 0) ix = tile_index<NB, RP>(rowptr, mask, n, t * kTileRows, tile_lane(t * kTileRows, n, lane));
  while (t >= 0) {
    const int64_t r0 = t * kTileRows;
    const bool own = r0 + lane < n;
    const uint32_t lr = tile_lane(r0, n, lane);
    const TileIndex<RP> cur = ix;
    pos += wk.stride;
    const int64_t tn = next_tile(pos);
    const int64_t tp = tn >= 0 ? tn : t;  // unconditional load (see k_cg_spmv_lines)
    ix = tile_index<NB, RP>(rowptr, mask, n, tp * kTileRows, tile_lane(tp * kTileRows, n, lane));
    // this row's own operands, loaded before the row sum's loads
    const double po = ld(pold + r0, lr);
    const double ro = ld(r + r0, lr);
    const double xo = ld(x + r0, lr);
    double acc;
    if constexpr (NB > 0) acc = band_row<NB, RP>(band, vals, n, nnz, r0, lr, own, cur, g);
    else acc = wave_tile_row<RP>(col, vals, cur, cap, lv, lc, g);
    // lanes past the last row store the same bits as the row's own lane
    const double pn = ro + beta * po;
    if (lag) st(x + r0, lr, xo + alpha * po);
    st(pnew + r0, lr, pn);
    st(q + r0, lr, acc);
    const double pq1 = pq + pn * acc;
    pq = own ? pq1 : pq;
    t = tn;
  }
  pq = block_sum_once<NT>(pq, red + 2 * W);
  if (threadIdx.x == 0) part[(2 + (k & 1)) * G + blockIdx.x] = pq;
}

// SpMV step k for a band whose far offsets are +-L and whose other offsets
// lie within +-63: the matrix of a stencil on a grid whose lines hold L
// points (the 5-point Laplacian on an N x N grid: L = N).  Same arithmetic as
// k_cg_spmv, different tiles and walk:
//   * tile (u, v) is the points u*64 .. u*64+63 of grid line v (rows
//     v*L + u*64 + lane; shorter at the end of a line and of the matrix), so
//     the +-L neighbours of a tile are the tiles (u, v+-1), lane for lane;
//   * each wave walks one tile column u down a chunk of lines.  It loads the
//     next tile's r and p_{k-1} once, as the current tile's +L neighbours,
//     and keeps them as that tile's own operands in the next step; the -L
//     neighbours are the previous tile's p_k, still in registers.  r and
//     p_{k-1} thus come from memory once per row (plus the tiles just above
//     and below each chunk), whatever the line length;
//   * NEAR1 (the offsets between -L and +L are -1, 0, +1): the +-1
//     neighbours are the current tile's own p_k, moved across lanes, and at
//     the two ends of the tile the rows just outside it, loaded (one address
//     for the whole wave) together with the next tile, when the waves of the
//     neighbouring columns load those rows' lines too;
//   * otherwise offsets within +-63 are gathered as in band_row: they fall
//     in the tile's own cache lines or the neighbouring columns'.
// Lines are split into kXcds contiguous ranges, one per XCD; a range into
// `chunks` chunks; a workgroup takes kLineWaves adjacent columns of one
// chunk.  Workgroups of kLineWaves waves, one per CU by default (two when
// asked for, which the register bound of 128 per lane allows), enough to
// keep the next tile, its edge rows and the current tile's values in flight
// together.
template <typename RP, int NB, bool NEAR1, bool PIPE>
__global__ __launch_bounds__(kLineWaves * kWave)
__attribute__((amdgpu_waves_per_eu(kLineWavesPerEu)))
void k_cg_spmv_lines(const Ctx* __restrict__ c) {
  constexpr int NT = kLineWaves * kWave;
  __shared__ double red[3 * kLineWaves];  // step head (2 areas), the p.Ap partial
  const int64_t s = blockIdx.y;
  // The context fields and the system's record, read before the first
  // branch: the pipelined walk takes them from one vector load (load_ctx),
  // which leaves its deeper pipeline fewer scalar registers to spill (2000^2
  // and 4000^2 grids 2.6 and 0.9 % faster per iteration); the one-tile walk
  // keeps scalar loads, which its waves find in the scalar cache (the vector
  // load measured slower there).
  struct WalkIn {
    int64_t n, nnz, tiles, L;
    int G, chunks;
    const void* rowptr;
    const uint8_t* mask;
    BandOffsets band;
    const double *vals, *rd;
    double *p0, *p1, *x, *q, *part;
    StepIn in;
  };
  WalkIn wi;
  if constexpr (PIPE) {
    const CtxWords cw = load_ctx(c, s);
    wi = WalkIn{SLA_CTX(cw, int64_t, n), SLA_CTX(cw, int64_t, nnz), SLA_CTX(cw, int64_t, tiles),
                SLA_CTX(cw, int64_t, line), SLA_CTX(cw, int32_t, grid),
                SLA_CTX(cw, int32_t, line_chunks), SLA_CTX(cw, const void*, rowptr),
                SLA_CTX(cw, const uint8_t*, mask), ctx_band(cw), SLA_CTX(cw, const double*, vals),
                SLA_CTX(cw, const double*, rd), SLA_CTX(cw, double*, p[0]),
                SLA_CTX(cw, double*, p[1]), SLA_CTX(cw, double*, x), SLA_CTX(cw, double*, q),
                SLA_CTX(cw, double*, part), step_in_words(cw)};
  } else {
    wi = WalkIn{c->n, c->nnz, c->tiles, c->line, c->grid, c->line_chunks, c->rowptr, c->mask,
                c->band, c->vals, c->rd, c->p[0], c->p[1], c->x, c->q, c->part, step_in(c, s)};
    pin(wi.n, wi.nnz, wi.tiles, wi.L, wi.G, wi.chunks, wi.rowptr, wi.mask, wi.band.count, wi.vals,
        wi.rd, wi.p0, wi.p1, wi.x, wi.q, wi.part);
  }
  const int64_t n = wi.n, nnz = wi.nnz, tiles = wi.tiles, L = wi.L;
  const int G = wi.G, chunks = wi.chunks;
  const RP* rowptr = static_cast<const RP*>(wi.rowptr);
  const uint8_t* mask = wi.mask;
  const BandOffsets band = wi.band;
  const double* vals = wi.vals + s * nnz;
  double* const p0 = wi.p0 + s * n;
  double* const p1 = wi.p1 + s * n;
  SLA_GLOBAL double* x = gmem(wi.x + s * n);
  const SLA_GLOBAL double* r = gmem(wi.rd + s * n);  // r, or z with Jacobi
  SLA_GLOBAL double* q = gmem(wi.q + s * n);
  SLA_GLOBAL double* part = gmem(wi.part + s * kPartSets * G);
  Scal* sc = scal_of(c, s);
  const StepIn in = wi.in;
  const int64_t k = in.k;
  const int32_t st_in = in.state;
  if (st_in != ST_RUNNING) {
    if (blockIdx.x == 0 && threadIdx.x == 0) sc->state_a = st_in;
    return;
  }
  const SLA_GLOBAL double* pold = gmem((k & 1) ? p0 : p1);
  SLA_GLOBAL double* pnew = gmem((k & 1) ? p1 : p0);
  const int w = wave_index();
  const uint32_t lane = lane_id();
  const int64_t U = (L + kTileRows - 1) / kTileRows;  // tile columns per line
  const int64_t V = (n + L - 1) / L;                  // lines
  const int64_t groups = (U + kLineWaves - 1) / kLineWaves;
  const int64_t units = groups * chunks;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds, per_xcd = G / kXcds;
  const int64_t va = V * xcd / kXcds, vb = V * (xcd + 1) / kXcds;
  // A unit of the walk: tile column u over the lines [v0, v1).  Units are
  // numbered group first, so that the workgroups of an XCD, which take
  // consecutive units, walk side by side across whole grid lines of one or
  // two chunks at a time: fewer places in memory are open at once than with
  // chunk-first numbering (the same units, 5-6 % faster at 169M unknowns),
  // and neighbouring groups' edge rows meet in the XCD's L2.  A unit with no
  // rows (past the last unit, a column past the line, an empty chunk) stands
  // for column 0 on line 0: its loads stay in the matrix, and it is not
  // walked.
  struct Unit {
    int64_t v0, v1, col0, lenu;
    bool ok;
  };
  auto unit_at = [&](int64_t unit) -> Unit {
    const int64_t u = (unit % groups) * kLineWaves + w;
    const int64_t ch = unit / groups;
    const int64_t v0 = va + (vb - va) * ch / chunks, v1 = va + (vb - va) * (ch + 1) / chunks;
    const int64_t col0 = u * kTileRows;
    if (unit >= units || u >= U || v0 >= v1 || v0 * L + col0 >= n)
      return Unit{0, 1, 0, L < kTileRows ? L : kTileRows, false};
    return Unit{v0, v1, col0, L - col0 < kTileRows ? L - col0 : kTileRows, true};
  };
  // rows of tile v: v*L + col0 + [0, len(v)); lane clamped to the last one
  auto tile_len = [&](const Unit& ug, int64_t v) -> int64_t {
    const int64_t left = n - (v * L + ug.col0);
    return left < ug.lenu ? left : ug.lenu;
  };
  auto clamp_lane = [&](int64_t len) -> uint32_t {
    return int64_t(lane) < len ? lane : uint32_t(len - 1);
  };
  // A tile of the walk: first row, the lane's (clamped) row, its length; a
  // line past the matrix stands for the tile before it (its loads repeat
  // that tile's, unconditionally, and nothing of them is used).
  struct TileRef {
    int64_t r0;
    int64_t len;
    uint32_t lr;
    bool has;
  };
  auto tile_ref = [&](const Unit& ug, int64_t v, const TileRef& before) -> TileRef {
    const int64_t lv = v < V ? tile_len(ug, v) : 0;
    if (lv > 0) return TileRef{v * L + ug.col0, lv, clamp_lane(lv), true};
    return TileRef{before.r0, before.len, before.lr, false};
  };
  // rows just outside a tile (NEAR1): r and p_{k-1} at r0 - 1 and r0 + len,
  // clamped into [0, n); the same value in every lane
  auto edges = [&](int64_t e0, int64_t elen, double& rl, double& pl, double& rr, double& pr) {
    const int64_t a = e0 > 0 ? e0 - 1 : 0;
    const int64_t b = e0 + elen < n ? e0 + elen : n - 1;
    rl = ld(r + a, 0u);
    pl = ld(pold + a, 0u);
    rr = ld(r + b, 0u);
    pr = ld(pold + b, 0u);
  };
  // A unit's loads that need no scalar of the step: r and p_{k-1} of the
  // tile below the first (the -L neighbours; the first tile itself on the
  // first line, not used), of the first tile and (PIPE) the second, their
  // index data, the first tile's edge rows and (PIPE) its x.
  struct Pre {
    double rb, pb, rc, pc, rn, pn;
    TileIndex<RP> ix0, ix1;
    double rl, pl, rr, pr, x0, q0;
  };
  // this step's x update (see below): known before the step's scalars
  const bool xs = k >= 2 && (k & 1) == 0;
  auto issue = [&](const Unit& ug) -> Pre {
    Pre e{};
    const int64_t first = ug.v0 * L + ug.col0;
    const int64_t len0 = tile_len(ug, ug.v0);
    const uint32_t l0 = clamp_lane(len0);
    const int64_t b0 = ug.v0 >= 1 ? first - L : first;
    const uint32_t lb = ug.v0 >= 1 ? clamp_lane(ug.lenu) : l0;
    e.rb = ld(r + b0, lb);
    e.pb = ld(pold + b0, lb);
    e.rc = ld(r + first, l0);
    e.pc = ld(pold + first, l0);
    if constexpr (PIPE) {
      const TileRef t0{first, len0, l0, true};
      const TileRef t1 = tile_ref(ug, ug.v0 + 1, t0);
      e.rn = ld(r + t1.r0, t1.lr);
      e.pn = ld(pold + t1.r0, t1.lr);
      e.ix0 = tile_index<NB, RP>(rowptr, mask, n, first, l0);
      e.ix1 = tile_index<NB, RP>(rowptr, mask, n, t1.r0, t1.lr);
    } else {
      e.ix0 = tile_index<NB, RP>(rowptr, mask, n, first, l0);
    }
    if constexpr (NEAR1) edges(first, len0, e.rl, e.pl, e.rr, e.pr);
    if constexpr (PIPE) {
      if (xs) {
        e.x0 = ld(x + first, l0);
        e.q0 = ld(pnew + first, l0);  // p_{k-2}, before p_k replaces it
      }
    }
    return e;
  };
  Pre pre = issue(unit_at(slot));
  const StepHead h = step_head<NT>(c, s, in, red);
  const double alpha = uniform(h.alpha), beta = uniform(h.beta);
  const bool lag = h.lag;
  if (h.stop != ST_RUNNING) {
    // last pass: only the pending x updates (two after an odd step: p_{k-2}
    // is still in the buffer this step would have overwritten)
    if (lag) {
      const bool two = (k & 1) == 0;
      const double alpha2 = uniform(h.alpha2);
      const TileWalk wk = wave_walk(tiles, G, blockIdx.x, kLineWaves, w);
      for (int64_t t = wk.first; t < wk.end; t += wk.stride) {
        const int64_t i0 = t * kTileRows;
        if (i0 + lane < n) {
          double xi = ld(x + i0, lane);
          if (two) xi = xi + alpha2 * ld(pnew + i0, lane);
          st(x + i0, lane, xi + alpha * ld(pold + i0, lane));
        }
      }
    }
    return;
  }
  // this step's x update: alpha_{k-2} p_{k-2} (read from the buffer before
  // p_k replaces it) and alpha_{k-1} p_{k-1} at even k >= 2, none at odd k;
  // the walk is compiled with and without it (a store behind a branch would
  // make the compiler wait for older stores)
  const double alpha2 = uniform(h.alpha2);
  // offsets: off[0] = -L and off[count-1] = +L (from registers), 0 (the row
  // itself), the others within +-63 (gathered)
  const Gather<true, false> g{r, pold, beta};
  double pq = 0.0;
  auto walk = [&](auto xs_tag) {
    constexpr bool XS = decltype(xs_tag)::value;
    for (int64_t unit = slot; unit < units; unit += per_xcd) {
      const Unit ug = unit_at(unit);
      if (ug.ok) {
        const int64_t v0 = ug.v0, v1 = ug.v1, col0 = ug.col0, lenu = ug.lenu;
        wait_vmem();
        // -L neighbours of the first tile
        double pprev = v0 >= 1 ? pre.rb + beta * pre.pb : 0.0;
        if constexpr (PIPE) {
          // the tile's values at the slot positions of the lane's row (see
          // band_row): issued from index data loaded a step earlier
          auto load_values = [&](const TileIndex<RP>& ixv, const TileRef& tr, double (&a)[NB],
                                 unsigned& m) {
            const int64_t s0 = uniform(int64_t(ixv.s0));
            m = ixv.m;
            const bool ownv = int64_t(lane) < tr.len;
            const int kx = wave_exclusive_sum(ownv ? __builtin_popcount(m) : 0);
            uint32_t kk = uint32_t(__shfl(kx, int(tr.lr), kWave));
            const SLA_GLOBAL double* vb_ = gmem(vals) + (s0 < nnz ? s0 : nnz - 1);
    #pragma unroll
            for (int t = 0; t < NB; ++t) {
              const bool use = t < band.count && ((m >> t) & 1u);
              a[t] = ld(vb_, use ? kk : 0u);
              kk += use ? 1u : 0u;
            }
          };
          // nothing past the chunk is loaded but the +L neighbours of its last
          // tile: later tiles' loads repeat the tile before (cache hits)
          auto pick = [&](bool c, const TileRef& a_, const TileRef& b_) -> TileRef {
            return TileRef{c ? a_.r0 : b_.r0, c ? a_.len : b_.len, c ? a_.lr : b_.lr,
                           c ? a_.has : b_.has};
          };
          // The walk is a pipeline two tiles deep: step v computes tile v from
          // data issued in the steps before, and issues r, p_{k-1} and the index
          // data of tile v + 2, and the values, x and edge rows of tile v + 1.
          TileRef tc{v0 * L + col0, tile_len(ug, v0), 0u, true};
          tc.lr = clamp_lane(tc.len);
          TileRef t1 = tile_ref(ug, v0 + 1, tc);
          double rc = pre.rc, pc = pre.pc, rn = pre.rn, pn = pre.pn;
          TileIndex<RP> ixc = pre.ix0, ix1 = pre.ix1;
          double rl = pre.rl, pl = pre.pl, rr = pre.rr, pr = pre.pr;
          double a[NB];
          unsigned m = 0;
          load_values(ixc, tc, a, m);
          double xo = pre.x0, xq = pre.q0;
          for (int64_t v = v0; v < v1; ++v) {
            const int64_t r0 = tc.r0;
            const uint32_t lr = tc.lr;
            const int64_t len = tc.len;
            const bool own = int64_t(lane) < len;
            // tile v + 2: r, p_{k-1} and index data (the +L neighbours of tile
            // v + 1, read in the next step; needed up to tile v1)
            const TileRef t2 = pick(v + 2 <= v1, tile_ref(ug, v + 2, t1), t1);
            const double rn2 = ld(r + t2.r0, t2.lr), pn2 = ld(pold + t2.r0, t2.lr);
            const TileIndex<RP> ix2 = tile_index<NB, RP>(rowptr, mask, n, t2.r0, t2.lr);
            // tile v + 1: x and edge rows, then its values (inside the chunk only)
            const bool in1 = v + 1 < v1;
            const TileRef tv = pick(in1, t1, tc);
            double xn = 0.0, qn = 0.0;
            if constexpr (XS) {
              xn = ld(x + tv.r0, tv.lr);
              qn = ld(pnew + tv.r0, tv.lr);  // p_{k-2}, before p_k replaces it
            }
            double rln = 0.0, pln = 0.0, rrn = 0.0, prn = 0.0;
            if constexpr (NEAR1) edges(tv.r0, tv.len, rln, pln, rrn, prn);
            double an[NB];
            unsigned mn = 0;
            TileIndex<RP> ixv = ixc;
            ixv.s0 = in1 ? ix1.s0 : ixc.s0;
            ixv.m = in1 ? ix1.m : ixc.m;
            load_values(ixv, tv, an, mn);
            // near offsets of tile v, gathered; the other kinds read the row
            // itself (no branch; the value is not used)
            const int64_t lo = r0 - kTileRows;
            const int64_t base = lo > 0 ? lo : 0;
            const int32_t d = int32_t(r0 - base) + int32_t(lr);
            const int32_t top = int32_t(n - 1 - base);
            // offsets are sorted: -L first, +L last, the near ones in between
            double gu[NB], gw[NB];
            if constexpr (!NEAR1) {
      #pragma unroll
              for (int t = 1; t < NB - 1; ++t) {
                const int32_t o = t < band.count - 1 ? band.off[t] : 0;
                int32_t j = d + o;
                j = j < 0 ? 0 : (j > top ? top : j);
                g.load_at(base, uint32_t(j), gu[t], gw[t]);
              }
            }
            // p_k at the row, below (-L) and above (+L)
            const double pcur = rc + beta * pc;
            const double pnext = rn + beta * pn;
            // lanes past the end of a short tile compute its last row: take that
            // row's -L value (the previous tile was loaded lane for lane)
            const double pbelow = len < lenu ? __shfl(pprev, int(lr), kWave) : pprev;
            // NEAR1: p_k at the rows before and after, from the neighbouring lanes
            // or, at the ends of the tile, from the rows just outside it
            double pm1 = 0.0, pp1 = 0.0;
            if constexpr (NEAR1) {
              const double sm = __shfl(pcur, int(lr) - 1 >= 0 ? int(lr) - 1 : 0, kWave);
              const double sp = __shfl(pcur, int64_t(lr) + 1 < len ? int(lr) + 1 : int(lr), kWave);
              pm1 = lr == 0 ? rl + beta * pl : sm;
              pp1 = int64_t(lr) + 1 >= len ? rr + beta * pr : sp;
            }
            double acc = 0.0;
      #pragma unroll
            for (int t = 0; t < NB; ++t) {
              const int32_t o = t < band.count ? band.off[t] : 0;
              const bool use = t < band.count && ((m >> t) & 1u);
              double gv;
              if (t == 0) gv = pbelow;
              else if (t == NB - 1) gv = pnext;
              else if (t == band.count - 1) gv = pnext;
              else if (o == 0) gv = pcur;
              else if constexpr (NEAR1) gv = o < 0 ? pm1 : pp1;
              else gv = g.value(gu[t], gw[t]);
              const double sum = acc + a[t] * gv;
              acc = use ? sum : acc;
            }
            // lanes past the last row store the same bits as the row's own lane
            if constexpr (XS) st(x + r0, lr, (xo + alpha2 * xq) + alpha * pc);
            st(pnew + r0, lr, pcur);
            st(q + r0, lr, acc);
            const double pq1 = pq + pcur * acc;
            pq = own ? pq1 : pq;
            // shift the walk down one line
            if (!t1.has) break;
            pprev = pcur;
            rc = rn;
            pc = pn;
            rn = rn2;
            pn = pn2;
      #pragma unroll
            for (int t = 0; t < NB; ++t) a[t] = an[t];
            m = mn;
            xo = xn;
            xq = qn;
            if constexpr (NEAR1) {
              rl = rln;
              pl = pln;
              rr = rrn;
              pr = prn;
            }
            ixc = ix1;
            ix1 = ix2;
            tc = t1;
            t1 = t2;
          }
        } else {
          // the walk with one tile of look-ahead (r, p_{k-1} and index data of
          // the next tile); shorter chunks run faster this way
          int64_t len = tile_len(ug, v0);
          uint32_t lr = clamp_lane(len);
          double rc = pre.rc, pc = pre.pc;
          TileIndex<RP> ix = pre.ix0;
          // the current tile's edge rows live in scalar registers (the same value
          // in every lane); the next tile's arrive in vector registers
          double rl = 0.0, pl = 0.0, rr = 0.0, pr = 0.0;
          if constexpr (NEAR1) {
            rl = uniform(pre.rl);
            pl = uniform(pre.pl);
            rr = uniform(pre.rr);
            pr = uniform(pre.pr);
          }
          for (int64_t v = v0; v < v1; ++v) {
            const int64_t r0 = v * L + col0;
            const bool own = int64_t(lane) < len;
            // the next tile: +L neighbours now, own operands in the next step
            const int64_t lenn = v + 1 < V ? tile_len(ug, v + 1) : 0;
            const bool hasn = lenn > 0;
            const int64_t rn0 = hasn ? r0 + L : r0;
            const uint32_t lrn = hasn ? clamp_lane(lenn) : lr;
            const double rn = ld(r + rn0, lrn), pn = ld(pold + rn0, lrn);
            double rln = 0.0, pln = 0.0, rrn = 0.0, prn = 0.0;
            if constexpr (NEAR1) edges(rn0, hasn ? lenn : len, rln, pln, rrn, prn);
            const TileIndex<RP> cur = ix;
            // unconditional (the current tile again when there is no next one): a
            // conditional load would make the compiler copy the old value into its
            // register first, which waits for older loads and stores
            ix = tile_index<NB, RP>(rowptr, mask, n, rn0, lrn);
            double xo = 0.0, xq = 0.0;
            if constexpr (XS) {
              xo = ld(x + r0, lr);
              xq = ld(pnew + r0, lr);  // p_{k-2}, before p_k replaces it
            }
            // near offsets, gathered; the other kinds read the row itself (no
            // branch; the value is not used)
            const int64_t lo = r0 - kTileRows;
            const int64_t base = lo > 0 ? lo : 0;
            const int32_t d = int32_t(r0 - base) + int32_t(lr);
            const int32_t top = int32_t(n - 1 - base);
            // offsets are sorted: -L first, +L last, the near ones in between
            double gu[NB], gw[NB];
            if constexpr (!NEAR1) {
      #pragma unroll
              for (int t = 1; t < NB - 1; ++t) {
                const int32_t o = t < band.count - 1 ? band.off[t] : 0;
                int32_t j = d + o;
                j = j < 0 ? 0 : (j > top ? top : j);
                g.load_at(base, uint32_t(j), gu[t], gw[t]);
              }
            }
            // values at the slot positions of the row (see band_row)
            const int64_t s0 = uniform(int64_t(cur.s0));
            const unsigned m = cur.m;
            const int kx = wave_exclusive_sum(own ? __builtin_popcount(m) : 0);
            uint32_t kk = uint32_t(__shfl(kx, int(lr), kWave));
            const SLA_GLOBAL double* vb_ = gmem(vals) + (s0 < nnz ? s0 : nnz - 1);
            double a[NB];
      #pragma unroll
            for (int t = 0; t < NB; ++t) {
              const bool use = t < band.count && ((m >> t) & 1u);
              a[t] = ld(vb_, use ? kk : 0u);
              kk += use ? 1u : 0u;
            }
            // p_k at the row, below (-L) and above (+L)
            const double pcur = rc + beta * pc;
            const double pnext = rn + beta * pn;
            // lanes past the end of a short tile compute its last row: take that
            // row's -L value (the previous tile was loaded lane for lane)
            const double pbelow = len < lenu ? __shfl(pprev, int(lr), kWave) : pprev;
            // NEAR1: p_k at the rows before and after, from the neighbouring lanes
            // or, at the ends of the tile, from the rows just outside it
            double pm1 = 0.0, pp1 = 0.0;
            if constexpr (NEAR1) {
              const double sm = __shfl(pcur, int(lr) - 1 >= 0 ? int(lr) - 1 : 0, kWave);
              const double sp = __shfl(pcur, int64_t(lr) + 1 < len ? int(lr) + 1 : int(lr), kWave);
              pm1 = lr == 0 ? rl + beta * pl : sm;
              pp1 = int64_t(lr) + 1 >= len ? rr + beta * pr : sp;
            }
            double acc = 0.0;
      #pragma unroll
            for (int t = 0; t < NB; ++t) {
              const int32_t o = t < band.count ? band.off[t] : 0;
              const bool use = t < band.count && ((m >> t) & 1u);
              double gv;
              if (t == 0) gv = pbelow;
              else if (t == NB - 1) gv = pnext;
              else if (t == band.count - 1) gv = pnext;
              else if (o == 0) gv = pcur;
              else if constexpr (NEAR1) gv = o < 0 ? pm1 : pp1;
              else gv = g.value(gu[t], gw[t]);
              const double sum = acc + a[t] * gv;
              acc = use ? sum : acc;
            }
            // lanes past the last row store the same bits as the row's own lane
            if constexpr (XS) st(x + r0, lr, (xo + alpha2 * xq) + alpha * pc);
            st(pnew + r0, lr, pcur);
            st(q + r0, lr, acc);
            const double pq1 = pq + pcur * acc;
            pq = own ? pq1 : pq;
            // shift the walk down one line
            pprev = pcur;
            rc = rn;
            pc = pn;
            if constexpr (NEAR1) {
              rl = uniform(rln);
              pl = uniform(pln);
              rr = uniform(rrn);
              pr = uniform(prn);
            }
            len = lenn;
            lr = lrn;
            if (!hasn) break;
          }
        }
      }
      // the next unit's first loads
      if (unit + per_xcd < units) pre = issue(unit_at(unit + per_xcd));
    }
  };
  if (xs) walk(std::true_type{});
  else walk(std::false_type{});
  pq = block_sum_once<NT>(pq, red + 2 * kLineWaves);
  if (threadIdx.x == 0) part[(2 + (k & 1)) * G + blockIdx.x] = pq;
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
  __shared__ double red[2 * kWaves];  // step head
  const int64_t s = blockIdx.y;
  // context fields first (scalar loads, see k_cg_spmv)
  const int64_t n = c->n, tiles = c->tiles;
  const int G = c->grid;
  double* const p0 = c->p[0] + s * n;
  double* const p1 = c->p[1] + s * n;
  const SLA_GLOBAL double* r = gmem(c->rd + s * n);  // r, or z with Jacobi
  SLA_GLOBAL double* x = gmem(c->x + s * n);
  Scal* sc = scal_of(c, s);
  const StepIn in = step_in(c, s);
  const int32_t st_in = in.state;
  if (st_in != ST_RUNNING) {
    if (blockIdx.x == 0 && threadIdx.x == 0) sc->state_a = st_in;
    return;
  }
  const StepHead h = step_head(c, s, in, red);
  const int64_t k = uniform(h.k);
  const double alpha = uniform(h.alpha), beta = uniform(h.beta);
  const SLA_GLOBAL double* pold = gmem((k & 1) ? p0 : p1);
  SLA_GLOBAL double* pnew = gmem((k & 1) ? p1 : p0);
  const uint32_t lane = lane_id();
  const TileWalk wk = wave_walk(tiles, G, blockIdx.x, kWaves, wave_index());
  const bool run = h.stop == ST_RUNNING;
  // kStreamTiles tiles per round, all loads first and unconditional (rows
  // past the range read a valid row whose value is not used: a conditional
  // load would make the compiler keep the old register value, which waits
  // for every older load)
  for (int64_t t0 = wk.first; t0 < wk.end; t0 += kStreamTiles * wk.stride) {
    double po[kStreamTiles], xv[kStreamTiles], rv[kStreamTiles];
#pragma unroll
    for (int u = 0; u < kStreamTiles; ++u) {
      const int64_t t = t0 + u * wk.stride;
      const int64_t i0 = (t < wk.end ? t : t0) * kTileRows;
      const uint32_t li = i0 + lane < n ? lane : uint32_t(n - 1 - i0);
      po[u] = ld(pold + i0, li);
      xv[u] = ld(x + i0, li);
      rv[u] = ld(r + i0, li);
    }
    // unconditional stores too (see k_cg_residual): a lane past the range
    // stores what its loaded row's own lane stores; without the lagged
    // update x is stored back unchanged, and in the last pass p_k is not
    // formed (the buffer gets p_{k-1}, unused afterwards)
#pragma unroll
    for (int u = 0; u < kStreamTiles; ++u) {
      const int64_t t = t0 + u * wk.stride;
      const int64_t i0 = (t < wk.end ? t : t0) * kTileRows;
      const uint32_t li = i0 + lane < n ? lane : uint32_t(n - 1 - i0);
      st(x + i0, li, h.lag ? xv[u] + alpha * po[u] : xv[u]);
      st(pnew + i0, li, run ? rv[u] + beta * po[u] : po[u]);
    }
  }
}

template <typename RP, bool WIDE>
__global__ __launch_bounds__(kIterBlock) __attribute__((amdgpu_waves_per_eu(kWavesPerEu)))
void k_cg_product(const Ctx* __restrict__ c) {
  extern __shared__ double lds_dyn[];
  __shared__ double red[kWaves];
  const int64_t s = blockIdx.y;
  const Scal* sc = scal_of(c, s);
  if (sc->state_a != ST_RUNNING) return;
  const int64_t k = sc->kr, n = c->n;
  const int G = c->grid, cap = c->wave_cap;
  const RP* rowptr = static_cast<const RP*>(c->rowptr);
  const int32_t* col = c->col;
  const double* vals = c->vals + s * c->nnz;
  const SLA_GLOBAL double* p = gmem(c->p[k & 1] + s * n);
  SLA_GLOBAL double* q = gmem(c->q + s * n);
  SLA_GLOBAL double* part = gmem(c->part + s * kPartSets * G);
  double* lv;
  int32_t* lc;
  wave_areas(lds_dyn, cap, lv, lc);
  const Gather<false, WIDE> g{p, nullptr, 0.0};
  const TileWalk wk = wave_walk(c->tiles, G, blockIdx.x, kWaves, wave_index());
  const uint32_t lane = lane_id();
  double pq = 0.0;
  // each tile's index data is loaded one tile ahead
  TileIndex<RP> ix{};
  if (wk.first < wk.end)
    ix = tile_index<0, RP>(rowptr, nullptr, n, wk.first * kTileRows,
                           tile_lane(wk.first * kTileRows, n, lane));
  for (int64_t t = wk.first; t < wk.end; t += wk.stride) {
    const int64_t r0 = t * kTileRows;
    const bool own = r0 + lane < n;
    const uint32_t lr = tile_lane(r0, n, lane);
    const TileIndex<RP> cur = ix;
    const int64_t tn = t + wk.stride;
    const int64_t tp = tn < wk.end ? tn : t;  // unconditional load (see k_cg_spmv_lines)
    ix = tile_index<0, RP>(rowptr, nullptr, n, tp * kTileRows, tile_lane(tp * kTileRows, n, lane));
    const double po = ld(p + r0, lr);
    const double acc = wave_tile_row<RP>(col, vals, cur, cap, lv, lc, g);
    st(q + r0, lr, acc);
    const double pq1 = pq + po * acc;
    pq = own ? pq1 : pq;
  }
  pq = block_sum_once<kIterBlock>(pq, red);
  if (threadIdx.x == 0) part[(2 + (k & 1)) * G + blockIdx.x] = pq;
}

// ---------------------------------------------------------------------------
// Small systems: one workgroup per system, the whole CG loop in one launch
// ---------------------------------------------------------------------------
// For a system of at most kOneGroupMaxN unknowns (banded, or with 64-row
// tiles of at most kWaveCap slots each), the two-kernel iteration is bound
// by launch gaps and by every workgroup summing partials.  Here one workgroup
// owns a system and iterates with workgroup barriers only (no cross-workgroup
// signal exists), with nothing in memory but LDS.  With NT threads (256 or
// 512 by size, one_group_block) of W = NT / 64 waves:
//   * thread t owns rows t + j * NT (j < R, R = 1, 2 or 4) and keeps their
//     r, x, p, s = A p (and the Jacobi diagonal) in registers;
//   * z = r (Jacobi: r / d) is published in LDS and every SpMV gathers it
//     there;
//   * banded rows: each thread holds its rows' values by band offset, loaded
//     once, and adds value x p[i + off] in ascending offset order;
//   * plain CSR rows: wave w owns tiles w + j * W; lane l holds the values
//     and columns of slots l, l + 64, ... of each of its tiles, loaded once;
//     the SpMV stores the products in the wave's LDS area and each lane adds
//     its own row's products in slot order.
// Both add a row's products in ascending column order (the bits of the
// sequential row sum).
// The iteration is CG in the single-reduction form described at the resident
// grid loop (k_cg_grid), preconditioned: w_k = A z_k, one block sum of r.r,
// z.w and r.z, p_k.A p_k = z_k.w_k - beta_k rz_k / alpha_{k-1}, p_k = z_k +
// beta_k p_{k-1}, s_k = w_k + beta_k s_{k-1}: one barrier fewer per
// iteration than the two sums of the Hestenes-Stiefel form.  Stopping rule,
// statuses and history as the two-kernel loop; results equal to it in exact
// arithmetic, differing by rounding.

// Two sums over a workgroup of W waves at once, fixed order, results in every
// thread.
template <int W = kWaves>
__device__ __forceinline__ void block_sum2(double& u, double& v, double* lds) {
  u = wave_sum(u);
  v = wave_sum(v);
  if ((threadIdx.x & (kWave - 1)) == 0) {
    lds[threadIdx.x / kWave] = u;
    lds[W + threadIdx.x / kWave] = v;
  }
  __syncthreads();
  double a = 0.0, b = 0.0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    a = a + lds[w];
    b = b + lds[W + w];
  }
  __syncthreads();
  u = a;
  v = b;
}

// K sums without the closing barrier, for a loop whose next use of `lds`
// ([K][W] doubles) comes after another barrier, by which every thread has
// read it.
template <int W, int K>
__device__ __forceinline__ void block_sums_open(double (&v)[K], double* lds) {
#pragma unroll
  for (int k = 0; k < K; ++k) v[k] = wave_sum(v[k]);
  if ((threadIdx.x & (kWave - 1)) == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) lds[k * W + threadIdx.x / kWave] = v[k];
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    double a = 0.0;
#pragma unroll
    for (int w = 0; w < W; ++w) a = a + lds[k * W + w];
    v[k] = a;
  }
}

// Threads per workgroup of the small-system kernel: 256 up to 256 unknowns
// (and up to 512 for banded rows, two rows per thread), 512 above, with up
// to four rows per thread.  Fewer waves meet at every barrier and sum fewer
// partials; the staged CSR rows prefer one row per thread at 257-512
// unknowns.  Per iteration, Poisson (banded rows, the same run): 484
// unknowns 1.29 -> 1.10 us with 256 threads instead of 512, 1024 unknowns
// 1.42 us with 512 (1.52 with 256 and four rows each), 2025 unknowns 2.40 ->
// 1.91 us with 512 and four rows each instead of 1024 and two.
int one_group_block(int64_t n, bool band) {
  return n <= 256 || (band && n <= 512) ? 256 : 512;
}

// Rows per thread of the small-system kernel: 1, 2 or 4.
int one_group_rows_per_thread(int64_t n, bool band) {
  const int64_t nt = one_group_block(n, band);
  return n <= nt ? 1 : (n <= 2 * nt ? 2 : 4);
}

// LDS of the small-system kernel: p [n rounded up to the workgroup] and, for
// plain CSR rows, one product area of kWaveCap doubles per wave.
size_t one_group_lds_bytes(int64_t n, bool band) {
  const int64_t nt = one_group_block(n, band);
  const int64_t rows = (n + nt - 1) / nt * nt;
  return size_t(rows + (band ? 0 : (nt / kWave) * kWaveCap)) * sizeof(double);
}

// BAND: a banded pattern (the context's mask and offsets).  Each thread then
// holds its rows' values by band offset and adds value x p[i + off] straight
// from the LDS copy of p in ascending offset (= column) order, which is the
// slot order the staged CSR rows are summed in: the same bits without the
// product area and its two wave barriers per tile.
//
// The context comes by value (no copy to the device before the launch);
// the systems' records `scal` are in device memory, read back after the
// solve.  gate (or nullptr): a device flag set when the adjoint's values are
// not symmetric; then every system is refused (status SLA_ERR_NOT_SYMMETRIC,
// no iteration) and x is not touched.
template <typename RP, int R, bool JAC, int NT, bool BAND>
__global__ __launch_bounds__(NT) void k_cg_onegroup(const Ctx cv, Scal* __restrict__ scal,
                                                            double tol, int64_t maxit,
                                                            int use_x0, const int* gate) {
  constexpr int W = NT / kWave;
  extern __shared__ double lds_dyn[];
  __shared__ double red[2 * W];
  __shared__ double red3[3 * W];  // the loop's sums
  const int64_t s = blockIdx.x;
  const int64_t n = cv.n, nnz = cv.nnz;
  const int64_t npad = (n + NT - 1) / NT * NT;
  double* pl = lds_dyn;                                         // p, or x0 at set-up
  double* prod = lds_dyn + npad + int64_t(wave_index()) * kWaveCap;  // this wave's products
  const SLA_GLOBAL RP* rowptr = gmem(static_cast<const RP*>(cv.rowptr));
  const SLA_GLOBAL int32_t* col = gmem(cv.col);
  const SLA_GLOBAL double* vals = gmem(cv.vals + s * nnz);
  const SLA_GLOBAL double* b = gmem(cv.b + s * n);
  SLA_GLOBAL double* x = gmem(cv.x + s * n);
  SLA_GLOBAL double* hist = cv.hist != nullptr ? gmem(cv.hist + s * cv.hist_cap * 3) : nullptr;
  const int64_t hist_cap = cv.hist_cap;
  const int t = threadIdx.x;
  const int lane = int(lane_id());
  if (gate != nullptr && *gate != 0) {  // uniform
    if (t == 0) {
      Scal* sc = scal + s;
      sc->bb = 0.0;
      sc->stop = 0.0;
      sc->maxit = maxit;
      sc->it = 0;
      sc->rr_final = 0.0;
      sc->state_a = SLA_ERR_NOT_SYMMETRIC;
      sc->state_r = SLA_ERR_NOT_SYMMETRIC;
    }
    return;
  }
  // this thread's rows and tiles; the held slots of each tile (CSR), or the
  // rows' values by band offset (BAND)
  int64_t row[R];
  int rlen[R], ra[R], re[R];   // tile length; the row's slots [ra, re) in the tile
  double hv[R][kStageLoads];
  int32_t hc[R][kStageLoads];
  double bv[R][kMaxBand];
  uint32_t bm[R];              // the row's bits among the band's offsets
  int32_t boff[kMaxBand];      // the offsets (uniform)
#pragma unroll
  for (int o = 0; o < kMaxBand; ++o) boff[o] = BAND ? cv.band.off[o] : 0;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int64_t r0 = (int64_t(j) * W + wave_index()) * kTileRows;
    row[j] = r0 + lane;
    rlen[j] = ra[j] = re[j] = 0;
    if constexpr (BAND) {
      const int cnt = cv.band.count;
      bm[j] = 0;
      int64_t k = 0;
      if (row[j] < n) {
        bm[j] = uint32_t(cv.mask[row[j]]) & ((1u << cnt) - 1u);
        k = int64_t(rowptr[row[j]]);
      }
#pragma unroll
      for (int o = 0; o < kMaxBand; ++o) {
        const bool use = (bm[j] >> o) & 1u;
        bv[j][o] = use ? vals[k] : 0.0;
        k += use ? 1 : 0;
      }
    } else if (r0 < n) {
      const int64_t last = (r0 + kTileRows < n ? r0 + kTileRows : n);
      const int64_t s0 = int64_t(rowptr[r0]);
      rlen[j] = int(int64_t(rowptr[last]) - s0);
      if (row[j] < n) {
        ra[j] = int(int64_t(rowptr[row[j]]) - s0);
        re[j] = int(int64_t(rowptr[row[j] + 1]) - s0);
      }
#pragma unroll
      for (int m = 0; m < kStageLoads; ++m) {
        const int k = lane + m * kWave;
        const int kc = k < rlen[j] ? k : (rlen[j] > 0 ? rlen[j] - 1 : 0);
        hv[j][m] = rlen[j] > 0 ? vals[s0 + kc] : 0.0;
        hc[j][m] = rlen[j] > 0 ? col[s0 + kc] : 0;
      }
    }
  }
  // q = A v for this thread's rows, v published in pl (every wave works on
  // its own tiles; the caller has made pl visible)
  auto spmv = [&](double (&q)[R]) {
#pragma unroll
    for (int j = 0; j < R; ++j) {
      q[j] = 0.0;
      if constexpr (BAND) {
        double g[kMaxBand];
#pragma unroll
        for (int o = 0; o < kMaxBand; ++o)
          g[o] = pl[((bm[j] >> o) & 1u) ? int32_t(row[j]) + boff[o] : 0];
        double acc = 0.0;
#pragma unroll
        for (int o = 0; o < kMaxBand; ++o) {
          const double sum = acc + bv[j][o] * g[o];
          acc = ((bm[j] >> o) & 1u) ? sum : acc;
        }
        q[j] = acc;
      } else if (rlen[j] > 0) {  // wave-uniform
#pragma unroll
        for (int m = 0; m < kStageLoads; ++m) {
          const int k = lane + m * kWave;
          if (k < rlen[j]) prod[k] = hv[j][m] * pl[hc[j][m]];
        }
        wave_sync();
        // slot order, four LDS reads in flight at a time
        double acc = 0.0;
        int k = ra[j];
        for (; k + 4 <= re[j]; k += 4) {
          const double p0 = prod[k], p1 = prod[k + 1], p2 = prod[k + 2], p3 = prod[k + 3];
          acc = acc + p0;
          acc = acc + p1;
          acc = acc + p2;
          acc = acc + p3;
        }
        for (; k < re[j]; ++k) acc = acc + prod[k];
        q[j] = acc;
        wave_sync();  // the area is reused by the next tile
      }
    }
  };
  double r[R], xv[R], pv[R], dv[R], q[R];
  // r0 = b - A x0 (or b, x0 = 0); the Jacobi diagonal
  if (use_x0) {
    for (int64_t i = t; i < npad; i += NT) pl[i] = i < n ? x[i] : 0.0;
    __syncthreads();
    spmv(q);
    __syncthreads();
  }
  double bb = 0.0, rr = 0.0, rz = 0.0, bad = 0.0;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int64_t i = t + int64_t(j) * NT;
    r[j] = xv[j] = pv[j] = 0.0;
    dv[j] = 1.0;
    if (i < n) {
      const double bi = b[i];
      xv[j] = use_x0 ? x[i] : 0.0;
      r[j] = use_x0 ? bi - q[j] : bi;
      bb = bb + bi * bi;
      rr = rr + r[j] * r[j];
      if constexpr (JAC) {
        double d = 0.0;  // the stored diagonal entry (0 when the row has none)
        for (int64_t k = int64_t(rowptr[i]); k < int64_t(rowptr[i + 1]); ++k)
          if (col[k] == i) d = vals[k];
        dv[j] = d;
        bad = (d > 0.0) ? bad : 1.0;
        rz = rz + r[j] * (r[j] / d);
      }
    }
  }
  block_sum2<W>(bb, rr, red);
  if constexpr (JAC) block_sum2<W>(rz, bad, red);
  const double stop = (tol * tol) * bb;
  int32_t state = (!isfinite(bb) || !isfinite(rr) || !isfinite(rz)) ? ST_NONFINITE : ST_RUNNING;
  if (JAC && bad != 0.0) state = ST_NOT_SPD;  // a diagonal entry is not > 0
  int64_t it = 0;
  double rr_final = rr;
  double alpha = 0.0;
  double sv[R];  // s = A p
#pragma unroll
  for (int j = 0; j < R; ++j) sv[j] = 0.0;
  // single-reduction form (see the resident grid loop): w_k = A z_k, one
  // block sum of r.r, r.z and z.w, then p.Ap = z.w - beta rz / alpha_{k-1};
  // every thread holds the same scalars, so every branch below is uniform
  for (int64_t k = 0; state == ST_RUNNING; ++k) {
    // z_k = r_k (Jacobi: r_k / d) published in LDS for the gathers (the
    // last sum's barrier ended every wave's gathers of z_{k-1} and every
    // read of red3)
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const int64_t i = t + int64_t(j) * NT;
      if (i < npad) pl[i] = JAC ? r[j] / dv[j] : r[j];
    }
    __syncthreads();
    spmv(q);
    // r.r, z.w and (Jacobi) r.z
    constexpr int K = JAC ? 3 : 2;
    double g[K];
#pragma unroll
    for (int c = 0; c < K; ++c) g[c] = 0.0;
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (t + int64_t(j) * NT < n) {
        const double zj = JAC ? r[j] / dv[j] : r[j];
        g[0] = g[0] + r[j] * r[j];
        g[1] = g[1] + zj * q[j];
        if constexpr (JAC) g[2] = g[2] + r[j] * zj;
      }
    block_sums_open<W, K>(g, red3);
    const double g_rr = g[0], g_zw = g[1], g_rz = g[JAC ? 2 : 0];
    double beta = 0.0;
    if (k > 0) {
      if (!isfinite(g_rr) || !isfinite(g_rz)) {
        state = ST_NONFINITE;  // iteration k-1 did not complete
        it = k - 1;
        rr_final = rr;
        break;
      }
      beta = g_rz / rz;
      if (hist != nullptr && t == 0 && k - 1 < hist_cap) {
        hist[(k - 1) * 3 + 0] = alpha;
        hist[(k - 1) * 3 + 1] = beta;
        hist[(k - 1) * 3 + 2] = g_rr;
      }
    }
    if (g_rr <= stop || k >= maxit) {
      state = g_rr <= stop ? ST_CONVERGED : ST_MAXIT;
      it = k;
      rr_final = g_rr;
      break;
    }
    const double pq = k > 0 ? g_zw - beta * (g_rz / alpha) : g_zw;  // p_k.A p_k
    if (!isfinite(pq) || !(pq > 0.0)) {
      state = !isfinite(pq) ? ST_NONFINITE : ST_NOT_SPD;
      it = k;
      rr_final = g_rr;
      break;
    }
    alpha = g_rz / pq;
    rr = g_rr;
    rz = g_rz;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      if (t + int64_t(j) * NT < n) {
        const double zj = JAC ? r[j] / dv[j] : r[j];
        pv[j] = zj + beta * pv[j];
        sv[j] = q[j] + beta * sv[j];
        xv[j] = xv[j] + alpha * pv[j];
        r[j] = r[j] - alpha * sv[j];
      }
    }
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int64_t i = t + int64_t(j) * NT;
    if (i < n) x[i] = xv[j];
  }
  if (t == 0) {
    Scal* sc = scal + s;
    sc->bb = bb;
    sc->stop = stop;
    sc->maxit = maxit;
    sc->it = it;
    sc->rr_final = rr_final;
    sc->state_a = state;
    sc->state_r = state;
  }
}

// ---------------------------------------------------------------------------
// Mid-size banded systems: the whole CG loop in one cooperative launch, the
// system resident on chip
// ---------------------------------------------------------------------------
// A banded system of a few hundred thousand to about a million unknowns fits
// the chip's registers and LDS (256 CUs hold 128 MB of VGPRs and 40 MB of
// LDS): workgroup g of G (one per CU, all resident: cooperative launch) owns
// rows [g rw, min(n, (g + 1) rw)), rw >= H = the band's largest |offset|,
// and keeps their values by band offset, r and s in registers and A r, p and
// x in LDS for the whole solve; r is published in LDS with H halo rows on
// each side.  The matrix is read once per solve; an iteration moves only
// halo rows and partial sums between workgroups, so it is bound by the
// latency of its grid-wide sum, not by HBM.
//
// The iteration is CG in the single-reduction form of Chronopoulos and Gear:
// the SpMV takes r instead of p, u_k = A r_k, and one grid sum carries both
// gamma_k = r_k.r_k and delta_k = r_k.u_k.  Then
//   beta_k = gamma_k / gamma_{k-1},
//   p_k.A p_k = delta_k - beta_k gamma_k / alpha_{k-1}   (delta_0 at k = 0),
//   alpha_k = gamma_k / p_k.A p_k,
//   p_k = r_k + beta_k p_{k-1},  s_k = u_k + beta_k s_{k-1}   (s_k = A p_k),
//   x_{k+1} = x_k + alpha_k p_k,  r_{k+1} = r_k - alpha_k s_k.
// The middle identity expands p_k.A p_k with r_k.r_{k-1} = 0 and
// A p_{k-1} = (r_{k-1} - r_k) / alpha_{k-1}.  In exact arithmetic these are
// the iterates, scalars, stopping rule and statuses of the loop with two sums
// (Hestenes-Stiefel, the two-kernel loop); in floating
// point they differ from it by rounding.  The sum's latency is most of an
// iteration here, so one sum per iteration instead of two is what counts.
//
// Grid sums (grid_sum): each workgroup writes its partials for round R into
// slot[R & 1], every double as two 8-byte words, its high and low halves
// each beside the tag R (a word is written whole, so a reader never sees a
// half of another round), with relaxed device-scope stores (sc1: written
// through the L2 to the device-coherent level), once into each of 8
// replicas; workgroup g polls replica g % 8 (its waves share the G slots, a
// slot per lane) with device-scope loads (sc1: served from that level) until
// every tag reads R, then adds the G partials in slot order (a wave sum per
// wave, then the waves in order), so every workgroup gets the same bits.  The
// replicas spread the polls of 256 workgroups over 8 times as many memory
// lines.  No fence that writes back or invalidates a whole L2 runs in the
// loop: on MI355X a release fence (an L2 write-back walk) costs about 2 us per
// sum, and acquire polls 8.7-10.5 us per round against about 3 us for these.
// A poll limit bounds every wait: past it the workgroup sets the shared
// failure flag, which every other poll reads, and all leave the loop
// (ST_GRID_TIMEOUT).
//
// Halo: the neighbours' rows of r are formed locally, by the same operations
// on the same operands as their owners', hence the owners' bits:
// s_k = u_k + beta_k s_{k-1} and r_{k+1} = r_k - alpha_k s_k from the
// neighbours' boundary rows of u_k (r_0's boundary rows are exchanged once).
// Each workgroup publishes its boundary rows of u_k during the sum, after its
// first barrier, into halo[k & 1], tagged as the slots are with the round of
// that sum; a reader loads them once the sum is complete and loads again
// while a tag is not that round (the writer issued them alongside its slot
// tags, so by the time every tag has been seen they have nearly always
// landed).  Nothing waits for the stores and no fence runs.
// Double buffering by parity suffices: a buffer is written again two
// iterations later, after a sum that needs every reader's partials, which
// each reader posts only after reading it.  Slots and halo words are cleared
// before every launch, so no tag of an earlier launch is read.
constexpr int kGridThreads = 512;   // threads per workgroup of the grid loop
constexpr int kGridVals = 2;        // values one grid sum carries at most
constexpr int kGridHaloPT = 4;      // halo rows per thread: 2 H <= 4 * 512

struct GridSync {
  // [2][reps][kGridVals][2][G] tagged words (round parity, replica, value,
  // high/low half, workgroup), a replica every rep_words words
  uint64_t* slot;
  // [2][G][2][2 H] tagged words (parity, workgroup, high/low half, entry:
  // first H rows, then last H rows), so a store or load of a wave is
  // contiguous
  uint64_t* halo;
  int* fail;           // set when a wait passed its poll limit
  int64_t rw;          // rows per workgroup
  int32_t H;           // halo rows on each side
  int32_t reps;        // replicas of the slots: workgroup g polls replica g % reps
  int64_t rep_words;   // words from one replica to the next
  int64_t poll_limit;  // polls per wait before giving up
};

__device__ __forceinline__ void dev_put(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t dev_get(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void dev_put(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int dev_get(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// v as two words at hi and lo: its high and low 32 bits each beside the tag
__device__ __forceinline__ void put_tagged(uint64_t* hi, uint64_t* lo, double v, uint32_t tag) {
  const uint64_t bits = uint64_t(__double_as_longlong(v));
  dev_put(hi, (bits & 0xffffffff00000000ull) | tag);
  dev_put(lo, (bits << 32) | tag);
}
__device__ __forceinline__ bool has_tag(uint64_t hi, uint64_t lo, uint32_t tag) {
  return uint32_t(hi) == tag && uint32_t(lo) == tag;
}
__device__ __forceinline__ double untag(uint64_t hi, uint64_t lo) {
  return __longlong_as_double((long long)((hi & 0xffffffff00000000ull) | (lo >> 32)));
}

// Slots, halo words and the failure flag cleared before a launch (a kernel:
// a caller's stream may be captured).
__global__ void k_grid_clear(uint64_t* __restrict__ slot, int64_t slot_words,
                             uint64_t* __restrict__ halo, int64_t halo_words,
                             int* __restrict__ fail) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < slot_words) slot[i] = 0;
  else if (i < slot_words + halo_words) halo[i - slot_words] = 0;
  if (i == 0) *fail = 0;
}

// RPT rows per thread (rows t + j * 512 of the block), NB band offsets at
// most.  gate: as in k_cg_onegroup.  Indices inside a block are 32-bit (a
// block and its halo hold fewer than 2^13 rows).
template <typename RP, int RPT, int NB>
__global__ __launch_bounds__(kGridThreads) void k_cg_grid(const Ctx cv, Scal* __restrict__ scal,
                                                          const GridSync gs, double tol,
                                                          int64_t maxit, int use_x0,
                                                          const int* gate) {
  constexpr int NT = kGridThreads, W = NT / kWave;
  extern __shared__ double lds_dyn[];
  __shared__ double red[kGridVals * W], red2[kGridVals * W];
  __shared__ int lfail, hfail;
  const int t = threadIdx.x;
  const int lane = int(lane_id()), w = wave_index();
  const int g = int(blockIdx.x), G = int(gridDim.x);
  const int64_t n = cv.n;
  const int H = gs.H;
  const int rw = int(gs.rw);
  const int64_t r0 = int64_t(g) * gs.rw;
  const int nloc = int((r0 + gs.rw < n ? r0 + gs.rw : n) - r0);
  // r of row r0 + l at rl[H + l], the halo rows below and above, a spare
  // slot; then u = A r, p and x of the rows, each with a spare slot at index
  // rw for the rows past the block
  double* rl = lds_dyn;
  double* ul = rl + (rw + 2 * H + 1);
  double* pl = ul + (rw + 1);
  double* xl = pl + (rw + 1);
  auto x_idx = [&](int l) -> int { return l < nloc ? l : rw; };
  // the block's slices of the arrays (bases uniform, offsets 32-bit)
  const SLA_GLOBAL RP* rowptr = gmem(static_cast<const RP*>(cv.rowptr) + r0);
  const SLA_GLOBAL uint8_t* mask = gmem(cv.mask + r0);
  const SLA_GLOBAL double* vals = gmem(cv.vals);
  const SLA_GLOBAL double* b = gmem(cv.b + r0);
  SLA_GLOBAL double* x = gmem(cv.x + r0);
  SLA_GLOBAL double* hist = cv.hist != nullptr ? gmem(cv.hist) : nullptr;
  const int64_t hist_cap = cv.hist_cap;
  if (gate != nullptr && *gate != 0) {  // uniform
    if (g == 0 && t == 0) {
      scal->bb = 0.0;
      scal->stop = 0.0;
      scal->maxit = maxit;
      scal->it = 0;
      scal->rr_final = 0.0;
      scal->state_a = SLA_ERR_NOT_SYMMETRIC;
      scal->state_r = SLA_ERR_NOT_SYMMETRIC;
    }
    return;
  }
  // this thread's rows: values by band offset, the rows' bits packed a byte
  // per row (NB <= 8)
  double bv[RPT][NB];
  uint64_t bmp = 0;
  int32_t boff[NB];
#pragma unroll
  for (int o = 0; o < NB; ++o) boff[o] = cv.band.off[o];
  const int cnt = cv.band.count;
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int l = t + j * NT;
    uint32_t bm = 0;
    int64_t k = 0;
    if (l < nloc) {
      bm = uint32_t(mask[l]) & ((1u << cnt) - 1u);
      k = int64_t(rowptr[l]);
    }
    bmp |= uint64_t(bm) << (8 * j);
#pragma unroll
    for (int o = 0; o < NB; ++o) {
      const bool use = (bm >> o) & 1u;
      bv[j][o] = use ? vals[k] : 0.0;
      k += use ? 1 : 0;
    }
    // one row's loads at a time (set-up only): all rows' 64-bit addresses at
    // once would not leave the registers the loop keeps
    __builtin_amdgcn_sched_barrier(0);
  }
  // this thread's halo entries e = t + u * 512 < 2 H: e < H the row
  // r0 - H + e (the lower neighbour's last rows), else r0 + nloc + e - H (the
  // upper neighbour's first rows); LDS index e, or nloc + e.  hsrc: the
  // high word's index in a halo buffer of one parity (the low word 2 H
  // further), or -1 (no such row).
  int32_t hsrc[kGridHaloPT];
#pragma unroll
  for (int u = 0; u < kGridHaloPT; ++u) {
    const int e = t + u * NT;
    hsrc[u] = -1;
    if (e < 2 * H) {
      const bool low = e < H;
      const int64_t row = low ? r0 - H + e : r0 + nloc + (e - H);
      if (row >= 0 && row < n)
        hsrc[u] = low ? (g - 1) * 4 * H + H + e : (g + 1) * 4 * H + (e - H);
    }
  }
  auto hidx = [&](int u) -> int { return t + u * NT < H ? t + u * NT : nloc + t + u * NT; };
  // the same entries as this workgroup's published boundary rows: e < H the
  // row l = e, else l = nloc - H + (e - H); psrc: the row's index in rl, or -1
  int32_t psrc[kGridHaloPT];
#pragma unroll
  for (int u = 0; u < kGridHaloPT; ++u) {
    const int e = t + u * NT;
    const int l = e < H ? e : nloc - H + (e - H);
    psrc[u] = (e < 2 * H && l >= 0 && l < nloc) ? H + l : -1;
  }
  // index of row l of the block in rl; rows past the block (lanes without a
  // row, whose values are all zero) store to one spare slot past the halo
  const int spare = nloc + 2 * H;
  auto own_idx = [&](int l) -> int { return l < nloc ? H + l : spare; };
  for (int i = t; i < nloc + 2 * H; i += NT) rl[i] = 0.0;
  if (t == 0) lfail = hfail = 0;
  __syncthreads();
  // q = A v for this thread's rows, v published in rl (rows and halo)
  auto spmv = [&](double (&q)[RPT]) {
    // an opaque zero: the gather addresses and the slot masks are formed
    // here at every call, not hoisted out of the CG loop into registers (40
    // lane masks would take 80 SGPRs) that the rows' values need
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int li = own_idx(t + j * NT) + z;  // (rows past the block: m = 0)
      const uint32_t m = uint32_t(bmp >> (8 * j)) + uint32_t(z);
      double gv[NB];
#pragma unroll
      for (int o = 0; o < NB; ++o) gv[o] = rl[((m >> o) & 1u) ? li + boff[o] : li];
      double acc = 0.0;
#pragma unroll
      for (int o = 0; o < NB; ++o) {
        const double sum = acc + bv[j][o] * gv[o];
        acc = ((m >> o) & 1u) ? sum : acc;
      }
      q[j] = acc;
    }
  };
  // this workgroup's entries in halo buffer `par` (first H rows for g - 1,
  // last H rows for g + 1)
  auto own_halo = [&](int par) -> uint64_t* {
    return gs.halo + (int64_t(par) * G + g) * (4 * int64_t(H));
  };
  // boundary rows of r_0 into halo buffer `par`, staged in rl's rows (the
  // halo of rl is left alone)
  auto publish_r = [&](int par, uint32_t tag, const double (&r)[RPT]) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) rl[own_idx(t + j * NT)] = r[j];
    __syncthreads();
    uint64_t* hb = own_halo(par);
#pragma unroll
    for (int u = 0; u < kGridHaloPT; ++u)
      if (psrc[u] >= 0) {
        const uint32_t e = uint32_t(t + u * NT);
        put_tagged(hb + e, hb + 2 * H + e, rl[psrc[u]], tag);
      }
  };
  // u_k of the rows staged in ul (rows past the block at ul[rw]) before the
  // sum's first barrier; its boundary rows go out from there after that
  // barrier: no row tests on the registers
  auto stage_u = [&](const double (&q)[RPT]) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) ul[x_idx(t + j * NT)] = q[j];
  };
  auto publish_u = [&](int par, uint32_t tag) {
    uint64_t* hb = own_halo(par);
#pragma unroll
    for (int u = 0; u < kGridHaloPT; ++u)
      if (psrc[u] >= 0) {
        const uint32_t e = uint32_t(t + u * NT);
        put_tagged(hb + e, hb + 2 * H + e, ul[psrc[u] - H], tag);
      }
  };
  // the neighbours' words of this thread's halo entries in buffer `par`
  // (entries without a row read as tagged zeros)
  auto halo_load = [&](int par, uint32_t tag, uint64_t (&hw)[kGridHaloPT][2]) {
    const uint64_t* hb = gs.halo + int64_t(par) * G * (4 * int64_t(H));
#pragma unroll
    for (int u = 0; u < kGridHaloPT; ++u) {
      hw[u][0] = hw[u][1] = tag;
      if (hsrc[u] >= 0) {
        hw[u][0] = dev_get(hb + uint32_t(hsrc[u]));
        hw[u][1] = dev_get(hb + uint32_t(hsrc[u]) + 2 * H);
      }
    }
  };
  // the halo values once every word carries `tag`, loading again meanwhile;
  // zeros and hfail set when a wait timed out (here or in another workgroup)
  auto halo_take = [&](int par, uint32_t tag, uint64_t (&hw)[kGridHaloPT][2],
                       double (&v)[kGridHaloPT]) {
    for (int64_t polls = 0;; ++polls) {
      bool ok = true;
#pragma unroll
      for (int u = 0; u < kGridHaloPT; ++u) ok = ok && has_tag(hw[u][0], hw[u][1], tag);
      if (__all(ok)) break;
      const int f = (polls & 15) == 15 ? __builtin_amdgcn_readfirstlane(dev_get(gs.fail)) : 0;
      if (f != 0 || polls >= gs.poll_limit) {
        if (lane == 0) {
          if (f == 0) dev_put(gs.fail, 1);
          hfail = 1;
        }
#pragma unroll
        for (int u = 0; u < kGridHaloPT; ++u) hw[u][0] = hw[u][1] = 0;
        break;
      }
      halo_load(par, tag, hw);
    }
#pragma unroll
    for (int u = 0; u < kGridHaloPT; ++u) v[u] = hsrc[u] >= 0 ? untag(hw[u][0], hw[u][1]) : 0.0;
  };
  // sum of K values over the grid, in place in every thread; false when a
  // wait timed out (here or in another workgroup).  after_barrier runs in
  // every thread once the partials are in red (wave 0: after posting its tag).
  uint32_t round = 0;
  auto no_hook = [] {};
  auto grid_sum = [&](auto kc, double* v, auto after_barrier) -> bool {
    constexpr int K = decltype(kc)::value;
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = wave_sum(v[k]);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < K; ++k) red[k * W + w] = v[k];
    }
    __syncthreads();
    ++round;
    uint64_t* sl = gs.slot + int64_t(round & 1) * gs.reps * gs.rep_words;
    // lane i < reps of wave 0 posts the partials into replica i: value k's
    // halves at words (2 k) G + g and (2 k + 1) G + g, so a poll's lanes read
    // consecutive words
    if (w == 0 && lane < gs.reps) {
      uint64_t* mine = sl + lane * gs.rep_words + g;
#pragma unroll
      for (int k = 0; k < K; ++k) {
        double a = 0.0;
        for (int ww = 0; ww < W; ++ww) a = a + red[k * W + ww];
        const uint64_t bits = uint64_t(__double_as_longlong(a));
        dev_put(mine + (2 * k) * G, (bits & 0xffffffff00000000ull) | round);
        dev_put(mine + (2 * k + 1) * G, (bits << 32) | round);
      }
    }
    after_barrier();
    // every wave polls its share of the slots, lane l the slot w S + l (a
    // few loads per lane, all the workgroup's waves at once, where one wave
    // alone took 4 slots per lane)
    sl += (g % gs.reps) * gs.rep_words;
    const int S = (G + W - 1) / W;  // (<= 64: G <= 512)
    const int gg = w * S + lane;
    const bool mine = lane < S && gg < G;
    uint64_t wa[K][2];
    auto poll = [&](uint64_t (&wd)[K][2]) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        wd[k][0] = wd[k][1] = round;  // (no slot: reads as tagged zero)
        if (mine) {
          wd[k][0] = dev_get(sl + (2 * k) * G + gg);
          wd[k][1] = dev_get(sl + (2 * k + 1) * G + gg);
        }
      }
    };
    auto ready = [&](const uint64_t (&wd)[K][2]) {
      bool ok = true;
#pragma unroll
      for (int k = 0; k < K; ++k) ok = ok && has_tag(wd[k][0], wd[k][1], round);
      return __all(ok);
    };
    double s[K];
    auto take = [&](const uint64_t (&wd)[K][2]) {
#pragma unroll
      for (int k = 0; k < K; ++k) s[k] = mine ? untag(wd[k][0], wd[k][1]) : 0.0;
    };
    bool failed = false;
    poll(wa);
    for (int64_t polls = 0;; ++polls) {
      if (ready(wa)) {
        take(wa);
        break;
      }
      poll(wa);
      const int f = (polls & 15) == 15 ? __builtin_amdgcn_readfirstlane(dev_get(gs.fail)) : 0;
      if (f != 0 || polls >= gs.poll_limit) {
        if (f == 0 && lane == 0) dev_put(gs.fail, 1);
        failed = true;
#pragma unroll
        for (int k = 0; k < K; ++k) s[k] = 0.0;
        break;
      }
    }
    // the waves' sums in wave order: the same bits in every workgroup
#pragma unroll
    for (int k = 0; k < K; ++k) s[k] = wave_sum(s[k]);
    if (lane == 0) {
#pragma unroll
      for (int k = 0; k < K; ++k) red2[k * W + w] = s[k];
      if (failed) lfail = 1;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < K; ++k) {
      double a = 0.0;
      for (int ww = 0; ww < W; ++ww) a = a + red2[k * W + ww];
      v[k] = a;
    }
    return lfail == 0;
  };
  using Two = std::integral_constant<int, 2>;

  // (the halo rows of r live in rl, whose entries hidx(u) only this thread
  // reads and writes; rh holds r_0's while they arrive)
  double r[RPT], s[RPT], q[RPT], rh[kGridHaloPT], sh[kGridHaloPT];
  uint64_t hw[kGridHaloPT][2];
  // r0 = b - A x0 (or b, x0 = 0): x0 of the rows and of the halo from x,
  // which no workgroup writes before every one has passed the first grid sum
  if (use_x0) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int l = t + j * NT;
      rl[own_idx(l)] = l < nloc ? x[l] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < kGridHaloPT; ++u)
      if (hsrc[u] >= 0) {
        const int e = t + u * NT;
        rl[hidx(u)] = x[e < H ? e - H : nloc + (e - H)];
      }
    __syncthreads();
    spmv(q);
    __syncthreads();
  }
  double sums[2] = {0.0, 0.0};  // b.b, r.r
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int l = t + j * NT;
    const int xi = x_idx(l);
    r[j] = s[j] = 0.0;
    pl[xi] = 0.0;
    xl[xi] = l < nloc && use_x0 ? x[l] : 0.0;
    if (l < nloc) {
      const double bi = b[l];
      r[j] = use_x0 ? bi - q[j] : bi;
      sums[0] = sums[0] + bi * bi;
      sums[1] = sums[1] + r[j] * r[j];
    }
  }
#pragma unroll
  for (int u = 0; u < kGridHaloPT; ++u) sh[u] = 0.0;
  // r_0's boundary rows into buffer 1 (iteration 0 writes buffer 0 while a
  // neighbour may still be reading them); the halo of rl takes them after the
  // sum (entries without a row keep their zeros)
  uint32_t tag = round + 1;
  publish_r(1, tag, r);
  const bool ok0 = grid_sum(Two{}, sums, no_hook);
  halo_load(1, tag, hw);
  halo_take(1, tag, hw, rh);
#pragma unroll
  for (int u = 0; u < kGridHaloPT; ++u)
    if (hsrc[u] >= 0) rl[hidx(u)] = rh[u];
  __syncthreads();
  const double bb = sums[0];
  double rr = sums[1];
  const double stop = (tol * tol) * bb;
  int32_t state = (!isfinite(bb) || !isfinite(rr)) ? ST_NONFINITE : ST_RUNNING;
  if (!ok0 || hfail != 0) state = ST_GRID_TIMEOUT;
  int64_t it = 0;
  double rr_final = rr;
  double alpha = 0.0;
  // every thread holds the same scalars, so every branch below is uniform
  for (int64_t k = 0; state == ST_RUNNING; ++k) {
    // rl holds r_k on the rows and the halo
    spmv(q);
    stage_u(q);
    // rows past the block hold zeros throughout (values, r, s, u, p, x), so
    // they add +0.0 to the sums and leave their bits alone: no row test here
    double gd[2] = {0.0, 0.0};  // r.r, r.u
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      gd[0] = gd[0] + r[j] * r[j];
      gd[1] = gd[1] + r[j] * q[j];
    }
    const int par = int(k & 1);
    tag = round + 1;
    // (the sum's barriers also end every wave's gathers of r_k)
    if (!grid_sum(Two{}, gd, [&] { publish_u(par, tag); })) {
      state = ST_GRID_TIMEOUT;
      it = k;
      rr_final = rr;
      break;
    }
    const double gk = gd[0], dk = gd[1];
    double beta = 0.0;
    if (k > 0) {
      if (!isfinite(gk)) {
        state = ST_NONFINITE;  // iteration k-1 did not complete
        it = k - 1;
        rr_final = rr;
        break;
      }
      beta = gk / rr;
      if (hist != nullptr && g == 0 && t == 0 && k - 1 < hist_cap) {
        hist[(k - 1) * 3 + 0] = alpha;
        hist[(k - 1) * 3 + 1] = beta;
        hist[(k - 1) * 3 + 2] = gk;
      }
    }
    if (gk <= stop || k >= maxit) {
      state = gk <= stop ? ST_CONVERGED : ST_MAXIT;
      it = k;
      rr_final = gk;
      break;
    }
    const double pap = k > 0 ? dk - beta * (gk / alpha) : dk;  // p_k.A p_k
    if (!isfinite(pap) || !(pap > 0.0)) {
      state = !isfinite(pap) ? ST_NONFINITE : ST_NOT_SPD;
      it = k;
      rr_final = gk;
      break;
    }
    alpha = gk / pap;
    rr = gk;
    // the neighbours' u_k: loaded before the rows' updates, taken after
    halo_load(par, tag, hw);
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int l = t + j * NT;
      const int xi = x_idx(l);
      s[j] = ul[xi] + beta * s[j];
      const double pj = r[j] + beta * pl[xi];
      pl[xi] = pj;
      xl[xi] = xl[xi] + alpha * pj;
      r[j] = r[j] - alpha * s[j];
      rl[own_idx(l)] = r[j];
    }
    double uh[kGridHaloPT];
    halo_take(par, tag, hw, uh);
#pragma unroll
    for (int u = 0; u < kGridHaloPT; ++u) {
      sh[u] = uh[u] + beta * sh[u];
      if (hsrc[u] >= 0) rl[hidx(u)] = rl[hidx(u)] - alpha * sh[u];
    }
    __syncthreads();
    if (hfail != 0) {
      state = ST_GRID_TIMEOUT;
      it = k + 1;
      rr_final = rr;
      break;
    }
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int l = t + j * NT;
    if (l < nloc) x[l] = xl[l];
  }
  if (g == 0 && t == 0) {
    scal->bb = bb;
    scal->stop = stop;
    scal->maxit = maxit;
    scal->it = it;
    scal->rr_final = rr_final;
    scal->state_a = state;
    scal->state_r = state;
  }
}

// Residual step k (see the file comment).  JAC: Jacobi preconditioning, so
// alpha = r.z / p.Ap, and the step also writes z = r / d and the r.z partials.
// NT threads per workgroup (residual_block).
template <bool JAC, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(2 * (NT / kWave) / 4)))
void k_cg_residual(const Ctx* __restrict__ c) {
  constexpr int W = NT / kWave;
  __shared__ double red[3 * W];  // p.Ap sum, r.r and r.z partials
  const int64_t s = blockIdx.y;
  // the context fields and the system's record (step index, state, r.r and
  // r.z by parity: an index from k would wait for k) in one round trip
  const CtxWords cw = load_ctx(c, s);
  const int64_t n = SLA_CTX(cw, int64_t, n), tiles = SLA_CTX(cw, int64_t, tiles);
  const int G = SLA_CTX(cw, int32_t, grid);
  SLA_GLOBAL double* part = gmem(SLA_CTX(cw, double*, part) + s * kPartSets * G);
  SLA_GLOBAL double* r = gmem(SLA_CTX(cw, double*, r) + s * n);
  const SLA_GLOBAL double* q = gmem(SLA_CTX(cw, double*, q) + s * n);
  const SLA_GLOBAL double* dg = gmem(SLA_CTX(cw, const double*, diag) + s * n);
  SLA_GLOBAL double* z = gmem(SLA_CTX(cw, double*, z) + s * n);
  int* const n_running = SLA_CTX(cw, int*, n_running);
  Scal* sc = scal_of(c, s);
  const bool lead = blockIdx.x == 0 && threadIdx.x == 0;
  const SLA_GLOBAL Scal* scg = gmem(static_cast<const Scal*>(sc));
  const int64_t k = SLA_REC(cw, int64_t, kr);
  const int32_t st_in = SLA_REC(cw, int32_t, state_a);
  const double rr0 = SLA_REC(cw, double, rr[0]), rr1 = SLA_REC(cw, double, rr[1]);
  const double rz0 = SLA_REC(cw, double, rz[0]), rz1 = SLA_REC(cw, double, rz[1]);
  const double rr = (k & 1) ? rr1 : rr0;
  const double num = JAC ? ((k & 1) ? rz1 : rz0) : rr;
  const uint32_t lane = lane_id();
  // blocks of kStreamTiles consecutive tiles (a wave's loads fall in a few
  // DRAM pages), walked like single tiles: each XCD owns a contiguous range
  // of blocks; a block is loaded in rounds of U tiles, all loads of a round
  // first (two tiles with Jacobi: the divisions need the registers); the
  // r.r (and r.z) terms are added in tile order, the same order with and
  // without Jacobi
  constexpr int B = kStreamTiles;
  constexpr int U = JAC ? 2 : kStreamTiles;
  static_assert(B % U == 0, "whole rounds per block");
  const TileWalk wk = wave_walk((tiles + B - 1) / B, G, blockIdx.x, W, wave_index());
  double rv[U], qv[U], dv[U];
  // unconditional loads: tiles past the matrix read the round's first tile
  // and lanes past the last row read that row (their values are not used,
  // or give the same stores; a conditional load would make the compiler
  // keep the old register value, which waits for every older load)
  auto load_round = [&](int64_t t0) {
    const int64_t tf = t0 < tiles ? t0 : tiles - 1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = t0 + u < tiles ? t0 + u : tf;
      const int64_t i0 = t * kTileRows;
      const uint32_t li = i0 + lane < n ? lane : uint32_t(n - 1 - i0);
      rv[u] = ld(r + i0, li);
      qv[u] = ld(q + i0, li);
      if constexpr (JAC) dv[u] = ld(dg + i0, li);
    }
  };
  // the first round's loads need no scalar: issued before the state is
  // known and the p.Ap partials are summed, so that the latencies overlap
  load_round(wk.first * B);
  if (st_in != ST_RUNNING) {
    if (lead) sc->state_r = st_in;
    return;
  }
  const double pq = sum_partials_once<NT>(part + (2 + (k & 1)) * G, G, red);
  int32_t stop = ST_RUNNING;
  if (!isfinite(pq)) stop = ST_NONFINITE;
  else if (!(pq > 0.0)) stop = ST_NOT_SPD;
  if (stop != ST_RUNNING) {
    // breakdown: x must hold x_k.  The SpMV step applied the lagged update,
    // except a line walk's odd step, which left alpha_{k-1} p_{k-1} pending
    if (c->xpair != 0 && (k & 1)) {
      SLA_GLOBAL double* x = gmem(c->x + s * n);
      const SLA_GLOBAL double* pk1 = gmem(c->p[0] + s * n);  // p_{k-1} (k odd)
      const double a1 = scg->alpha[0];                        // alpha_{k-1}
      const TileWalk tw = wave_walk(tiles, G, blockIdx.x, W, wave_index());
      for (int64_t t = tw.first; t < tw.end; t += tw.stride) {
        const int64_t i0 = t * kTileRows;
        if (i0 + lane < n) st(x + i0, lane, ld(x + i0, lane) + a1 * ld(pk1 + i0, lane));
      }
    }
    if (lead) {
      sc->it = k;
      sc->rr_final = rr;
      sc->state_r = stop;
      atomicSub(n_running, 1);
    }
    return;
  }
  const double alpha = uniform(num / pq);
  if (lead) {
    sc->alpha[k & 1] = alpha;
    sc->ka = k + 1;
  }
  double rn = 0.0, rzn = 0.0;
  for (int64_t bk = wk.first; bk < wk.end; bk += wk.stride) {
#pragma unroll
    for (int h = 0; h < B; h += U) {
      const int64_t t0 = bk * B + h;  // the round's first tile
      if (h > 0 && t0 >= tiles) break;  // (wave-uniform) the block ends early
      if (bk != wk.first || h != 0) load_round(t0);
      // no branch around the stores either (a branch makes the compiler wait
      // for every older store before the next one): a lane past the range
      // stores what the loaded row's own lane stores (from the same values,
      // loaded before this round's stores), and only owned rows enter the
      // sums, in tile order
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t t = t0 + u;
        const int64_t i0 = (t < tiles ? t : t0) * kTileRows;
        const bool own = t < tiles && i0 + lane < n;
        const uint32_t li = i0 + lane < n ? lane : uint32_t(n - 1 - i0);
        const double ri = rv[u] - alpha * qv[u];
        st(r + i0, li, ri);
        const double rn1 = rn + ri * ri;
        rn = own ? rn1 : rn;
        if constexpr (JAC) {
          const double zi = ri / dv[u];
          st(z + i0, li, zi);
          const double rzn1 = rzn + ri * zi;
          rzn = own ? rzn1 : rzn;
        }
      }
    }
  }
  rn = block_sum_once<NT>(rn, red + W);
  if constexpr (JAC) rzn = block_sum_once<NT>(rzn, red + 2 * W);
  if (threadIdx.x == 0) {
    part[((k + 1) & 1) * G + blockIdx.x] = rn;
    if constexpr (JAC) part[(5 + ((k + 1) & 1)) * G + blockIdx.x] = rzn;
  }
}

// grad_vals[s][k] = -lambda[s][i] * x[s][col[k]] for every stored slot k of
// row i (NEG; without it the product itself, the .matvec backward).  The lanes of a wave walk the tile's slots in order (coalesced
// column loads and gradient stores); each slot's row comes from an LDS map
// the lanes fill for their own rows.
template <typename RP, bool NEG>
__global__ __launch_bounds__(kIterBlock) void k_pattern_grad(const RP* __restrict__ rowptr,
                                                             const int32_t* __restrict__ col,
                                                             int64_t n, int64_t nnz, int64_t tiles,
                                                             int cap,
                                                             const double* __restrict__ lambda,
                                                             const double* __restrict__ x,
                                                             double* __restrict__ grad,
                                                             const int* __restrict__ gate) {
  if (gate != nullptr && *gate != 0) return;  // refused: nothing written
  extern __shared__ double lds_dyn[];
  const int w = wave_index();
  const int lane = threadIdx.x & (kWave - 1);
  uint8_t* rowmap = reinterpret_cast<uint8_t*>(lds_dyn) + int64_t(w) * cap;
  const int64_t s = blockIdx.y;
  const SLA_GLOBAL double* l = gmem(lambda + s * n);
  const SLA_GLOBAL double* xs = gmem(x + s * n);
  SLA_GLOBAL double* gs = gmem(grad + s * nnz);
  // contiguous tile ranges per XCD (the grid is a multiple of kXcds): tiles
  // that gather the same entries of x run close together on one L2
  const TileWalk walk = wave_walk(tiles, int(gridDim.x), int(blockIdx.x), kWaves, w);
  for (int64_t t = walk.first; t < walk.end; t += walk.stride) {
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
      for (int64_t k = lane; k < clen; k += kWave) {
        const double pr = l[r0 + rowmap[k]] * xs[col[s0 + c0 + k]];
        gs[s0 + c0 + k] = NEG ? -pr : pr;
      }
      wave_sync();
    }
  }
}

size_t lds_bytes(const sla_csr A) { return use_band(A) ? 0 : solver_lds_bytes(A->wave_cap, kWaves); }

// Vectors of 4 GiB or more need 64-bit gather addresses.
bool wide_vectors(const sla_csr A) { return uint64_t(A->n) * sizeof(double) >= (uint64_t(1) << 32); }

// Kernel family of the row sums: the smallest of 3, 5, 8 offsets that holds
// a band, else 0 (plain CSR) or -1 (plain CSR, vectors of 4 GiB or more).
// Line-walk chunks per XCD, so that every workgroup of an XCD gets the same
// number of (kLineWaves-column group, chunk) units: per_xcd / gcd(groups,
// per_xcd).
int64_t line_chunks(const sla_csr A, int32_t grid) {
  const int64_t per_xcd = grid / kXcds;
  const int64_t U = (A->line + kTileRows - 1) / kTileRows;
  const int64_t groups = (U + kLineWaves - 1) / kLineWaves;
  int64_t a = per_xcd, b = groups;
  while (b != 0) {
    const int64_t t = a % b;
    a = b;
    b = t;
  }
  return per_xcd / a;
}

// Lines a wave walks in one chunk (about).
int64_t line_chunk_lines(const sla_csr A, int32_t grid) {
  const int64_t V = (A->n + A->line - 1) / A->line;
  return V / kXcds / std::max<int64_t>(1, line_chunks(A, grid));
}

int band_class(const sla_csr A) {
  if (!use_band(A)) return wide_vectors(A) ? -1 : 0;
  return A->band.count <= 3 ? 3 : (A->band.count <= 5 ? 5 : 8);
}

template <typename RP>
const void* spmv_step_kernel(const sla_csr A, int32_t grid) {
  const int nb = band_class(A);
  if (use_lines(A)) {
    // NEAR1: the offsets between -L and +L are only -1, 0, +1
    bool near1 = true;
    for (int t = 1; t + 1 < A->band.count; ++t)
      near1 = near1 && A->band.off[t] >= -1 && A->band.off[t] <= 1;
    // the two-deep pipeline pays off once a wave walks a dozen lines or more,
    // on matrices whose vectors stay partly in the Infinity Cache
    if (line_chunk_lines(A, grid) >= kPipeLines && A->n <= kPipeMaxRows) {
      if (near1 && nb <= 5)
        return nb == 3 ? reinterpret_cast<const void*>(&k_cg_spmv_lines<RP, 3, true, true>)
                       : reinterpret_cast<const void*>(&k_cg_spmv_lines<RP, 5, true, true>);
      switch (nb) {
        case 3: return reinterpret_cast<const void*>(&k_cg_spmv_lines<RP, 3, false, true>);
        case 5: return reinterpret_cast<const void*>(&k_cg_spmv_lines<RP, 5, false, true>);
        default: return reinterpret_cast<const void*>(&k_cg_spmv_lines<RP, 8, false, true>);
      }
    }
    if (near1 && nb <= 5)
      return nb == 3 ? reinterpret_cast<const void*>(&k_cg_spmv_lines<RP, 3, true, false>)
                     : reinterpret_cast<const void*>(&k_cg_spmv_lines<RP, 5, true, false>);
    switch (nb) {
      case 3: return reinterpret_cast<const void*>(&k_cg_spmv_lines<RP, 3, false, false>);
      case 5: return reinterpret_cast<const void*>(&k_cg_spmv_lines<RP, 5, false, false>);
      default: return reinterpret_cast<const void*>(&k_cg_spmv_lines<RP, 8, false, false>);
    }
  }
  switch (nb) {
    case 3:
      return A->panel > 0 ? reinterpret_cast<const void*>(&k_cg_spmv<RP, 3, 512>)
                          : reinterpret_cast<const void*>(&k_cg_spmv<RP, 3, 1024>);
    case 5:
      return A->panel > 0 ? reinterpret_cast<const void*>(&k_cg_spmv<RP, 5, 512>)
                          : reinterpret_cast<const void*>(&k_cg_spmv<RP, 5, 1024>);
    case 8:
      return A->panel > 0 ? reinterpret_cast<const void*>(&k_cg_spmv<RP, 8, 512>)
                          : reinterpret_cast<const void*>(&k_cg_spmv<RP, 8, 1024>);
    case -1: return reinterpret_cast<const void*>(&k_cg_spmv<RP, -1>);
    default: return reinterpret_cast<const void*>(&k_cg_spmv<RP, 0>);
  }
}

template <typename RP>
const void* product_kernel(const sla_csr A) {
  return wide_vectors(A) ? reinterpret_cast<const void*>(&k_cg_product<RP, true>)
                         : reinterpret_cast<const void*>(&k_cg_product<RP, false>);
}

// Threads per workgroup of the SpMV step kernel: the line walk's; 8 waves for
// a band in panel order (measured on the 7-point 3D Laplacian: 23.5 vs 30.6
// us per step at 100^3, 216 vs 280 us at 200^3, against 16 waves); 16 for the
// other bands (a 2D band without panels, 1000^2: 17.2 us, 18.7 with 8 waves)
// and plain CSR rows.
unsigned spmv_step_block(const sla_csr A) {
  if (use_lines(A)) return kLineWaves * kWave;
  return use_band(A) && A->panel > 0 ? 512u : unsigned(kIterBlock);
}

// Threads per workgroup of the residual step: 8 waves, whose blocks of
// kStreamTiles tiles stream faster than 16 waves' (at 169M unknowns 0.77 vs
// 0.81 ms per step: fewer waves per CU keep fewer DRAM pages open), and 16
// where that lets every wave finish in one round of loads while 8 waves
// would need two (the 10^6-unknown grid at one workgroup per CU).
unsigned residual_block(const sla_csr A, int32_t grid) {
  const int64_t blocks = (A->tiles + kStreamTiles - 1) / kStreamTiles;
  const int64_t g = grid;
  return blocks > g * (512 / kWave) && blocks <= g * (1024 / kWave) ? 1024u : 512u;
}

const void* residual_kernel(bool jacobi, unsigned threads) {
  if (threads == 1024u)
    return jacobi ? reinterpret_cast<const void*>(&k_cg_residual<true, 1024>)
                  : reinterpret_cast<const void*>(&k_cg_residual<false, 1024>);
  return jacobi ? reinterpret_cast<const void*>(&k_cg_residual<true, 512>)
                : reinterpret_cast<const void*>(&k_cg_residual<false, 512>);
}

sla_status launch_ctx_kernel(const void* fn, dim3 grid, unsigned block, size_t lds, const Ctx* cd,
                             hipStream_t st) {
  void* args[1] = {&cd};
  const hipError_t e = hipLaunchKernel(fn, grid, dim3(block), args, lds, st);
  if (e != hipSuccess) {
    set_error("kernel launch failed: %s", hipGetErrorString(e));
    return SLA_ERR_DEVICE;
  }
  return SLA_OK;
}

template <typename RP>
sla_status enqueue_iteration(sla_csr A, const CgSpace& sp, int64_t batch, bool jacobi,
                             hipStream_t st) {
  const dim3 grid2(unsigned(sp.grid), unsigned(batch));
  if (use_split(A)) {
    k_cg_direction<<<grid2, kIterBlock, 0, st>>>(sp.ctx_dev);
    SLA_TRY(launch_ctx_kernel(product_kernel<RP>(A), grid2, kIterBlock, lds_bytes(A), sp.ctx_dev,
                              st));
  } else {
    SLA_TRY(launch_ctx_kernel(spmv_step_kernel<RP>(A, sp.grid), grid2, spmv_step_block(A),
                              lds_bytes(A), sp.ctx_dev, st));
  }
  const unsigned rb = residual_block(A, sp.grid);
  SLA_TRY(launch_ctx_kernel(residual_kernel(jacobi, rb), grid2, rb, 0, sp.ctx_dev, st));
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status enqueue_block(sla_csr A, const CgSpace& sp, int64_t batch, bool jacobi,
                         int64_t iters, hipStream_t st) {
  for (int64_t k = 0; k < iters; ++k) {
    if (A->rp_idx == SLA_I32) SLA_TRY(enqueue_iteration<int32_t>(A, sp, batch, jacobi, st));
    else SLA_TRY(enqueue_iteration<int64_t>(A, sp, batch, jacobi, st));
  }
  return SLA_OK;
}

sla_status get_graph(sla_csr A, int64_t batch, bool jacobi, hipGraphExec_t* exec) {
  // one graph per (batch, preconditioner): the kernels differ
  const int64_t key = batch * 2 + (jacobi ? 1 : 0);
  auto it = A->graphs.find(key);
  if (it != A->graphs.end()) {
    *exec = it->second.second;
    return SLA_OK;
  }
  if (A->capture_stream == nullptr)
    SLA_TRY_HIP(hipStreamCreateWithFlags(&A->capture_stream, hipStreamNonBlocking));
  hipGraph_t g = nullptr;
  hipGraphExec_t e = nullptr;
  SLA_TRY_HIP(hipStreamBeginCapture(A->capture_stream, hipStreamCaptureModeThreadLocal));
  sla_status s = enqueue_block(A, own_space(A), batch, jacobi, A->graph_block, A->capture_stream);
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
  A->graphs[key] = {g, e};
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

void fill_ctx(sla_csr A, const CgSpace& sp, Ctx& c, const double* b, double* x, int64_t batch,
              bool hist, bool jacobi = false) {
  c = Ctx{};
  c.rowptr = A->rowptr;
  c.col = A->col;
  c.vals = A->vals;
  c.x = x;
  c.b = b;
  c.r = sp.r;
  c.jacobi = jacobi ? 1 : 0;
  c.diag = jacobi ? A->jdiag : nullptr;
  c.z = jacobi ? A->jz : nullptr;
  c.bad = jacobi ? A->jbad : nullptr;
  c.rd = jacobi ? A->jz : sp.r;
  c.p[0] = sp.p0;
  c.p[1] = sp.p1;
  c.q = sp.q;
  c.part = sp.part;
  c.scal = scal_of(sp.ctx_dev, 0);
  c.hist = hist ? A->hist : nullptr;
  c.hist_cap = hist ? A->hist_cap : 0;
  c.n_running = sp.n_running;
  c.n = A->n;
  c.nnz = A->nnz;
  c.batch = batch;
  c.tiles = A->tiles;
  c.grid = sp.grid;
  c.wave_cap = A->wave_cap;
  c.mask = use_band(A) ? A->band_mask : nullptr;
  c.band = A->band;
  c.panel = A->panel;
  c.pblock = A->pblock;
  c.line = use_lines(A) ? A->line : 0;
  c.line_chunks = c.line > 0 ? line_chunks(A, sp.grid) : 0;
  c.xpair = c.line > 0 ? 1 : 0;
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

bool use_lines(const sla_csr A) {
  if (A->line <= 0 || !use_band(A)) return false;
  return A->spmv_variant == SLA_SPMV_AUTO || A->spmv_variant == SLA_SPMV_LINES;
}

bool use_band(const sla_csr A) {
  if (A->band_mask == nullptr || A->spmv_variant == SLA_SPMV_CSR ||
      A->spmv_variant == SLA_SPMV_SPLIT)
    return false;
  // automatic: whenever a band was detected (fewer bytes per slot, and no
  // LDS staging between the index loads and the gathers)
  return true;
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
  dev_free(A->n_running);
  dev_free(A->ctx_dev);
  dev_free(A->hist);
  dev_free(A->jz);
  dev_free(A->jdiag);
  dev_free(A->jbad);
  A->jz = A->jdiag = nullptr;
  A->jbad = nullptr;
  dev_free(A->grid_slot);
  dev_free(A->grid_halo);
  dev_free(A->grid_fail);
  A->grid_slot = nullptr;
  A->grid_halo = nullptr;
  A->grid_fail = nullptr;
  A->grid_slot_words = A->grid_halo_len = 0;
  for (auto& e : A->grid_ev)
    if (e) (void)hipEventDestroy(e);
  A->grid_ev[0] = A->grid_ev[1] = nullptr;
  A->grid_timed = false;
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
  A->ws_batch = A->ws_cap = A->part_cap = 0;
  A->hist_cap = A->hist_batch = 0;
}

// Solver grid: wg_per_cu workgroups per CU in total, a multiple of the XCD
// count per system, never more than the wave tiles need (rounded up)
// (automatic: one per CU up to kSmallSolve unknowns over the batch, where
// the kernels' fixed costs -- each workgroup summing the partials of the
// previous kernel -- weigh more than the latency hiding of a second one)
// (and for line walks at any size: their waves stream long chunks, and
// with half the workgroups each chunk is twice as long)
int32_t solver_grid(const sla_csr A, int64_t batch) {
  const int wg = A->wg_per_cu > 0 ? A->wg_per_cu
                                  : (A->n * batch <= kSmallSolve || use_lines(A) ? 1 : 2);
  const int64_t target = std::max<int64_t>(kXcds, int64_t(device_cus()) * wg / batch);
  int64_t g = std::min<int64_t>((A->tiles + kWaves - 1) / kWaves, target);
  g = (g + kXcds - 1) / kXcds * kXcds;
  return int32_t(std::max<int64_t>(g, kXcds));
}

CgSpace own_space(sla_csr A) {
  CgSpace sp;
  sp.r = A->r;
  sp.p0 = A->p0;
  sp.p1 = A->p1;
  sp.q = A->q;
  sp.part = A->part;
  sp.ctx_dev = A->ctx_dev;
  sp.n_running = A->n_running;
  sp.ctx_host = A->ctx_host;
  sp.scal_host = A->scal_host;
  sp.poll_host = A->poll_host;
  sp.poll_ev = A->poll_ev;
  sp.grid = A->grid;
  sp.own = true;
  return sp;
}

// The buffers of a larger batch serve a smaller one as they are (a handle
// that alternates batch sizes, e.g. one system and then a batch of them, is
// not reallocated on every call; the captured graphs are kept per batch and
// stay valid as long as the buffers do).  A larger batch, or more partials
// than the buffers hold, reallocates everything.
sla_status ensure_workspace(sla_csr A, int64_t batch) {
  const int32_t grid = solver_grid(A, batch);
  const int64_t parts = int64_t(kPartSets) * batch * grid;
  if (A->r != nullptr && batch <= A->ws_cap && parts <= A->part_cap) {
    A->grid = grid;
    A->ws_batch = batch;
    return SLA_OK;
  }
  release_workspace(A);
  const int64_t n = A->n;
  A->grid = grid;
  const size_t vec = size_t(batch) * size_t(n);
  SLA_TRY(dev_alloc(&A->r, vec, "r"));
  SLA_TRY(dev_alloc(&A->p0, vec, "p"));
  SLA_TRY(dev_alloc(&A->p1, vec, "p"));
  SLA_TRY(dev_alloc(&A->q, vec, "q"));
  SLA_TRY(dev_alloc(&A->part, size_t(parts), "partials"));
  SLA_TRY(dev_alloc(&A->n_running, 1, "running count"));
  // the context, then the systems' scalars (scal_of)
  SLA_TRY(dev_alloc(reinterpret_cast<void**>(&A->ctx_dev), sizeof(Ctx) + sizeof(Scal) * batch,
                    "context and scalars"));
  A->scal = scal_of(A->ctx_dev, 0);
  SLA_TRY_HIP(hipHostMalloc(reinterpret_cast<void**>(&A->ctx_host), sizeof(Ctx)));
  SLA_TRY_HIP(hipHostMalloc(reinterpret_cast<void**>(&A->scal_host), sizeof(Scal) * batch));
  SLA_TRY_HIP(hipHostMalloc(reinterpret_cast<void**>(&A->poll_host), sizeof(int) * 2));
  for (auto& e : A->poll_ev) SLA_TRY_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  A->ws_batch = A->ws_cap = batch;
  A->part_cap = parts;
  return SLA_OK;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
// Workgroups per system of the plain SpMV: a multiple of kXcds (its tile
// walk splits the tiles by XCD).
static unsigned spmv_grid(int64_t tiles, int64_t batch) {
  const unsigned g = plain_grid(tiles, batch);
  return (g + kXcds - 1) / kXcds * kXcds;
}

template <int ND>
static sla_status launch_spmv_nd(sla_csr A, const double* vals, int64_t batch, const double* x,
                                 double* y, const double* wdot, double* part, int64_t pstride,
                                 int set0, int set1, hipStream_t st) {
  const dim3 grid(spmv_grid(A->tiles, batch), unsigned(batch));
  const size_t lds = lds_bytes(A);
  const int nb = band_class(A);
  // banded rows on 8-wave workgroups once 16 waves would walk 4 tiles or more
  // each (4000^2 Poisson: 198 vs 214 us per product; at 1000^2, 2 tiles per
  // wave, 16 waves are faster: 11.3 vs 12.3 us)
  const bool eight = nb > 0 && A->tiles >= int64_t(grid.x) * 64;
  if (A->rp_idx == SLA_I32) {
    auto k = nb == 3 ? (eight ? k_spmv<int32_t, 3, ND, 512> : k_spmv<int32_t, 3, ND>)
             : nb == 5 ? (eight ? k_spmv<int32_t, 5, ND, 512> : k_spmv<int32_t, 5, ND>)
             : nb == 8 ? (eight ? k_spmv<int32_t, 8, ND, 512> : k_spmv<int32_t, 8, ND>)
             : nb == 0 ? k_spmv<int32_t, 0, ND> : k_spmv<int32_t, -1, ND>;
    k<<<grid, eight ? 512 : kIterBlock, lds, st>>>((const int32_t*)A->rowptr, A->col, A->band_mask, A->band,
                                     vals, A->n, A->nnz, A->tiles, A->wave_cap, x, y, wdot, part,
                                     pstride, set0, set1);
  } else {
    auto k = nb == 3 ? (eight ? k_spmv<int64_t, 3, ND, 512> : k_spmv<int64_t, 3, ND>)
             : nb == 5 ? (eight ? k_spmv<int64_t, 5, ND, 512> : k_spmv<int64_t, 5, ND>)
             : nb == 8 ? (eight ? k_spmv<int64_t, 8, ND, 512> : k_spmv<int64_t, 8, ND>)
             : nb == 0 ? k_spmv<int64_t, 0, ND> : k_spmv<int64_t, -1, ND>;
    k<<<grid, eight ? 512 : kIterBlock, lds, st>>>((const int64_t*)A->rowptr, A->col, A->band_mask, A->band,
                                     vals, A->n, A->nnz, A->tiles, A->wave_cap, x, y, wdot, part,
                                     pstride, set0, set1);
  }
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status launch_spmv(sla_csr A, const double* vals, int64_t batch, const double* x, double* y,
                       hipStream_t st) {
  return launch_spmv_nd<0>(A, vals, batch, x, y, nullptr, nullptr, 0, 0, 0, st);
}

int64_t spmv_groups(const sla_csr A, int64_t batch) { return spmv_grid(A->tiles, batch); }

sla_status launch_spmv_dots(sla_csr A, const double* vals, int64_t batch, const double* x,
                            double* y, const double* wdot, int nd, double* part, int64_t pstride,
                            int set0, int set1, hipStream_t st) {
  if (nd == 1)
    return launch_spmv_nd<1>(A, vals, batch, x, y, wdot, part, pstride, set0, set1, st);
  return launch_spmv_nd<2>(A, vals, batch, x, y, wdot, part, pstride, set0, set1, st);
}

sla_status launch_slot_products(sla_csr A, int64_t batch, const double* g, const double* x,
                                double* out, bool negate, hipStream_t st, const int* gate) {
  const unsigned per_xcd = std::max(1u, plain_grid(A->tiles, batch) / unsigned(kXcds));
  const dim3 grid(per_xcd * kXcds, unsigned(batch));
  const int cap = A->wave_cap;
  const size_t lds = size_t(kWaves) * size_t(cap);
  if (A->rp_idx == SLA_I32) {
    auto k = negate ? k_pattern_grad<int32_t, true> : k_pattern_grad<int32_t, false>;
    k<<<grid, kIterBlock, lds, st>>>((const int32_t*)A->rowptr, A->col, A->n, A->nnz, A->tiles,
                                     cap, g, x, out, gate);
  } else {
    auto k = negate ? k_pattern_grad<int64_t, true> : k_pattern_grad<int64_t, false>;
    k<<<grid, kIterBlock, lds, st>>>((const int64_t*)A->rowptr, A->col, A->n, A->nnz, A->tiles,
                                     cap, g, x, out, gate);
  }
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status launch_pattern_grad(sla_csr A, int64_t batch, const double* lambda, const double* x,
                               double* grad_vals, hipStream_t st) {
  return launch_slot_products(A, batch, lambda, x, grad_vals, true, st);
}

static sla_status finish_cg(const CgSpace& sp, int64_t batch, sla_cg_info* info,
                            hipStream_t st);

// Rows per thread of the small-system kernel (1, 2 or 4), 0 when it does not
// apply: more than kOneGroupMaxN unknowns, plain CSR rows whose 64-row tile
// has more slots than a wave stages, or LDS beyond the device's limit.
static int one_group_rows(const sla_csr A) {
  if (A->n <= 0 || A->n > kOneGroupMaxN) return 0;
  const bool band = use_band(A);
  if (!band && A->max_tile_nnz > kWaveCap) return 0;
  int lim = 0;
  if (hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, A->device) !=
          hipSuccess ||
      one_group_lds_bytes(A->n, band) + 5 * kWaves * sizeof(double) > size_t(lim))  // + red*
    return 0;
  return one_group_rows_per_thread(A->n, band);
}

bool use_one_group(const sla_csr A) {
  return A->one_group == SLA_ONE_GROUP_AUTO && one_group_rows(A) > 0;
}

// The small-system kernel for `rows` rows per thread and `nt` threads per
// workgroup (one_group_rows, one_group_block), Jacobi or not, banded rows or
// plain CSR; nullptr for a combination the size rule never picks.
using OneGroupFn = void (*)(const Ctx, Scal*, double, int64_t, int, const int*);

template <typename RP, bool BAND>
static OneGroupFn one_group_kernel(int rows, int nt, bool jac) {
#define SLA_OG(R_, NT_) \
  (jac ? k_cg_onegroup<RP, R_, true, NT_, BAND> : k_cg_onegroup<RP, R_, false, NT_, BAND>)
  if (nt == 256) {
    if (rows == 1) return SLA_OG(1, 256);
    if constexpr (BAND)
      if (rows == 2) return SLA_OG(2, 256);
  } else if (nt == 512) {
    if constexpr (!BAND)
      if (rows == 1) return SLA_OG(1, 512);
    if (rows == 2) return SLA_OG(2, 512);
    if (rows == 4) return SLA_OG(4, 512);
  }
  return nullptr;
#undef SLA_OG
}

static sla_status launch_one_group(sla_csr A, const Ctx& ctx, Scal* scal, int64_t batch,
                                   bool jac, double tol, int64_t maxit, bool x0,
                                   const int* gate, hipStream_t st) {
  const bool band = use_band(A);
  const size_t lds = one_group_lds_bytes(A->n, band);
  const unsigned g = unsigned(batch);
  const int u = x0 ? 1 : 0;
  const int rows = one_group_rows(A);
  const int nt = one_group_block(A->n, band);
  if (A->rp_idx == SLA_I32) {
    auto k = band ? one_group_kernel<int32_t, true>(rows, nt, jac)
                  : one_group_kernel<int32_t, false>(rows, nt, jac);
    if (k == nullptr) {
      set_error("small-system kernel: no variant for %d rows x %d threads", rows, nt);
      return SLA_ERR_DEVICE;
    }
    k<<<g, unsigned(nt), lds, st>>>(ctx, scal, tol, maxit, u, gate);
  } else {
    auto k = band ? one_group_kernel<int64_t, true>(rows, nt, jac)
                  : one_group_kernel<int64_t, false>(rows, nt, jac);
    if (k == nullptr) {
      set_error("small-system kernel: no variant for %d rows x %d threads", rows, nt);
      return SLA_ERR_DEVICE;
    }
    k<<<g, unsigned(nt), lds, st>>>(ctx, scal, tol, maxit, u, gate);
  }
  LAUNCH_CHECK();
  return SLA_OK;
}

// ---------------------------------------------------------------------------
// The resident grid loop: plan and launch
// ---------------------------------------------------------------------------
// Single banded systems above the one-workgroup loop's range (that loop is
// faster up to its 2048 unknowns: 1.9 us per iteration at 45^2) while the
// rows fit: per iteration on Poisson grids, 100^2 5.8 us against 10.4 on the
// two-kernel loop, 300^2 7.1 / 10.9, 512^2 7.8 / 12.3, 1000^2 10.5 / 22.9:
// rw = max(ceil(n / CUs),
// H) rows per workgroup, at most 8 per thread, p with its halo in 64 KB of
// LDS, 2 H halo rows at most 4 per thread, every workgroup resident.
constexpr int64_t kGridMinN = kOneGroupMaxN + 1;
constexpr int64_t kGridPollLimit = int64_t(1) << 20;  // about a second of polling
// Copies of the sum slots: every workgroup posts its partials into each, and
// polls the copy g % kGridReps, so no few memory lines take every poll
constexpr int32_t kGridReps = 8;
constexpr int64_t kGridRepAlign = 528;  // words (4 KB + 128 B: replicas on other lines)

struct GridPlan {
  int32_t G = 0;
  int64_t rw = 0;
  int32_t H = 0;
  int32_t rpt = 0;
  int32_t nb = 0;
  size_t lds = 0;
};

using GridFn = void (*)(const Ctx, Scal*, const GridSync, double, int64_t, int, const int*);

template <typename RP>
static GridFn grid_kernel_rp(int rpt, int nb) {
#define SLA_GK(R_)                                                                     \
  (nb == 3 ? k_cg_grid<RP, R_, 3> : nb == 5 ? k_cg_grid<RP, R_, 5> : k_cg_grid<RP, R_, 8>)
  switch (rpt) {
    case 1: return SLA_GK(1);
    case 2: return SLA_GK(2);
    case 4: return SLA_GK(4);
    case 8: return SLA_GK(8);
    default: return nullptr;
  }
#undef SLA_GK
}

static GridFn grid_kernel(const sla_csr A, int rpt, int nb) {
  return A->rp_idx == SLA_I32 ? grid_kernel_rp<int32_t>(rpt, nb) : grid_kernel_rp<int64_t>(rpt, nb);
}

static bool grid_plan(const sla_csr A, int64_t batch, bool jacobi, GridPlan* gp) {
  if (A->one_group != SLA_ONE_GROUP_AUTO || batch != 1 || jacobi || !use_band(A)) return false;
  const int64_t n = A->n;
  if (n < kGridMinN) return false;
  int32_t H = 0;
  for (int o = 0; o < A->band.count; ++o)
    H = std::max<int32_t>(H, A->band.off[o] < 0 ? -A->band.off[o] : A->band.off[o]);
  const int cus = device_cus();
  const int64_t rw = std::max<int64_t>((n + cus - 1) / cus, std::max<int32_t>(H, 1));
  const int64_t G = (n + rw - 1) / rw;
  const int64_t need = (rw + kGridThreads - 1) / kGridThreads;
  const int rpt = need <= 1 ? 1 : need <= 2 ? 2 : need <= 4 ? 4 : need <= 8 ? 8 : 0;
  if (rpt == 0 || 2 * int64_t(H) > int64_t(kGridHaloPT) * kGridThreads) return false;
  if (G > int64_t(kGridThreads / kWave) * kWave) return false;  // a slot per polling lane
  const int nb = band_class(A);
  if (rpt == 8 && nb == 8) return false;  // (that variant spills registers)
  // r with its halo and a spare slot, then A r, p and x of the rows, each
  // with a spare slot
  const size_t lds = size_t(4 * rw + 2 * int64_t(H) + 4) * sizeof(double);
  int lds_max = 0;
  if (hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, A->device) !=
          hipSuccess ||
      lds + 1024 > size_t(lds_max))  // + the static areas
    return false;
  int coop = 0;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, A->device) != hipSuccess ||
      !coop)
    return false;
  const GridFn fn = grid_kernel(A, rpt, nb);
  if (fn != nullptr && lds > size_t(64) * 1024 &&
      hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                          hipFuncAttributeMaxDynamicSharedMemorySize, int(lds)) != hipSuccess)
    return false;
  int per_cu = 0;
  if (fn == nullptr ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn),
                                                   kGridThreads, lds) != hipSuccess ||
      G > int64_t(per_cu) * cus)
    return false;
  gp->G = int32_t(G);
  gp->rw = rw;
  gp->H = H;
  gp->rpt = rpt;
  gp->nb = nb;
  gp->lds = lds;
  return true;
}

bool use_grid(const sla_csr A, int64_t batch, bool jacobi) {
  GridPlan gp;
  return grid_plan(A, batch, jacobi, &gp);
}

static sla_status launch_grid(sla_csr A, const GridPlan& gp, const Ctx& ctx, Scal* scal,
                              double tol, int64_t maxit, bool x0, const int* gate,
                              hipStream_t st) {
  // replicas kGridRepAlign words apart at least, each a whole number of
  // those
  const int64_t rep_words =
      (int64_t(2) * kGridVals * gp.G + kGridRepAlign - 1) / kGridRepAlign * kGridRepAlign;
  const int64_t words = int64_t(2) * kGridReps * rep_words;
  const int64_t halo = int64_t(2) * gp.G * 2 * gp.H * 2;  // tagged words
  if (A->grid_slot == nullptr || A->grid_slot_words < words || A->grid_halo_len < halo) {
    dev_free(A->grid_slot);
    dev_free(A->grid_halo);
    A->grid_slot = nullptr;
    A->grid_halo = nullptr;
    A->grid_slot_words = A->grid_halo_len = 0;
    SLA_TRY(dev_alloc(&A->grid_slot, size_t(words), "grid sum slots"));
    SLA_TRY(dev_alloc(&A->grid_halo, size_t(std::max<int64_t>(halo, 1)), "grid halo rows"));
    A->grid_slot_words = words;
    A->grid_halo_len = halo;
  }
  if (A->grid_fail == nullptr) SLA_TRY(dev_alloc(&A->grid_fail, 1, "grid failure flag"));
  if (A->grid_ev[0] == nullptr)
    for (auto& e : A->grid_ev) SLA_TRY_HIP(hipEventCreate(&e));
  k_grid_clear<<<unsigned((words + halo + 255) / 256), 256, 0, st>>>(A->grid_slot, words,
                                                                     A->grid_halo, halo,
                                                                     A->grid_fail);
  LAUNCH_CHECK();
  GridSync gs;
  gs.slot = A->grid_slot;
  gs.halo = A->grid_halo;
  gs.fail = A->grid_fail;
  gs.rw = gp.rw;
  gs.H = gp.H;
  gs.reps = kGridReps;
  gs.rep_words = rep_words;
  gs.poll_limit = kGridPollLimit;
  const GridFn fn = grid_kernel(A, gp.rpt, gp.nb);
  if (fn == nullptr) {
    set_error("resident CG loop: no variant for %d rows per thread", gp.rpt);
    return SLA_ERR_DEVICE;
  }
  Ctx c = ctx;
  int u = x0 ? 1 : 0;
  void* args[] = {&c, &scal, &gs, &tol, &maxit, &u, const_cast<const int**>(&gate)};
  SLA_TRY_HIP(hipEventRecord(A->grid_ev[0], st));
  SLA_TRY_HIP(hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fn), dim3(unsigned(gp.G)),
                                         dim3(kGridThreads), args, gp.lds, st));
  SLA_TRY_HIP(hipEventRecord(A->grid_ev[1], st));
  A->grid_timed = true;
  return SLA_OK;
}

// After a resident grid solve: a wait that timed out anywhere is an error,
// whatever the state the first workgroup recorded.
static sla_status grid_check(sla_csr A, sla_status s, hipStream_t st) {
  int h = 0;
  SLA_TRY_HIP(hipMemcpyAsync(&h, A->grid_fail, sizeof(int), hipMemcpyDeviceToHost, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));
  if (h != 0) {
    set_error("resident CG loop: a grid-wide wait timed out");
    return SLA_ERR_DEVICE;
  }
  return s;
}

sla_status grid_loop_ms(sla_csr A, double* ms) {
  if (!A->grid_timed) return SLA_ERR_ARG;
  float f = 0.0f;
  SLA_TRY_HIP(hipEventSynchronize(A->grid_ev[1]));
  SLA_TRY_HIP(hipEventElapsedTime(&f, A->grid_ev[0], A->grid_ev[1]));
  *ms = double(f);
  return SLA_OK;
}

sla_status run_cg(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                  uint32_t flags, sla_cg_info* info, hipStream_t st, const AdjointTail* tail) {
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
  const bool jacobi = (flags & SLA_FLAG_JACOBI) != 0;
  if (jacobi && A->jz == nullptr) {
    // Jacobi workspace: z and the diagonal [ws_cap][n], a flag per system
    // (zero here, and cleared again by every solve that sets it)
    const size_t vec = size_t(A->ws_cap) * size_t(A->n);
    SLA_TRY(dev_alloc(&A->jz, vec, "z"));
    SLA_TRY(dev_alloc(&A->jdiag, vec, "diagonal"));
    SLA_TRY(dev_alloc(&A->jbad, size_t(A->ws_cap), "diagonal flags"));
    SLA_TRY_HIP(hipMemsetAsync(A->jbad, 0, sizeof(int) * size_t(A->ws_cap), st));
  }
  return run_cg_space(A, own_space(A), b, x, tol, maxit, flags, info, st, tail);
}

// The context of a solve written into device memory by a one-thread kernel
// (the context passed by value): no host staging buffer is involved.
__global__ void k_store_ctx(Ctx c, Ctx* __restrict__ dst) { *dst = c; }

sla_status run_cg_space(sla_csr A, const CgSpace& sp, const double* b, double* x, double tol,
                        int64_t maxit, uint32_t flags, sla_cg_info* info, hipStream_t st,
                        const AdjointTail* tail) {
  const int64_t batch = A->batch;
  const bool want_hist = (flags & SLA_FLAG_HISTORY) != 0;
  const bool jacobi = (flags & SLA_FLAG_JACOBI) != 0;
  fill_ctx(A, sp, *sp.ctx_host, b, x, batch, want_hist, jacobi);
  const bool x0 = (flags & SLA_FLAG_X0) != 0;
  GridPlan gp;
  if (sp.own && (flags & kFlagNoResident) == 0 && grid_plan(A, batch, jacobi, &gp)) {
    // the context by value; the record is read back from the device
    SLA_TRY(launch_grid(A, gp, *sp.ctx_host, scal_of(sp.ctx_dev, 0), tol, maxit, x0,
                        tail ? tail->gate : nullptr, st));
    if (tail != nullptr && tail->grad_vals != nullptr)
      SLA_TRY(launch_slot_products(A, batch, x, tail->x, tail->grad_vals, true, st, tail->gate));
    return grid_check(A, finish_cg(sp, batch, info, st), st);
  }
  if (use_one_group(A)) {
    // the context by value; the records are read back from the device
    SLA_TRY(launch_one_group(A, *sp.ctx_host, scal_of(sp.ctx_dev, 0), batch, jacobi, tol, maxit,
                             x0, tail ? tail->gate : nullptr, st));
    if (tail != nullptr && tail->grad_vals != nullptr)  // from the last iterate, as below
      SLA_TRY(launch_slot_products(A, batch, x, tail->x, tail->grad_vals, true, st, tail->gate));
    return finish_cg(sp, batch, info, st);
  }
  if (tail != nullptr) {
    set_error("CG: an adjoint tail needs the one-workgroup loop (internal error)");
    return SLA_ERR_DEVICE;
  }
  if (sp.own) {
    SLA_TRY_HIP(hipMemcpyAsync(sp.ctx_dev, sp.ctx_host, sizeof(Ctx), hipMemcpyHostToDevice, st));
  } else {
    k_store_ctx<<<1, 1, 0, st>>>(*sp.ctx_host, sp.ctx_dev);
    LAUNCH_CHECK();
  }

  if (x0) SLA_TRY(launch_spmv(A, A->vals, batch, x, sp.q, st));  // q = A x0
  const dim3 grid2(unsigned(sp.grid), unsigned(batch));
  if (A->rp_idx == SLA_I32) k_cg_init<int32_t><<<grid2, kIterBlock, 0, st>>>(sp.ctx_dev, x0 ? 1 : 0);
  else k_cg_init<int64_t><<<grid2, kIterBlock, 0, st>>>(sp.ctx_dev, x0 ? 1 : 0);
  k_cg_init_scalars<<<unsigned(batch), kIterBlock, 0, st>>>(sp.ctx_dev, tol, maxit);
  LAUNCH_CHECK();
  SLA_TRY_HIP(hipMemcpyAsync(sp.poll_host, sp.n_running, sizeof(int), hipMemcpyDeviceToHost,
                             st));
  SLA_TRY_HIP(hipStreamSynchronize(st));

  if (sp.poll_host[0] > 0) {
    // at most maxit + 1 SpMV steps: the last one only applies the x update
    // (without graphs: 16 iterations between polls on the handle's workspace,
    // whose events keep one block queued; 32 on a space without events, where
    // every poll waits for the stream)
    const int64_t K = sp.own ? (A->graph_block > 0 ? A->graph_block : 16) : 32;
    const int64_t nblocks = (maxit + 1 + K - 1) / K;
    hipGraphExec_t exec = nullptr;
    if (sp.own && A->graph_block > 0) SLA_TRY(get_graph(A, batch, jacobi, &exec));
    for (int64_t j = 0; j < nblocks; ++j) {
      if (exec) SLA_TRY_HIP(hipGraphLaunch(exec, st));
      else SLA_TRY(enqueue_block(A, sp, batch, jacobi, K, st));
      SLA_TRY_HIP(hipMemcpyAsync(sp.poll_host + (j & 1), sp.n_running, sizeof(int),
                                 hipMemcpyDeviceToHost, st));
      if (sp.poll_ev != nullptr) {
        SLA_TRY_HIP(hipEventRecord(sp.poll_ev[j & 1], st));
        if (j >= 1) {
          // wait for the previous block only, so one block is always queued
          SLA_TRY_HIP(hipEventSynchronize(sp.poll_ev[(j - 1) & 1]));
          if (sp.poll_host[(j - 1) & 1] == 0) break;
        }
      } else {
        // no events: wait for this block
        SLA_TRY_HIP(hipStreamSynchronize(st));
        if (sp.poll_host[j & 1] == 0) break;
      }
    }
  }
  return finish_cg(sp, batch, info, st);
}

// The per-system scalars back to the host, the infos and the status of the
// solve (the first failing system's).
static sla_status finish_cg(const CgSpace& sp, int64_t batch, sla_cg_info* info,
                            hipStream_t st) {
  SLA_TRY_HIP(hipMemcpyAsync(sp.scal_host, scal_of(sp.ctx_dev, 0), sizeof(Scal) * batch,
                             hipMemcpyDeviceToHost, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));

  sla_status first = SLA_OK;
  for (int64_t s = 0; s < batch; ++s) {
    const Scal& sc = sp.scal_host[s];
    const int32_t state = sc.state_a != ST_RUNNING ? sc.state_a : sc.state_r;
    if (state == ST_GRID_TIMEOUT) {
      set_error("resident CG loop: a grid-wide wait timed out");
      if (info) {
        info[s].iterations = sc.it;
        info[s].rel_residual = 0.0;
        info[s].converged = 0;
        info[s].status = SLA_ERR_DEVICE;
      }
      if (first == SLA_OK) first = SLA_ERR_DEVICE;
      continue;
    }
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
  // the SpMV step is one kernel, or the direction and product passes
  const bool split = use_split(A);
  const void* fns[4];
  size_t ldss[4];
  unsigned blocks[4];
  int nk = 0;
  if (split) {
    fns[nk] = reinterpret_cast<const void*>(&k_cg_direction);
    blocks[nk] = kIterBlock;
    ldss[nk++] = 0;
    fns[nk] = product_kernel<RP>(A);
    blocks[nk] = kIterBlock;
    ldss[nk++] = lds_bytes(A);
  } else {
    fns[nk] = spmv_step_kernel<RP>(A, A->grid);
    blocks[nk] = spmv_step_block(A);
    ldss[nk++] = lds_bytes(A);
  }
  blocks[nk] = residual_block(A, A->grid);
  fns[nk] = residual_kernel(false, blocks[nk]);
  ldss[nk++] = 0;
  const int res_k = nk - 1;  // the residual step's entry
  // a one-kernel SpMV step is timed again after the residual launches, which
  // move the solve to the next step: the line walk's steps alternate between
  // two kinds (x updated at even steps only), and the result is their mean
  if (!split) {
    fns[nk] = fns[0];
    blocks[nk] = blocks[0];
    ldss[nk++] = ldss[0];
  }
  const double spmv_w = split ? 1.0 : 0.5;
  std::vector<hipEvent_t> ev(size_t(2 * reps), nullptr);
  for (auto& e : ev) SLA_TRY_HIP(hipEventCreate(&e));
  sla_status status = SLA_OK;
  avg_ms[0] = avg_ms[1] = 0.0;
  for (int k = 0; k < nk && status == SLA_OK; ++k) {
    void* args[1] = {&A->ctx_dev};
    for (int64_t r = 0; r < reps; ++r) {
      hipError_t e = hipExtLaunchKernel(fns[k], grid2, dim3(blocks[k]), args, ldss[k], st,
                                        ev[2 * r], ev[2 * r + 1], 0);
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
    if (k == res_k) avg_ms[1] += total / double(reps);
    else avg_ms[0] += spmv_w * total / double(reps);
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
  fill_ctx(A, own_space(A), *A->ctx_host, b, x, 1, false);
  SLA_TRY_HIP(hipMemcpyAsync(A->ctx_dev, A->ctx_host, sizeof(Ctx), hipMemcpyHostToDevice, st));
  const dim3 grid2(unsigned(A->grid), 1u);
  if (A->rp_idx == SLA_I32) k_cg_init<int32_t><<<grid2, kIterBlock, 0, st>>>(A->ctx_dev, 0);
  else k_cg_init<int64_t><<<grid2, kIterBlock, 0, st>>>(A->ctx_dev, 0);
  k_cg_init_scalars<<<1u, kIterBlock, 0, st>>>(A->ctx_dev, 0.0, huge);
  LAUNCH_CHECK();
  if (A->rp_idx == SLA_I32) SLA_TRY(enqueue_iteration<int32_t>(A, own_space(A), 1, false, st));
  else SLA_TRY(enqueue_iteration<int64_t>(A, own_space(A), 1, false, st));
  if (A->rp_idx == SLA_I32) return time_kernels<int32_t>(A, reps, avg_ms, st);
  return time_kernels<int64_t>(A, reps, avg_ms, st);
}

}  // namespace sla
