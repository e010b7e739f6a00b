// Locality ordering of the unknowns for the iterative solvers.
//
// A pattern whose unknowns come in an order unrelated to its graph (the
// random geometric graph of the torch-sla explainer's benchmark set, whose
// nodes are numbered in sampling order) makes every gathered p[col] of the
// SpMV a miss in every cache.  Renumbering the unknowns in the breadth-first
// order of the pattern's graph (Cuthill-McKee's level structure) puts the
// neighbours of consecutive rows within a narrow window of indices, so the
// gathers hit L2.  The solvers then run on B = P A P^T with b and x permuted
// on the way in and out; CG's iterates are those of the original system
// permuted, in exact arithmetic.
//
// The order (the same as the breadth-first order of the visit the graph
// libraries make, e.g. scipy's breadth_first_order):
//   s0 = the smallest index of largest row length;
//   s1 = the smallest index among the nodes farthest from s0 (in edges);
//   a visit from s1, each node's neighbours taken in ascending column order,
//   then from the smallest unvisited index while nodes remain.
// It is computed on the device by one workgroup, level by level: every node
// reached from the current level is claimed by its earliest parent (an
// atomic minimum of parent positions), each parent counts its claims, a
// block scan of the counts gives each parent its place, and each parent
// writes its claimed nodes in its row's column order.  The result does not
// depend on the timing of the atomics, so the order is reproducible.
#include <algorithm>
#include <climits>

#include "handle.h"

namespace sla {

struct Reorder {
  sla_csr B = nullptr;          // P A P^T: pattern and solver workspace
  int32_t* order = nullptr;     // [n] original index of the unknown at each position
  double* vals = nullptr;       // [vals_batch][nnz] values of B (gathered each call)
  int64_t vals_batch = 0;
  double* vin = nullptr;        // [vec_batch][n] permuted right-hand sides
  double* vout = nullptr;       // [vec_batch][n] permuted solutions
  int64_t vec_batch = 0;
};

namespace {

constexpr int kBfsThreads = 1024;
constexpr int kBfsWaves = kBfsThreads / kWave;

inline unsigned blocks_for(int64_t work) {
  const int64_t g = (work + kBlock - 1) / kBlock;
  return unsigned(std::max<int64_t>(1, std::min<int64_t>(g, 1 << 20)));
}

// Every global write of the workgroup is complete and every wave sees it:
// agent-scope release, barrier, agent-scope acquire (the acquire drops the
// CU's vector L1, so later loads read what other waves wrote or claimed).
__device__ __forceinline__ void bfs_sync() {
  __threadfence();
  __syncthreads();
  __threadfence();
}

// Exclusive prefix sum of v over the workgroup (thread order); *total gets
// the sum.  Every thread must call it.
__device__ __forceinline__ int32_t bfs_scan(int32_t v, int32_t* lds, int32_t* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  int32_t inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int32_t o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == kWave - 1) lds[w] = inc;
  __syncthreads();
  int32_t before = 0, all = 0;
  for (int j = 0; j < kBfsWaves; ++j) {
    const int32_t t = lds[j];
    before += j < w ? t : 0;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + inc - v;
}

// Smallest v over the workgroup.  Every thread must call it.
__device__ __forceinline__ int64_t bfs_min(int64_t v, int64_t* lds) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int64_t o = __shfl_xor(v, off, kWave);
    v = o < v ? o : v;
  }
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  int64_t m = lds[0];
  for (int j = 1; j < kBfsWaves; ++j) m = lds[j] < m ? lds[j] : m;
  __syncthreads();
  return m;
}

// Largest v over the workgroup.  Every thread must call it.
__device__ __forceinline__ int64_t bfs_max(int64_t v, int64_t* lds) {
  return -bfs_min(-v, lds);
}

// One visit structure of the pattern's graph, by one workgroup of
// kBfsThreads threads.  pos [n] must hold -1 and key [n] INT_MAX on entry;
// cnt [n] is scratch.
//   full == 0: start at s0 (found here, written to io[0]), visit the start's
//              piece only and write s1, the smallest index of its last level,
//              to io[1];
//   full == 1: start at io[1] and visit every piece: order [n] receives the
//              original index of each position.
// io[2] is set to 1 if the bookkeeping ever disagrees with n (never, for a
// validated pattern); the kernel then stops.
template <typename RP>
__global__ __launch_bounds__(kBfsThreads) void k_bfs_order(int64_t n,
                                                           const RP* __restrict__ rowptr,
                                                           const int32_t* __restrict__ col,
                                                           int32_t* pos, int32_t* key,
                                                           int32_t* order, int32_t* cnt,
                                                           int32_t* io, int full) {
  __shared__ int32_t s_i32[kBfsWaves];
  __shared__ int64_t s_i64[kBfsWaves];
  const int tid = threadIdx.x;
  int64_t start;
  if (!full) {
    // s0: the longest row, smallest index among equals (rows longer than
    // 2^31 slots cannot occur: columns in a row are distinct and below n)
    int64_t best = -1;
    for (int64_t i = tid; i < n; i += kBfsThreads) {
      const int64_t len = int64_t(rowptr[i + 1] - rowptr[i]);
      const int64_t k = (len << 32) | int64_t(INT32_MAX - int32_t(i));
      best = k > best ? k : best;
    }
    best = bfs_max(best, s_i64);
    start = int64_t(INT32_MAX - int32_t(best & 0xffffffff));
    if (tid == 0) io[0] = int32_t(start);
  } else {
    start = io[1];
  }
  if (tid == 0) {
    order[0] = int32_t(start);
    pos[start] = 0;
  }
  bfs_sync();
  int64_t a = 0, b = 1, cursor = 0;
  // each pass of the loop places at least one node or returns
  for (int64_t guard = 0; guard <= n + 1; ++guard) {
    // claims: every unplaced neighbour of the level gets its earliest parent
    for (int64_t q = a + tid; q < b; q += kBfsThreads) {
      const int64_t p = order[q];
      const int64_t e = int64_t(rowptr[p + 1]);
      for (int64_t k = int64_t(rowptr[p]); k < e; ++k) {
        const int32_t u = col[k];
        if (pos[u] < 0) atomicMin(&key[u], int32_t(q));
      }
    }
    bfs_sync();
    // counts of claims per parent
    for (int64_t q = a + tid; q < b; q += kBfsThreads) {
      const int64_t p = order[q];
      const int64_t e = int64_t(rowptr[p + 1]);
      int32_t c = 0;
      for (int64_t k = int64_t(rowptr[p]); k < e; ++k) {
        const int32_t u = col[k];
        c += (pos[u] < 0 && key[u] == int32_t(q)) ? 1 : 0;
      }
      cnt[q - a] = c;
    }
    bfs_sync();
    // exclusive scan of the counts, in chunks of the workgroup's size
    int64_t total = 0;
    for (int64_t c0 = a; c0 < b; c0 += kBfsThreads) {
      const int64_t q = c0 + tid;
      const int32_t v = q < b ? cnt[q - a] : 0;
      int32_t chunk = 0;
      const int32_t ex = bfs_scan(v, s_i32, &chunk);
      if (q < b) cnt[q - a] = int32_t(total) + ex;
      total += chunk;
    }
    if (b + total > n) {
      if (tid == 0) io[2] = 1;
      return;
    }
    bfs_sync();
    // placement: each parent writes its claims in column order
    for (int64_t q = a + tid; q < b; q += kBfsThreads) {
      const int64_t p = order[q];
      const int64_t e = int64_t(rowptr[p + 1]);
      int64_t t = b + cnt[q - a];
      for (int64_t k = int64_t(rowptr[p]); k < e; ++k) {
        const int32_t u = col[k];
        if (pos[u] < 0 && key[u] == int32_t(q) && t < n) {
          order[t] = u;
          pos[u] = int32_t(t);
          ++t;
        }
      }
    }
    bfs_sync();
    if (total > 0) {
      a = b;
      b += total;
      continue;
    }
    // the piece is complete; [a, b) is its last level
    if (!full) {
      int64_t m = INT64_MAX;
      for (int64_t q = a + tid; q < b; q += kBfsThreads) m = order[q] < m ? order[q] : m;
      m = bfs_min(m, s_i64);
      if (tid == 0) io[1] = int32_t(m);
      return;
    }
    if (b >= n) return;
    // the next piece starts at the smallest unplaced index.  Unplaced nodes
    // whose neighbours are all placed are pieces of their own: they are
    // placed in index order up to the first node that has an unplaced
    // neighbour, which starts the next visit.
    bool started = false;
    while (cursor < n) {
      const int64_t i = cursor + tid;
      bool un = false, alone = false;
      if (i < n && pos[i] < 0) {
        un = true;
        alone = true;
        const int64_t e = int64_t(rowptr[i + 1]);
        for (int64_t k = int64_t(rowptr[i]); k < e; ++k) {
          const int32_t u = col[k];
          if (u != int32_t(i) && pos[u] < 0) alone = false;
        }
      }
      const int64_t f = bfs_min(un && !alone ? i : INT64_MAX, s_i64);
      const bool place = un && alone && i < f;
      int32_t placed = 0;
      const int32_t rk = bfs_scan(place ? 1 : 0, s_i32, &placed);
      if (place && b + rk < n) {
        order[b + rk] = int32_t(i);
        pos[i] = int32_t(b + rk);
      }
      b += placed;
      if (f != INT64_MAX) {
        if (b >= n) {
          if (tid == 0) io[2] = 1;
          return;
        }
        if (tid == 0) {
          order[b] = int32_t(f);
          pos[f] = int32_t(b);
        }
        a = b;
        b += 1;
        cursor = f + 1;
        started = true;
        bfs_sync();
        break;
      }
      cursor += kBfsThreads;
      bfs_sync();
    }
    if (!started) {
      if (b != n && tid == 0) io[2] = 1;
      return;
    }
  }
  if (tid == 0) io[2] = 1;
}

__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    p[i] = v;
}

// COO triplets of B = P A P^T, one per slot k of A (in slot order): row
// pos[i] and column pos[col[k]] for slot k of row i.
template <typename RP>
__global__ void k_permuted_coo(int64_t n, const RP* __restrict__ rowptr,
                               const int32_t* __restrict__ col, const int32_t* __restrict__ pos,
                               int32_t* __restrict__ rows, int32_t* __restrict__ cols) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int32_t pi = pos[i];
    const int64_t e = int64_t(rowptr[i + 1]);
    for (int64_t k = int64_t(rowptr[i]); k < e; ++k) {
      rows[k] = pi;
      cols[k] = pos[col[k]];
    }
  }
}

// out[s][t] = in[s][src[t]] (values of B's slots from A's), grid.y = system
__global__ void k_gather_slots(int64_t nnz, const uint32_t* __restrict__ src,
                               const double* __restrict__ in, double* __restrict__ out) {
  const double* a = in + int64_t(blockIdx.y) * nnz;
  double* o = out + int64_t(blockIdx.y) * nnz;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < nnz;
       t += int64_t(gridDim.x) * blockDim.x)
    o[t] = a[src[t]];
}

// out[s][t] = in[s][order[t]]
__global__ void k_gather_vec(int64_t n, const int32_t* __restrict__ order,
                             const double* __restrict__ in, double* __restrict__ out) {
  const double* a = in + int64_t(blockIdx.y) * n;
  double* o = out + int64_t(blockIdx.y) * n;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < n;
       t += int64_t(gridDim.x) * blockDim.x)
    o[t] = a[order[t]];
}

// out[s][order[t]] = in[s][t]
__global__ void k_scatter_vec(int64_t n, const int32_t* __restrict__ order,
                              const double* __restrict__ in, double* __restrict__ out) {
  const double* a = in + int64_t(blockIdx.y) * n;
  double* o = out + int64_t(blockIdx.y) * n;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < n;
       t += int64_t(gridDim.x) * blockDim.x)
    o[order[t]] = a[t];
}

template <typename RP>
sla_status compute_order(sla_csr A, int32_t* order, int32_t* pos, hipStream_t st) {
  const int64_t n = A->n;
  int32_t* key = nullptr;
  int32_t* cnt = nullptr;
  int32_t* io = nullptr;
  sla_status s = dev_alloc(&key, size_t(n), "ordering keys");
  if (s == SLA_OK) s = dev_alloc(&cnt, size_t(n), "ordering counts");
  if (s == SLA_OK) s = dev_alloc(&io, 4, "ordering scalars");
  int32_t hio[4] = {0, 0, 0, 0};
  hipError_t e = hipSuccess;
  if (s == SLA_OK) {
    const RP* rp = static_cast<const RP*>(A->rowptr);
    k_fill_i32<<<blocks_for(4), kBlock, 0, st>>>(io, 4, 0);
    for (int full = 0; full <= 1 && e == hipSuccess; ++full) {
      k_fill_i32<<<blocks_for(n), kBlock, 0, st>>>(pos, n, -1);
      k_fill_i32<<<blocks_for(n), kBlock, 0, st>>>(key, n, INT32_MAX);
      // every position holds a valid node before it is written
      k_fill_i32<<<blocks_for(n), kBlock, 0, st>>>(order, n, 0);
      k_bfs_order<RP><<<1, kBfsThreads, 0, st>>>(n, rp, A->col, pos, key, order, cnt, io, full);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipMemcpyAsync(hio, io, sizeof(hio), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
  }
  dev_free(key);
  dev_free(cnt);
  dev_free(io);
  if (s != SLA_OK) return s;
  if (e != hipSuccess) {
    set_error("ordering: %s", hipGetErrorString(e));
    return SLA_ERR_DEVICE;
  }
  if (hio[2] != 0) {
    set_error("ordering: inconsistent visit (internal error)");
    return SLA_ERR_DEVICE;
  }
  return SLA_OK;
}

template <typename RP>
sla_status build_permuted(sla_csr A, const int32_t* pos, sla_csr* out, hipStream_t st) {
  const int64_t nnz = A->nnz;
  int32_t* rows = nullptr;
  int32_t* cols = nullptr;
  sla_status s = dev_alloc(&rows, size_t(nnz > 0 ? nnz : 1), "permuted rows");
  if (s == SLA_OK) s = dev_alloc(&cols, size_t(nnz > 0 ? nnz : 1), "permuted columns");
  sla_csr B = nullptr;
  if (s == SLA_OK) {
    k_permuted_coo<RP><<<blocks_for(A->n), kBlock, 0, st>>>(
        A->n, static_cast<const RP*>(A->rowptr), A->col, pos, rows, cols);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
      set_error("ordering: kernel launch failed: %s", hipGetErrorString(e));
      s = SLA_ERR_DEVICE;
    }
  }
  if (s == SLA_OK) {
    B = new sla_csr_s();
    B->device = A->device;
    B->n = A->n;
    B->nnz_coo = nnz;
    B->rp_idx = A->rp_idx;
    s = build_from_coo(B, SLA_I32, rows, cols, st);  // synchronises
    if (s == SLA_OK) s = analyse_pattern(B, st);
    if (s == SLA_OK && B->nnz != nnz) {
      set_error("ordering: %lld slots became %lld", (long long)nnz, (long long)B->nnz);
      s = SLA_ERR_CSR;
    }
  }
  dev_free(rows);
  dev_free(cols);
  if (s != SLA_OK) {
    free_handle(B);
    return s;
  }
  // only the slot map (sorted_idx: B's slot -> A's slot) is used later
  dev_free(B->perm);
  dev_free(B->grp);
  B->perm = nullptr;
  B->grp = nullptr;
  // the ordering serves patterns whose gathers miss the caches: B keeps the
  // separate search-direction pass whenever A's pattern would take it
  B->wide_cols = B->wide_cols || A->wide_cols;
  *out = B;
  return SLA_OK;
}

}  // namespace

void release_reorder(sla_csr A) {
  if (A == nullptr || A->ro == nullptr) return;
  Reorder* R = A->ro;
  free_handle(R->B);
  dev_free(R->order);
  dev_free(R->vals);
  dev_free(R->vin);
  dev_free(R->vout);
  delete R;
  A->ro = nullptr;
}

sla_status make_reorder(sla_csr A, hipStream_t st) {
  if (A->nnz >= (int64_t(1) << 32)) {
    set_error("sla_csr_reorder: %lld slots; at most 2^32 - 1", (long long)A->nnz);
    return SLA_ERR_ARG;
  }
  Reorder* R = new Reorder();
  int32_t* pos = nullptr;
  sla_status s = dev_alloc(&R->order, size_t(A->n > 0 ? A->n : 1), "ordering");
  if (s == SLA_OK) s = dev_alloc(&pos, size_t(A->n > 0 ? A->n : 1), "ordering positions");
  if (s == SLA_OK && A->n > 0) {
    if (A->rp_idx == SLA_I32) s = compute_order<int32_t>(A, R->order, pos, st);
    else s = compute_order<int64_t>(A, R->order, pos, st);
  }
  if (s == SLA_OK) {
    if (A->rp_idx == SLA_I32) s = build_permuted<int32_t>(A, pos, &R->B, st);
    else s = build_permuted<int64_t>(A, pos, &R->B, st);
  }
  dev_free(pos);
  if (s != SLA_OK) {
    free_handle(R->B);
    dev_free(R->order);
    delete R;
    return s;
  }
  release_reorder(A);
  A->ro = R;
  return SLA_OK;
}

// B takes A's solver settings and the values bound to A, gathered into B's
// slot order; the permuted-vector buffers hold at least `batch` systems.
static sla_status prepare(sla_csr A, hipStream_t st) {
  Reorder* R = A->ro;
  sla_csr B = R->B;
  const int64_t batch = A->batch;
  if (B->spmv_variant != A->spmv_variant || B->graph_block != A->graph_block ||
      B->wg_per_cu != A->wg_per_cu) {
    SLA_TRY_HIP(hipStreamSynchronize(st));
    release_workspace(B);  // captured graphs and grids follow the settings
    B->spmv_variant = A->spmv_variant;
    B->graph_block = A->graph_block;
    B->wg_per_cu = A->wg_per_cu;
  }
  if (R->vals_batch < batch) {
    SLA_TRY_HIP(hipStreamSynchronize(st));
    dev_free(R->vals);
    R->vals = nullptr;
    R->vals_batch = 0;
    SLA_TRY(dev_alloc(&R->vals, size_t(batch) * size_t(A->nnz > 0 ? A->nnz : 1), "values"));
    R->vals_batch = batch;
  }
  if (R->vec_batch < batch) {
    SLA_TRY_HIP(hipStreamSynchronize(st));
    dev_free(R->vin);
    dev_free(R->vout);
    R->vin = R->vout = nullptr;
    R->vec_batch = 0;
    const size_t len = size_t(batch) * size_t(A->n > 0 ? A->n : 1);
    SLA_TRY(dev_alloc(&R->vin, len, "permuted vector"));
    SLA_TRY(dev_alloc(&R->vout, len, "permuted vector"));
    R->vec_batch = batch;
  }
  if (A->nnz > 0) {
    k_gather_slots<<<dim3(blocks_for(A->nnz), unsigned(batch)), kBlock, 0, st>>>(
        A->nnz, B->sorted_idx, A->vals, R->vals);
    LAUNCH_CHECK();
  }
  B->vals = R->vals;
  B->batch = batch;
  return SLA_OK;
}

static sla_status permute_in(sla_csr A, const double* v, double* out, hipStream_t st) {
  if (A->n == 0) return SLA_OK;
  k_gather_vec<<<dim3(blocks_for(A->n), unsigned(A->batch)), kBlock, 0, st>>>(
      A->n, A->ro->order, v, out);
  LAUNCH_CHECK();
  return SLA_OK;
}

static sla_status permute_out(sla_csr A, const double* v, double* out, hipStream_t st) {
  if (A->n == 0) return SLA_OK;
  k_scatter_vec<<<dim3(blocks_for(A->n), unsigned(A->batch)), kBlock, 0, st>>>(
      A->n, A->ro->order, v, out);
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status run_cg_any(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                      uint32_t flags, sla_cg_info* info, hipStream_t st) {
  if (A->ro == nullptr) return run_cg(A, b, x, tol, maxit, flags, info, st);
  Reorder* R = A->ro;
  SLA_TRY(prepare(A, st));
  SLA_TRY(permute_in(A, b, R->vin, st));
  if (flags & SLA_FLAG_X0) SLA_TRY(permute_in(A, x, R->vout, st));
  const sla_status s = run_cg(R->B, R->vin, R->vout, tol, maxit, flags, info, st);
  if (s != SLA_OK && s != SLA_ERR_NOT_SPD && s != SLA_ERR_NONFINITE) return s;
  // the result, or the last iterate after a breakdown
  SLA_TRY(permute_out(A, R->vout, x, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));
  return s;
}

sla_status profile_kernels_any(sla_csr A, const double* b, double* x, int64_t reps,
                               double* avg_ms, hipStream_t st) {
  if (A->ro == nullptr) return profile_kernels(A, b, x, reps, avg_ms, st);
  Reorder* R = A->ro;
  SLA_TRY(prepare(A, st));
  SLA_TRY(permute_in(A, b, R->vin, st));
  return profile_kernels(R->B, R->vin, R->vout, reps, avg_ms, st);
}

sla_status copy_order(sla_csr A, int32_t* out, hipStream_t st) {
  if (A->n > 0)
    SLA_TRY_HIP(hipMemcpyAsync(out, A->ro->order, sizeof(int32_t) * size_t(A->n),
                               hipMemcpyDeviceToDevice, st));
  return SLA_OK;
}

sla_csr solver_handle(sla_csr A) { return A->ro != nullptr ? A->ro->B : A; }

}  // namespace sla
