// Locality ordering of the unknowns for the iterative solvers.
//
// A pattern whose unknowns come in an order unrelated to its graph (a random
// geometric graph whose nodes are numbered in the order the points were
// drawn, say) makes every gathered p[col] of the SpMV a miss in every cache.  Renumbering the unknowns in the breadth-first
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
// It is computed on the device level by level, four kernels per level: every
// node reached from the current level is claimed by its earliest parent (an
// atomic minimum of parent positions, over the whole grid), each parent
// counts its claims, one workgroup scans the counts into each parent's place
// (and starts the next piece when a level claims nothing), and each parent
// writes its claimed nodes in its row's column order.  The result does not
// depend on the timing of the atomics, so the order is reproducible.  The
// level bounds live on the device; the host enqueues blocks of levels and
// polls a done flag between blocks, as the CG loop does.
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

constexpr int kBfsParents = 2;  // parents a thread works on at once
constexpr int kBfsSlots = 8;    // slots of each parent loaded at once
constexpr int kBfsLevels = 32;  // levels enqueued between two polls of the host (even)

// Device state of one visit.  The parents of level L are the positions
// [a[L & 1], b[L & 1]) of the order; the scan of level L writes the bounds of
// level L + 1 into the other parity.
struct BfsState {
  int64_t a[2], b[2];
  int64_t cursor;  // every index below it is placed (where restarts look)
  int32_t done;    // the visit is complete: later level kernels return at once
  int32_t err;     // the bookkeeping disagreed with n (never, for a valid pattern)
  int32_t s0, s1;
};

enum : int { kClaim = 0, kCount = 1, kPlace = 2 };

// One pass over the parents q in [a, b) of a level, by every thread of the
// grid, each taking kBfsParents of them at a time with their row loads issued
// together:
//   kClaim: every unplaced neighbour u gets key[u] = min(key[u], q);
//   kCount: cnt[q - a] = the number of u with key[u] == q still unplaced;
//   kPlace: those u are written at b + cnt[q - a], b + cnt[q - a] + 1, ...
//           in column order (cnt holding the scanned counts).
// A node passes the kCount / kPlace test only for its one claiming parent,
// so the placements of different parents never touch the same node.
template <int PH, typename RP>
__global__ __launch_bounds__(kBlock) void k_bfs_pass(int64_t n, const RP* __restrict__ rowptr,
                                                     const int32_t* __restrict__ col,
                                                     int32_t* pos, int32_t* key, int32_t* order,
                                                     int32_t* cnt, const BfsState* st,
                                                     int parity) {
  if (st->done) return;
  const int64_t a = st->a[parity], b = st->b[parity];
  constexpr int R = kBfsParents, C = kBfsSlots;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t q0 = a + int64_t(blockIdx.x) * blockDim.x + threadIdx.x; q0 < b;
       q0 += stride * R) {
    int64_t q[R], p[R], s[R], e[R], t[R];
    bool ok[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      q[r] = q0 + int64_t(r) * stride;
      ok[r] = q[r] < b;
      p[r] = ok[r] ? order[q[r]] : 0;
    }
    int64_t len = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s[r] = int64_t(rowptr[p[r]]);
      e[r] = ok[r] ? int64_t(rowptr[p[r] + 1]) : s[r];
      len = e[r] - s[r] > len ? e[r] - s[r] : len;
      if constexpr (PH == kPlace) t[r] = ok[r] ? b + cnt[q[r] - a] : n;
    }
    int32_t c[R];
#pragma unroll
    for (int r = 0; r < R; ++r) c[r] = 0;
    for (int64_t k0 = 0; k0 < len; k0 += C) {
      int32_t u[R][C], pu[R][C], ku[R][C];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const int64_t k = s[r] + k0 + j;
          u[r][j] = k < e[r] ? col[k] : -1;
        }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          pu[r][j] = u[r][j] >= 0 ? pos[u[r][j]] : 0;
          if constexpr (PH != kClaim) ku[r][j] = u[r][j] >= 0 ? key[u[r][j]] : -1;
        }
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < C; ++j) {
          const int32_t uu = u[r][j];
          if constexpr (PH == kClaim) {
            if (uu >= 0 && pu[r][j] < 0) atomicMin(&key[uu], int32_t(q[r]));
          } else {
            const bool f = uu >= 0 && pu[r][j] < 0 && ku[r][j] == int32_t(q[r]);
            if constexpr (PH == kCount) {
              c[r] += f ? 1 : 0;
            } else if (f && t[r] < n) {
              order[t[r]] = uu;
              pos[uu] = int32_t(t[r]);
              ++t[r];
            }
          }
        }
    }
    if constexpr (PH == kCount) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        if (ok[r]) cnt[q[r] - a] = c[r];
    }
  }
}

// s0: the longest row, smallest index among equals, as the largest key
// (length << 32) | (INT32_MAX - i) (rows cannot be longer than n < 2^31).
template <typename RP>
__global__ __launch_bounds__(kBlock) void k_bfs_longest(int64_t n, const RP* __restrict__ rowptr,
                                                        unsigned long long* best) {
  __shared__ int64_t s_i64[kBlock / kWave];
  int64_t m = -1;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t len = int64_t(rowptr[i + 1] - rowptr[i]);
    const int64_t k = (len << 32) | int64_t(INT32_MAX - int32_t(i));
    m = k > m ? k : m;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const int64_t o = __shfl_xor(m, off, kWave);
    m = o > m ? o : m;
  }
  if ((threadIdx.x & (kWave - 1)) == 0) s_i64[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int j = 1; j < kBlock / kWave; ++j) m = s_i64[j] > m ? s_i64[j] : m;
    if (m >= 0) atomicMax(best, (unsigned long long)m);
  }
}

// The first node of a visit: s0 (full == 0, from the longest-row key) or s1.
__global__ void k_bfs_start(BfsState* st, const unsigned long long* best, int32_t* pos,
                            int32_t* order, int full) {
  int32_t s;
  if (!full) {
    s = INT32_MAX - int32_t(*best & 0xffffffffull);
    st->s0 = s;
  } else {
    s = st->s1;
  }
  order[0] = s;
  pos[s] = 0;
  st->a[0] = 0;
  st->b[0] = 1;
  st->cursor = 0;
  st->done = 0;
}

// The end of level `parity`, by one workgroup of kBfsThreads threads: the
// exclusive scan of the claim counts (cnt, in place) and the bounds of the
// next level.  When the level claimed nothing, its piece is complete:
//   full == 0: s1 = the smallest index of the piece's last level; done;
//   full == 1: the next piece starts at the smallest unplaced index.
//              Unplaced nodes whose neighbours are all placed are pieces of
//              their own: they are placed in index order up to the first
//              node that has an unplaced neighbour, which starts the next
//              piece; done when every node is placed.
template <typename RP>
__global__ __launch_bounds__(kBfsThreads) void k_bfs_scan(int64_t n,
                                                          const RP* __restrict__ rowptr,
                                                          const int32_t* __restrict__ col,
                                                          int32_t* pos, int32_t* order,
                                                          int32_t* cnt, BfsState* st,
                                                          int parity, int full) {
  __shared__ int32_t s_i32[kBfsWaves];
  __shared__ int64_t s_i64[kBfsWaves];
  if (st->done) return;
  const int tid = threadIdx.x;
  const int64_t a = st->a[parity];
  int64_t b = st->b[parity];
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
    if (tid == 0) {
      st->err = 1;
      st->done = 1;
    }
    return;
  }
  if (total > 0) {
    if (tid == 0) {
      st->a[parity ^ 1] = b;
      st->b[parity ^ 1] = b + total;
    }
    return;
  }
  if (!full) {
    int64_t m = INT64_MAX;
    for (int64_t q = a + tid; q < b; q += kBfsThreads) m = order[q] < m ? order[q] : m;
    m = bfs_min(m, s_i64);
    if (tid == 0) {
      st->s1 = int32_t(m);
      st->done = 1;
    }
    return;
  }
  int64_t cursor = st->cursor;
  while (b < n && cursor < n) {
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
      if (tid == 0) {
        if (b < n) {
          order[b] = int32_t(f);
          pos[f] = int32_t(b);
          st->a[parity ^ 1] = b;
          st->b[parity ^ 1] = b + 1;
          st->cursor = f + 1;
        } else {
          st->err = 1;
          st->done = 1;
        }
      }
      return;
    }
    cursor += kBfsThreads;
    __syncthreads();  // the placements above before the next chunk's tests
  }
  if (tid == 0) {
    if (b != n) st->err = 1;
    st->done = 1;
  }
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
  const RP* rp = static_cast<const RP*>(A->rowptr);
  int32_t* key = nullptr;
  int32_t* cnt = nullptr;
  BfsState* state = nullptr;
  unsigned long long* best = nullptr;
  int32_t* poll = nullptr;  // pinned: the done flag after each block of levels
  hipEvent_t ev[2] = {nullptr, nullptr};
  sla_status s = dev_alloc(&key, size_t(n), "ordering keys");
  if (s == SLA_OK) s = dev_alloc(&cnt, size_t(n), "ordering counts");
  if (s == SLA_OK) s = dev_alloc(&state, 1, "ordering state");
  if (s == SLA_OK) s = dev_alloc(&best, 1, "longest row");
  hipError_t e = hipSuccess;
  if (s == SLA_OK) e = hipHostMalloc(reinterpret_cast<void**>(&poll), 2 * sizeof(int32_t));
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ev[0], hipEventDisableTiming);
  if (e == hipSuccess) e = hipEventCreateWithFlags(&ev[1], hipEventDisableTiming);
  BfsState hs{};
  const unsigned pass_grid = unsigned(std::max(1, device_cus()));
  // every level places at least one node or ends the visit
  const int64_t max_blocks = (n + 1) / kBfsLevels + 2;
  for (int full = 0; full <= 1 && s == SLA_OK && e == hipSuccess; ++full) {
    k_fill_i32<<<blocks_for(n), kBlock, 0, st>>>(pos, n, -1);
    k_fill_i32<<<blocks_for(n), kBlock, 0, st>>>(key, n, INT32_MAX);
    // every position holds a valid node before it is written
    k_fill_i32<<<blocks_for(n), kBlock, 0, st>>>(order, n, 0);
    if (!full) {
      e = hipMemsetAsync(state, 0, sizeof(BfsState), st);
      if (e == hipSuccess) e = hipMemsetAsync(best, 0, sizeof(unsigned long long), st);
      if (e == hipSuccess) k_bfs_longest<RP><<<blocks_for(n), kBlock, 0, st>>>(n, rp, best);
    }
    if (e == hipSuccess) k_bfs_start<<<1, 1, 0, st>>>(state, best, pos, order, full);
    for (int64_t blk = 0; blk < max_blocks && e == hipSuccess; ++blk) {
      for (int j = 0; j < kBfsLevels; ++j) {
        const int par = j & 1;
        k_bfs_pass<kClaim, RP><<<pass_grid, kBlock, 0, st>>>(n, rp, A->col, pos, key, order, cnt,
                                                             state, par);
        k_bfs_pass<kCount, RP><<<pass_grid, kBlock, 0, st>>>(n, rp, A->col, pos, key, order, cnt,
                                                             state, par);
        k_bfs_scan<RP><<<1, kBfsThreads, 0, st>>>(n, rp, A->col, pos, order, cnt, state, par,
                                                   full);
        k_bfs_pass<kPlace, RP><<<pass_grid, kBlock, 0, st>>>(n, rp, A->col, pos, key, order, cnt,
                                                             state, par);
      }
      e = hipGetLastError();
      if (e == hipSuccess)
        e = hipMemcpyAsync(poll + (blk & 1), &state->done, sizeof(int32_t),
                           hipMemcpyDeviceToHost, st);
      if (e == hipSuccess) e = hipEventRecord(ev[blk & 1], st);
      // wait for the previous block only, so that one block is always queued
      if (e == hipSuccess && blk >= 1) {
        e = hipEventSynchronize(ev[(blk - 1) & 1]);
        if (e == hipSuccess && poll[(blk - 1) & 1]) break;
      }
    }
    if (e == hipSuccess) e = hipMemcpyAsync(&hs, state, sizeof(hs), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e == hipSuccess && (!hs.done || hs.err)) break;
  }
  if (ev[0]) (void)hipEventDestroy(ev[0]);
  if (ev[1]) (void)hipEventDestroy(ev[1]);
  if (poll) (void)hipHostFree(poll);
  dev_free(key);
  dev_free(cnt);
  dev_free(state);
  dev_free(best);
  if (s != SLA_OK) return s;
  if (e != hipSuccess) {
    set_error("ordering: %s", hipGetErrorString(e));
    return SLA_ERR_DEVICE;
  }
  if (!hs.done || hs.err) {
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
  B->one_group = A->one_group;
  // automatic grid: one workgroup per CU (the ordered pattern's gathers hit
  // the L2, and half the waves per CU contend less for it: 2.4 % more
  // iterations/s on the ordered 4M-node random geometric graph)
  const int wg = A->wg_per_cu > 0 ? A->wg_per_cu : 1;
  if (B->spmv_variant != A->spmv_variant || B->graph_block != A->graph_block ||
      B->wg_per_cu != wg) {
    SLA_TRY_HIP(hipStreamSynchronize(st));
    release_workspace(B);  // captured graphs and grids follow the settings
    B->spmv_variant = A->spmv_variant;
    B->graph_block = A->graph_block;
    B->wg_per_cu = wg;
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

sla_status run_bicgstab_any(sla_csr A, const double* b, double* x, double tol, int64_t maxit,
                            uint32_t flags, sla_cg_info* info, hipStream_t st) {
  if (A->ro == nullptr) return run_bicgstab(A, b, x, tol, maxit, flags, info, st);
  Reorder* R = A->ro;
  SLA_TRY(prepare(A, st));
  SLA_TRY(permute_in(A, b, R->vin, st));
  if (flags & SLA_FLAG_X0) SLA_TRY(permute_in(A, x, R->vout, st));
  const sla_status s = run_bicgstab(R->B, R->vin, R->vout, tol, maxit, flags, info, st);
  if (s != SLA_OK && s != SLA_ERR_BREAKDOWN && s != SLA_ERR_NONFINITE) return s;
  SLA_TRY(permute_out(A, R->vout, x, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));
  return s;
}

// (P A P^T)^T = P A^T P^T: the adjoint of the permuted system with P g is
// P lambda; the slot gradient is formed on A's own slots.
sla_status run_bicgstab_adjoint_any(sla_csr A, const double* x, const double* grad_x,
                                    double* grad_b, double* grad_vals, double tol,
                                    int64_t maxit, uint32_t flags, sla_cg_info* info,
                                    hipStream_t st) {
  if (A->ro == nullptr)
    return run_bicgstab_adjoint(A, x, grad_x, grad_b, grad_vals, tol, maxit, flags, info, st);
  Reorder* R = A->ro;
  SLA_TRY(prepare(A, st));
  SLA_TRY(permute_in(A, grad_x, R->vin, st));
  const sla_status s = run_bicgstab_adjoint(R->B, nullptr, R->vin, R->vout, nullptr, tol, maxit,
                                            flags, info, st);
  if (s != SLA_OK && s != SLA_ERR_BREAKDOWN && s != SLA_ERR_NONFINITE) return s;
  SLA_TRY(permute_out(A, R->vout, grad_b, st));
  if (grad_vals != nullptr && A->nnz > 0)
    SLA_TRY(launch_slot_products(A, A->batch, grad_b, x, grad_vals, true, st));
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
