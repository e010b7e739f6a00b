// Sparsity-pattern construction: COO -> CSR, CSR validation, value mapping.
//
// The pattern is the one a SparseTensor shares across a batch (torch-sla
// explainer, technical summary, Methodology 1).  The result of the COO path
// is unique: triplets ordered by (row, col), ties by input position, equal
// (row, col) merged into one slot.  Integer atomics decide only where a
// triplet lands before its row is sorted, and every row is then sorted by the
// total order (col, input position), so the output is bit-identical on every
// run whatever order the atomics took.
#include <algorithm>
#include <vector>

#include "handle.h"

namespace sla {
namespace {

constexpr int kScanItems = 16;
constexpr int64_t kScanTile = int64_t(kBlock) * kScanItems;  // 4096
constexpr int kSmallRow = 32;    // rows up to this length: one thread sorts
constexpr int kMidRow = 4096;    // up to this: one workgroup sorts in LDS

inline unsigned grid_for(int64_t work, int64_t per_block = kBlock) {
  int64_t g = (work + per_block - 1) / per_block;
  return (unsigned)std::max<int64_t>(1, std::min<int64_t>(g, 1 << 20));
}

// ---------------------------------------------------------------------------
// Exclusive scan of non-negative integers into int64 (out has L+1 entries)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int64_t block_sum_i64(int64_t v, int64_t* lds) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  int64_t t = lds[0] + lds[1] + lds[2] + lds[3];
  __syncthreads();
  return t;
}

__device__ __forceinline__ int64_t block_exclusive_i64(int64_t v, int64_t* lds) {
  const int lane = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  int64_t inc = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int64_t o = __shfl_up(inc, off, kWave);
    if (lane >= off) inc += o;
  }
  if (lane == kWave - 1) lds[w] = inc;
  __syncthreads();
  int64_t before = 0;
  for (int j = 0; j < w; ++j) before += lds[j];
  __syncthreads();
  return before + inc - v;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_scan_reduce(const T* __restrict__ in, int64_t L,
                                                        int64_t* __restrict__ bsum) {
  __shared__ int64_t lds[4];
  const int64_t base = int64_t(blockIdx.x) * kScanTile;
  int64_t s = 0;
  for (int j = 0; j < kScanItems; ++j) {
    const int64_t i = base + int64_t(j) * kBlock + threadIdx.x;
    if (i < L) s += int64_t(in[i]);
  }
  s = block_sum_i64(s, lds);
  if (threadIdx.x == 0) bsum[blockIdx.x] = s;
}

template <typename T>
__global__ __launch_bounds__(kBlock) void k_scan_down(const T* __restrict__ in, int64_t L,
                                                      const int64_t* __restrict__ boff,
                                                      int64_t* __restrict__ out) {
  __shared__ int64_t lds[4];
  const int64_t base = int64_t(blockIdx.x) * kScanTile + int64_t(threadIdx.x) * kScanItems;
  int64_t v[kScanItems];
  int64_t tsum = 0;
#pragma unroll
  for (int j = 0; j < kScanItems; ++j) {
    const int64_t i = base + j;
    v[j] = i < L ? int64_t(in[i]) : 0;
    tsum += v[j];
  }
  int64_t run = boff[blockIdx.x] + block_exclusive_i64(tsum, lds);
#pragma unroll
  for (int j = 0; j < kScanItems; ++j) {
    const int64_t i = base + j;
    if (i < L) out[i] = run;
    run += v[j];
    if (i == L - 1) out[L] = run;
  }
}

__global__ void k_set_i64(int64_t* p, int64_t v) { *p = v; }

template <typename T>
sla_status exclusive_scan(const T* in, int64_t L, int64_t* out, hipStream_t st) {
  if (L == 0) {
    k_set_i64<<<1, 1, 0, st>>>(out, 0);
    SLA_TRY_HIP(hipGetLastError());
    return SLA_OK;
  }
  const int64_t nb = (L + kScanTile - 1) / kScanTile;
  int64_t* bsum = nullptr;
  int64_t* boff = nullptr;
  SLA_TRY(dev_alloc(&bsum, nb, "scan block sums"));
  sla_status s = dev_alloc(&boff, nb + 1, "scan block offsets");
  if (s == SLA_OK) {
    k_scan_reduce<T><<<(unsigned)nb, kBlock, 0, st>>>(in, L, bsum);
    s = hipGetLastError() == hipSuccess ? SLA_OK : SLA_ERR_DEVICE;
    if (s != SLA_OK) set_error("scan launch failed");
  }
  if (s == SLA_OK) {
    if (nb == 1) {
      // one tile: its offset is 0 (recursing would scan a 1-element array
      // that is again one tile, forever)
      k_set_i64<<<1, 1, 0, st>>>(boff, 0);
      if (hipGetLastError() != hipSuccess) {
        set_error("scan launch failed");
        s = SLA_ERR_DEVICE;
      }
    } else {
      s = exclusive_scan<int64_t>(bsum, nb, boff, st);
    }
  }
  if (s == SLA_OK) {
    k_scan_down<T><<<(unsigned)nb, kBlock, 0, st>>>(in, L, boff, out);
    if (hipGetLastError() != hipSuccess) {
      set_error("scan launch failed");
      s = SLA_ERR_DEVICE;
    }
  }
  (void)hipStreamSynchronize(st);
  dev_free(bsum);
  dev_free(boff);
  return s;
}

// ---------------------------------------------------------------------------
// COO -> CSR kernels
// ---------------------------------------------------------------------------
template <typename CI>
__global__ void k_coo_count(int64_t m, int64_t n, const CI* __restrict__ row,
                            const CI* __restrict__ col, uint32_t* __restrict__ cnt,
                            int* __restrict__ err) {
  for (int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; k < m;
       k += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = row[k];
    const int64_t c = col[k];
    if (r < 0 || r >= n || c < 0 || c >= n) {
      atomicOr(err, 1);
      continue;
    }
    atomicAdd(&cnt[r], 1u);
  }
}

template <typename CI>
__global__ void k_coo_scatter(int64_t m, const CI* __restrict__ row, const CI* __restrict__ col,
                              const int64_t* __restrict__ start, uint32_t* __restrict__ fill,
                              uint64_t* __restrict__ key, int32_t* __restrict__ rowid) {
  for (int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; k < m;
       k += int64_t(gridDim.x) * blockDim.x) {
    const int64_t r = row[k];
    const int64_t pos = start[r] + atomicAdd(&fill[r], 1u);
    key[pos] = (uint64_t(uint32_t(col[k])) << 32) | uint64_t(uint32_t(k));
    rowid[pos] = int32_t(r);
  }
}

// Rows of up to kSmallRow triplets are insertion-sorted by one thread; longer
// rows are listed for the workgroup / global sorts.
__global__ void k_sort_rows_small(int64_t n, const int64_t* __restrict__ start,
                                  uint64_t* __restrict__ key, int32_t* __restrict__ mid_list,
                                  int* __restrict__ n_mid, int32_t* __restrict__ long_list,
                                  int* __restrict__ n_long) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t a = start[i];
    const int64_t len = start[i + 1] - a;
    if (len <= 1) continue;
    if (len <= kSmallRow) {
      uint64_t v[kSmallRow];
      for (int j = 0; j < len; ++j) v[j] = key[a + j];
      for (int j = 1; j < len; ++j) {
        const uint64_t x = v[j];
        int t = j - 1;
        while (t >= 0 && v[t] > x) {
          v[t + 1] = v[t];
          --t;
        }
        v[t + 1] = x;
      }
      for (int j = 0; j < len; ++j) key[a + j] = v[j];
    } else if (len <= kMidRow) {
      mid_list[atomicAdd(n_mid, 1)] = int32_t(i);
    } else {
      long_list[atomicAdd(n_long, 1)] = int32_t(i);
    }
  }
}

__device__ __forceinline__ int64_t next_pow2(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

// One workgroup per listed row: bitonic sort in LDS, padded with keys above
// every real key (real keys have a column < 2^31 in the high word).
__global__ __launch_bounds__(kBlock) void k_sort_rows_mid(const int32_t* __restrict__ list,
                                                          const int64_t* __restrict__ start,
                                                          uint64_t* __restrict__ key) {
  __shared__ uint64_t s[kMidRow];
  const int64_t row = list[blockIdx.x];
  const int64_t a = start[row];
  const int64_t len = start[row + 1] - a;
  const int64_t P = next_pow2(len);
  for (int64_t i = threadIdx.x; i < P; i += kBlock) s[i] = i < len ? key[a + i] : ~uint64_t(0);
  __syncthreads();
  for (int64_t k = 2; k <= P; k <<= 1) {
    for (int64_t j = k >> 1; j > 0; j >>= 1) {
      for (int64_t i = threadIdx.x; i < P; i += kBlock) {
        const int64_t ixj = i ^ j;
        if (ixj > i) {
          const bool up = (i & k) == 0;
          const uint64_t x = s[i], y = s[ixj];
          if ((x > y) == up) {
            s[i] = y;
            s[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int64_t i = threadIdx.x; i < len; i += kBlock) key[a + i] = s[i];
}

// Rows longer than kMidRow: bitonic network over a padded copy in memory.
__global__ void k_long_fill(const uint64_t* __restrict__ key, int64_t a, int64_t len,
                            uint64_t* __restrict__ tmp, int64_t P) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < P;
       i += int64_t(gridDim.x) * blockDim.x)
    tmp[i] = i < len ? key[a + i] : ~uint64_t(0);
}
__global__ void k_long_step(uint64_t* __restrict__ tmp, int64_t P, int64_t j, int64_t k) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < P;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t ixj = i ^ j;
    if (ixj > i) {
      const bool up = (i & k) == 0;
      const uint64_t x = tmp[i], y = tmp[ixj];
      if ((x > y) == up) {
        tmp[i] = y;
        tmp[ixj] = x;
      }
    }
  }
}
__global__ void k_long_back(uint64_t* __restrict__ key, int64_t a, int64_t len,
                            const uint64_t* __restrict__ tmp) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < len;
       i += int64_t(gridDim.x) * blockDim.x)
    key[a + i] = tmp[i];
}

__global__ void k_heads(int64_t m, const uint64_t* __restrict__ key,
                        const int32_t* __restrict__ rowid, uint8_t* __restrict__ head) {
  for (int64_t s = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; s < m;
       s += int64_t(gridDim.x) * blockDim.x) {
    head[s] = (s == 0 || rowid[s] != rowid[s - 1] || (key[s] >> 32) != (key[s - 1] >> 32))
                  ? 1 : 0;
  }
}

__global__ void k_coo_emit(int64_t m, const uint64_t* __restrict__ key,
                           const uint8_t* __restrict__ head, const int64_t* __restrict__ hscan,
                           int32_t* __restrict__ col_out, int64_t* __restrict__ perm,
                           uint32_t* __restrict__ sorted_idx, int64_t* __restrict__ grp) {
  for (int64_t s = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; s < m;
       s += int64_t(gridDim.x) * blockDim.x) {
    const int64_t slot = hscan[s] + head[s] - 1;
    const uint64_t kv = key[s];
    const uint32_t k = uint32_t(kv);
    if (head[s]) {
      col_out[slot] = int32_t(kv >> 32);
      grp[slot] = s;
    }
    perm[k] = slot;
    sorted_idx[s] = k;
  }
}

template <typename RP>
__global__ void k_coo_rowptr(int64_t n, const int64_t* __restrict__ start,
                             const int64_t* __restrict__ hscan, RP* __restrict__ rowptr) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i <= n;
       i += int64_t(gridDim.x) * blockDim.x)
    rowptr[i] = RP(hscan[start[i]]);
}

// vals[s][slot] = first COO value of the slot, then + the others in input order
__global__ void k_values_from_coo(int64_t nnz, int64_t m, const int64_t* __restrict__ grp,
                                  const uint32_t* __restrict__ sidx,
                                  const double* __restrict__ coo_val, double* __restrict__ vals) {
  const double* cv = coo_val + int64_t(blockIdx.y) * m;
  double* out = vals + int64_t(blockIdx.y) * nnz;
  for (int64_t slot = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; slot < nnz;
       slot += int64_t(gridDim.x) * blockDim.x) {
    const int64_t g0 = grp[slot], g1 = grp[slot + 1];
    double v = cv[sidx[g0]];
    for (int64_t g = g0 + 1; g < g1; ++g) v = v + cv[sidx[g]];
    out[slot] = v;
  }
}

__global__ void k_grad_to_coo(int64_t m, int64_t nnz, const int64_t* __restrict__ perm,
                              const double* __restrict__ gv, double* __restrict__ gc) {
  const double* g = gv + int64_t(blockIdx.y) * nnz;
  double* o = gc + int64_t(blockIdx.y) * m;
  for (int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; k < m;
       k += int64_t(gridDim.x) * blockDim.x)
    o[k] = g[perm[k]];
}

// Every row pointer and column is range-checked before it is used as an
// index, so malformed input becomes an error code, never a stray access.
template <typename RP>
__global__ void k_validate_csr(int64_t n, int64_t nnz, const RP* __restrict__ rowptr,
                               const int32_t* __restrict__ col, int* __restrict__ err) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t a = rowptr[i], e = rowptr[i + 1];
    if (i == 0 && a != 0) atomicOr(err, 1);
    if (i == n - 1 && e != nnz) atomicOr(err, 2);
    if (a < 0 || e > nnz || e < a) {
      atomicOr(err, 4);
      continue;
    }
    int64_t prev = -1;
    for (int64_t k = a; k < e; ++k) {
      const int64_t c = col[k];
      if (c < 0 || c >= n) atomicOr(err, 8);
      else if (c <= prev) atomicOr(err, 16);
      prev = c;
    }
  }
}

template <typename RP>
__global__ void k_tile_nnz_max(int64_t n, int64_t tiles, const RP* __restrict__ rowptr,
                               unsigned long long* __restrict__ out) {
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < tiles;
       t += int64_t(gridDim.x) * blockDim.x) {
    const int64_t lo = t * kTileRows;
    const int64_t hi = lo + kTileRows < n ? lo + kTileRows : n;
    atomicMax(out, (unsigned long long)(int64_t(rowptr[hi]) - int64_t(rowptr[lo])));
  }
}

// RAII list of temporary device buffers for the build.
struct Temps {
  std::vector<void*> ptrs;
  ~Temps() {
    for (void* p : ptrs) dev_free(p);
  }
  template <typename T>
  sla_status get(T** p, size_t count, const char* what) {
    SLA_TRY(dev_alloc(p, count == 0 ? 1 : count, what));
    ptrs.push_back(*p);
    return SLA_OK;
  }
};

template <typename CI>
sla_status coo_build(sla_csr A, const CI* row, const CI* col, hipStream_t st) {
  const int64_t n = A->n, m = A->nnz_coo;
  Temps T;
  uint32_t* cnt;
  uint32_t* fill;
  int64_t* start;
  int* flags;  // [0] range error, [1] mid rows, [2] long rows
  SLA_TRY(T.get(&cnt, n, "row counts"));
  SLA_TRY(T.get(&fill, n, "row fill"));
  SLA_TRY(T.get(&start, n + 1, "row starts"));
  SLA_TRY(T.get(&flags, 4, "flags"));
  SLA_TRY_HIP(hipMemsetAsync(cnt, 0, sizeof(uint32_t) * n, st));
  SLA_TRY_HIP(hipMemsetAsync(fill, 0, sizeof(uint32_t) * n, st));
  SLA_TRY_HIP(hipMemsetAsync(flags, 0, sizeof(int) * 4, st));

  if (m > 0) {
    k_coo_count<CI><<<grid_for(m), kBlock, 0, st>>>(m, n, row, col, cnt, flags);
    LAUNCH_CHECK();
  }
  int hflags[4] = {0, 0, 0, 0};
  SLA_TRY_HIP(hipMemcpyAsync(hflags, flags, sizeof(hflags), hipMemcpyDeviceToHost, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));
  if (hflags[0]) {
    set_error("sla_csr_create: a COO row or column index is outside [0, n)");
    return SLA_ERR_CSR;
  }
  SLA_TRY(exclusive_scan<uint32_t>(cnt, n, start, st));

  uint64_t* key;
  int32_t* rowid;
  uint8_t* head;
  int64_t* hscan;
  int32_t* mid_list;
  int32_t* long_list;
  SLA_TRY(T.get(&key, m, "sort keys"));
  SLA_TRY(T.get(&rowid, m, "row ids"));
  SLA_TRY(T.get(&head, m, "head flags"));
  SLA_TRY(T.get(&hscan, m + 1, "head scan"));
  SLA_TRY(T.get(&mid_list, n, "mid rows"));
  SLA_TRY(T.get(&long_list, n, "long rows"));

  if (m > 0) {
    k_coo_scatter<CI><<<grid_for(m), kBlock, 0, st>>>(m, row, col, start, fill, key, rowid);
    LAUNCH_CHECK();
    k_sort_rows_small<<<grid_for(n), kBlock, 0, st>>>(n, start, key, mid_list, flags + 1,
                                                       long_list, flags + 2);
    LAUNCH_CHECK();
    SLA_TRY_HIP(hipMemcpyAsync(hflags, flags, sizeof(hflags), hipMemcpyDeviceToHost, st));
    SLA_TRY_HIP(hipStreamSynchronize(st));
    if (hflags[1] > 0) {
      k_sort_rows_mid<<<(unsigned)hflags[1], kBlock, 0, st>>>(mid_list, start, key);
      LAUNCH_CHECK();
    }
    if (hflags[2] > 0) {
      std::vector<int32_t> longs(hflags[2]);
      std::vector<int64_t> hstart(n + 1);
      SLA_TRY_HIP(hipMemcpyAsync(longs.data(), long_list, sizeof(int32_t) * longs.size(),
                                 hipMemcpyDeviceToHost, st));
      SLA_TRY_HIP(hipMemcpyAsync(hstart.data(), start, sizeof(int64_t) * (n + 1),
                                 hipMemcpyDeviceToHost, st));
      SLA_TRY_HIP(hipStreamSynchronize(st));
      int64_t maxlen = 0;
      for (int32_t r : longs) maxlen = std::max(maxlen, hstart[r + 1] - hstart[r]);
      int64_t P = 1;
      while (P < maxlen) P <<= 1;
      uint64_t* tmp;
      SLA_TRY(T.get(&tmp, P, "long row sort"));
      for (int32_t r : longs) {
        const int64_t a = hstart[r], len = hstart[r + 1] - a;
        int64_t Pr = 1;
        while (Pr < len) Pr <<= 1;
        k_long_fill<<<grid_for(Pr), kBlock, 0, st>>>(key, a, len, tmp, Pr);
        for (int64_t k = 2; k <= Pr; k <<= 1)
          for (int64_t j = k >> 1; j > 0; j >>= 1)
            k_long_step<<<grid_for(Pr), kBlock, 0, st>>>(tmp, Pr, j, k);
        k_long_back<<<grid_for(len), kBlock, 0, st>>>(key, a, len, tmp);
        LAUNCH_CHECK();
      }
    }
    k_heads<<<grid_for(m), kBlock, 0, st>>>(m, key, rowid, head);
    LAUNCH_CHECK();
  }
  SLA_TRY(exclusive_scan<uint8_t>(head, m, hscan, st));
  int64_t nnz = 0;
  SLA_TRY_HIP(hipMemcpyAsync(&nnz, hscan + m, sizeof(int64_t), hipMemcpyDeviceToHost, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));
  if (A->rp_idx == SLA_I32 && nnz >= (int64_t(1) << 31)) {
    set_error("sla_csr_create: %lld slots do not fit int32 row pointers", (long long)nnz);
    return SLA_ERR_ARG;
  }
  A->nnz = nnz;
  SLA_TRY(dev_alloc(&A->rowptr, size_t(n + 1) * A->rp_idx, "rowptr"));
  SLA_TRY(dev_alloc(&A->col, nnz == 0 ? 1 : nnz, "col"));
  SLA_TRY(dev_alloc(&A->perm, m == 0 ? 1 : m, "perm"));
  SLA_TRY(dev_alloc(&A->sorted_idx, m == 0 ? 1 : m, "sorted index"));
  SLA_TRY(dev_alloc(&A->grp, nnz + 1, "slot groups"));
  if (m > 0) {
    k_coo_emit<<<grid_for(m), kBlock, 0, st>>>(m, key, head, hscan, A->col, A->perm,
                                                A->sorted_idx, A->grp);
    LAUNCH_CHECK();
  }
  k_set_i64<<<1, 1, 0, st>>>(A->grp + nnz, m);
  if (A->rp_idx == SLA_I32)
    k_coo_rowptr<int32_t><<<grid_for(n + 1), kBlock, 0, st>>>(n, start, hscan,
                                                              (int32_t*)A->rowptr);
  else
    k_coo_rowptr<int64_t><<<grid_for(n + 1), kBlock, 0, st>>>(n, start, hscan,
                                                              (int64_t*)A->rowptr);
  LAUNCH_CHECK();
  SLA_TRY_HIP(hipStreamSynchronize(st));
  return SLA_OK;
}

// Band verification: every slot (i, j) of row i must have j - i in the
// candidate offsets off[0..noff) (ascending); mask[i] gets bit t for offset t.
// Columns are strictly increasing inside a row (validated), so the slots of a
// row are exactly its set bits in ascending order.  Any other slot clears
// *ok, and the plain CSR kernels are used.
template <typename RP>
__global__ void k_band_masks(int64_t n, const RP* __restrict__ rowptr,
                             const int32_t* __restrict__ col, BandOffsets bo,
                             uint8_t* __restrict__ mask, int* __restrict__ ok) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x) {
    unsigned m = 0;
    int prev = -1;
    bool good = true;
    for (int64_t k = rowptr[i]; k < int64_t(rowptr[i + 1]); ++k) {
      const int64_t d = int64_t(col[k]) - i;
      int t = -1;
      for (int u = 0; u < bo.count; ++u)
        if (int64_t(bo.off[u]) == d) t = u;
      if (t <= prev) {
        good = false;
        break;
      }
      m |= 1u << t;
      prev = t;
    }
    if (!good) atomicAnd(ok, 0);
    mask[i] = uint8_t(m);
  }
}

// Candidate band offsets from 64 samples of 64 consecutive rows spread over
// the matrix (a heuristic: the device pass verifies every slot).  Returns
// false when the samples already show more than kMaxBand offsets.
template <typename RP>
bool sample_offsets(sla_csr A, hipStream_t st, BandOffsets* bo) {
  const int64_t n = A->n;
  std::vector<int64_t> offs;
  const int64_t samples = 64, rows = 64;
  for (int64_t sidx = 0; sidx < samples; ++sidx) {
    const int64_t r0 = std::min<int64_t>(n - 1, (n - 1) * sidx / std::max<int64_t>(1, samples - 1));
    const int64_t r1 = std::min<int64_t>(n, r0 + rows);
    std::vector<RP> rp(size_t(r1 - r0 + 1));
    if (hipMemcpyAsync(rp.data(), (const RP*)A->rowptr + r0, sizeof(RP) * rp.size(),
                       hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return false;
    const int64_t k0 = rp.front(), k1 = rp.back();
    if (k1 <= k0) continue;
    std::vector<int32_t> cc(size_t(k1 - k0));
    if (hipMemcpyAsync(cc.data(), A->col + k0, sizeof(int32_t) * cc.size(),
                       hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return false;
    for (int64_t i = r0; i < r1; ++i)
      for (int64_t k = rp[i - r0]; k < int64_t(rp[i - r0 + 1]); ++k) {
        const int64_t d = int64_t(cc[k - k0]) - i;
        if (std::find(offs.begin(), offs.end(), d) == offs.end()) offs.push_back(d);
        if (int(offs.size()) > kMaxBand) return false;
      }
  }
  if (offs.empty()) return false;
  std::sort(offs.begin(), offs.end());
  bo->count = int32_t(offs.size());
  for (int u = 0; u < bo->count; ++u) bo->off[u] = int32_t(offs[u]);
  return true;
}

// Column locality: the median, over 64 sampled 64-row tiles, of the span
// (largest - smallest column) of the tile.  A wide span means the gathers of
// a tile land all over the vectors and are not reused from cache.
template <typename RP>
sla_status sample_locality(sla_csr A, hipStream_t st) {
  const int64_t n = A->n;
  std::vector<int64_t> spans;
  for (int64_t sidx = 0; sidx < 64; ++sidx) {
    const int64_t r0 = std::min<int64_t>(n - 1, (n - 1) * sidx / 63);
    const int64_t r1 = std::min<int64_t>(n, r0 + kTileRows);
    RP rp[2];
    SLA_TRY_HIP(hipMemcpyAsync(&rp[0], (const RP*)A->rowptr + r0, sizeof(RP),
                               hipMemcpyDeviceToHost, st));
    SLA_TRY_HIP(hipMemcpyAsync(&rp[1], (const RP*)A->rowptr + r1, sizeof(RP),
                               hipMemcpyDeviceToHost, st));
    SLA_TRY_HIP(hipStreamSynchronize(st));
    if (rp[1] <= rp[0]) continue;
    std::vector<int32_t> cc(size_t(rp[1] - rp[0]));
    SLA_TRY_HIP(hipMemcpyAsync(cc.data(), A->col + rp[0], sizeof(int32_t) * cc.size(),
                               hipMemcpyDeviceToHost, st));
    SLA_TRY_HIP(hipStreamSynchronize(st));
    const auto mm = std::minmax_element(cc.begin(), cc.end());
    spans.push_back(int64_t(*mm.second) - int64_t(*mm.first));
  }
  if (!spans.empty()) {
    std::nth_element(spans.begin(), spans.begin() + spans.size() / 2, spans.end());
    A->wide_cols = spans[spans.size() / 2] > kLocalSpan;
  }
  return SLA_OK;
}

template <typename RP>
sla_status detect_band(sla_csr A, hipStream_t st) {
  A->band.count = 0;
  A->line = 0;
  BandOffsets bo{};
  if (A->nnz == 0 || !sample_offsets<RP>(A, st, &bo)) return SLA_OK;
  // the banded kernels address a tile's gathers by 32-bit offsets from one
  // base row, which holds for spans below kMaxBandSpan
  if (int64_t(bo.off[bo.count - 1]) - int64_t(bo.off[0]) >= kMaxBandSpan) return SLA_OK;
  uint8_t* mask = nullptr;
  int* ok = nullptr;
  SLA_TRY(dev_alloc(&mask, A->n, "band masks"));
  sla_status s = dev_alloc(&ok, 1, "band flag");
  int h = 0;
  if (s == SLA_OK) {
    const int one = 1;
    hipError_t e = hipMemcpyAsync(ok, &one, sizeof(int), hipMemcpyHostToDevice, st);
    k_band_masks<RP><<<grid_for(A->n), kBlock, 0, st>>>(A->n, (const RP*)A->rowptr, A->col, bo,
                                                         mask, ok);
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(&h, ok, sizeof(int), hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
      set_error("band detection failed: %s", hipGetErrorString(e));
      s = SLA_ERR_DEVICE;
    }
  }
  dev_free(ok);
  if (s != SLA_OK || !h) {
    dev_free(mask);
    return s;
  }
  A->band_mask = mask;
  A->band = bo;
  // panel order when the band reaches further than kPanelTiles tiles: column
  // blocks of at most kPanelTiles tiles (equal widths) across panels of
  // ceil(span / 64) tiles
  int64_t span = 0;
  for (int u = 0; u < bo.count; ++u) span = std::max<int64_t>(span, std::abs(int64_t(bo.off[u])));
  const int64_t P = (span + kTileRows - 1) / kTileRows;
  if (P > kPanelTiles) {
    const int64_t nb = (P + kPanelTiles - 1) / kPanelTiles;
    A->panel = int32_t(P);
    A->pblock = int32_t((P + nb - 1) / nb);
  }
  // line walk: every offset of 64 or more in magnitude is +-L (one grid
  // line), and both are present
  int64_t L = 0;
  bool lines = true;
  for (int u = 0; u < bo.count; ++u) {
    const int64_t a = std::abs(int64_t(bo.off[u]));
    if (a < kTileRows) continue;
    if (L == 0) L = a;
    else if (a != L) lines = false;
  }
  // the walk takes -L and +L as the first and the last offset
  lines = lines && bo.count >= 2 && bo.off[0] == -L && bo.off[bo.count - 1] == L;
  A->line = (lines && L >= kMinWalkLine) ? L : 0;
  return SLA_OK;
}

template <typename RP>
sla_status tile_stats(sla_csr A, hipStream_t st) {
  unsigned long long* d = nullptr;
  SLA_TRY(dev_alloc(&d, 1, "tile stats"));
  SLA_TRY_HIP(hipMemsetAsync(d, 0, sizeof(*d), st));
  k_tile_nnz_max<RP><<<grid_for(A->tiles), kBlock, 0, st>>>(A->n, A->tiles,
                                                            (const RP*)A->rowptr, d);
  unsigned long long h = 0;
  hipError_t e = hipMemcpyAsync(&h, d, sizeof(h), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  dev_free(d);
  if (e != hipSuccess) {
    set_error("pattern analysis failed: %s", hipGetErrorString(e));
    return SLA_ERR_DEVICE;
  }
  A->max_tile_nnz = int64_t(h);
  return SLA_OK;
}

// rows[k] = the row of slot k (the row index of every stored entry)
template <typename RP>
__global__ void k_expand_rows(int64_t n, const RP* __restrict__ rowptr, int32_t* __restrict__ rows) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  for (int64_t k = rowptr[i]; k < int64_t(rowptr[i + 1]); ++k) rows[k] = int32_t(i);
}

// y[s][j] = (A_s^T x_s)_j from the transposed pattern T: row j of T holds
// the slots of column j of A in ascending row i, and src maps each slot of T
// to the slot of A it came from, so A's values are read in place.  One wave
// per 64-row tile of T: its lanes form the products a x of consecutive slots
// (`cap` at a time) in LDS, then each lane adds its row's products in slot
// order, y = 0, then y = y + a x: an explicit transpose followed by a CSR
// product, bit for bit.
template <typename RP>
__global__ __launch_bounds__(kIterBlock) void k_spmv_transpose(
    int64_t n, int64_t nnz, int64_t tiles, int cap, const RP* __restrict__ rowptr_t,
    const int32_t* __restrict__ col_t, const uint32_t* __restrict__ src,
    const double* __restrict__ vals, const double* __restrict__ x, double* __restrict__ y) {
  extern __shared__ double prod_lds[];
  constexpr int kW = kIterBlock / kWave;
  const int wv = wave_index();
  const int lane = int(lane_id());
  double* pr = prod_lds + int64_t(wv) * cap;
  const int64_t s = blockIdx.y;
  const double* v = vals + s * nnz;
  const double* xs = x + s * n;
  double* ys = y + s * n;
  // each XCD walks a contiguous range of tiles, so the tiles that read the
  // same lines of A's values (rows i and i +- the band's reach) run close
  // together in time on one L2
  const TileWalk walk = wave_walk(tiles, int(gridDim.x), int(blockIdx.x), kW, wv);
  for (int64_t t = walk.first; t < walk.end; t += walk.stride) {
    const int64_t r0 = t * kTileRows;
    const int64_t r1 = r0 + kTileRows < n ? r0 + kTileRows : n;
    const int64_t s0 = rowptr_t[r0];
    const int64_t len = int64_t(rowptr_t[r1]) - s0;
    const int64_t i = r0 + lane;
    int64_t a = 0, e = 0;
    if (i < r1) {
      a = int64_t(rowptr_t[i]) - s0;
      e = int64_t(rowptr_t[i + 1]) - s0;
    }
    double acc = 0.0;
    for (int64_t c0 = 0; c0 < len; c0 += cap) {
      const int64_t clen = len - c0 < cap ? len - c0 : cap;
      for (int64_t q = lane; q < clen; q += kWave) {
        const int64_t k = s0 + c0 + q;
        pr[q] = v[src[k]] * xs[col_t[k]];
      }
      wave_sync();
      const int64_t qa = a > c0 ? a : c0, qe = e < c0 + clen ? e : c0 + clen;
      for (int64_t q = qa; q < qe; ++q) acc = acc + pr[q - c0];
      wave_sync();
    }
    if (i < r1) ys[i] = acc;
  }
}

// Symmetry: every stored (i, j) must have its mirror (j, i) stored, found by
// a binary search of row j's ascending columns; with values, the two slots
// must hold the same value in every system: equal, or within 1e-12 of the
// larger magnitude (symmetric expressions such as D A D round the two
// mirror entries differently by a few ulps).  One thread per row (a row's
// slots in turn), bit 0 of *bad for a missing mirror, bit 1 for unequal
// values.  Both slots of a pair are visited, each finding the other.
constexpr double kSymRel = 1e-12;

__global__ void k_zero_flag(int* __restrict__ flag) { *flag = 0; }

template <typename RP>
__global__ void k_symmetry(int64_t n, int64_t nnz, const RP* __restrict__ rowptr,
                           const int32_t* __restrict__ col, const double* __restrict__ vals,
                           int64_t batch, int* __restrict__ bad) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x) {
    const int64_t a = rowptr[i], e = rowptr[i + 1];
    for (int64_t k = a; k < e; ++k) {
      const int64_t j = col[k];
      if (j == i) continue;
      const int64_t ja = rowptr[j], je = rowptr[j + 1];
      int64_t lo = ja, hi = je;
      while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (int64_t(col[mid]) < i) lo = mid + 1;
        else hi = mid;
      }
      if (lo == je || int64_t(col[lo]) != i) {
        atomicOr(bad, 1);
        continue;
      }
      if (vals == nullptr) continue;
      for (int64_t s = 0; s < batch; ++s) {
        const double u = vals[s * nnz + k], w = vals[s * nnz + lo];
        if (__double_as_longlong(u) == __double_as_longlong(w)) continue;
        const double m = fabs(u) > fabs(w) ? fabs(u) : fabs(w);
        if (!(fabs(u - w) <= kSymRel * m)) {
          atomicOr(bad, 2);
          break;
        }
      }
    }
  }
}

}  // namespace

static sla_status enqueue_check(sla_csr A, bool values, hipStream_t st, int* flag) {
  const double* v = values ? A->vals : nullptr;
  const int64_t batch = values ? A->batch : 0;
  k_zero_flag<<<1, 1, 0, st>>>(flag);  // a kernel, not a memset: callers may capture
  if (A->rp_idx == SLA_I32)
    k_symmetry<int32_t><<<grid_for(A->n), kBlock, 0, st>>>(A->n, A->nnz, (const int32_t*)A->rowptr,
                                                           A->col, v, batch, flag);
  else
    k_symmetry<int64_t><<<grid_for(A->n), kBlock, 0, st>>>(A->n, A->nnz, (const int64_t*)A->rowptr,
                                                           A->col, v, batch, flag);
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status enqueue_symmetry_check(sla_csr A, bool values, hipStream_t st, int** flag_out) {
  *flag_out = nullptr;
  if (A->nnz == 0) return SLA_OK;
  if (A->sym_flag == nullptr) SLA_TRY(dev_alloc(&A->sym_flag, 1, "symmetry flag"));
  SLA_TRY(enqueue_check(A, values, st, A->sym_flag));
  *flag_out = A->sym_flag;
  return SLA_OK;
}

sla_status check_symmetry(sla_csr A, bool values, int* bad, hipStream_t st, int* flag_dev) {
  *bad = 0;
  if (A->nnz == 0) return SLA_OK;
  int* flag = flag_dev;
  if (flag == nullptr) {
    if (A->sym_flag == nullptr) SLA_TRY(dev_alloc(&A->sym_flag, 1, "symmetry flag"));
    flag = A->sym_flag;
  }
  SLA_TRY(enqueue_check(A, values, st, flag));
  int h = 0;
  SLA_TRY_HIP(hipMemcpyAsync(&h, flag, sizeof(int), hipMemcpyDeviceToHost, st));
  SLA_TRY_HIP(hipStreamSynchronize(st));
  *bad = h;
  return SLA_OK;
}

sla_status analyse_pattern(sla_csr A, hipStream_t st) {
  A->tiles = (A->n + kTileRows - 1) / kTileRows;
  if (A->rp_idx == SLA_I32) SLA_TRY(tile_stats<int32_t>(A, st));
  else SLA_TRY(tile_stats<int64_t>(A, st));
  // LDS stage per wave: the largest tile, up to kWaveCap slots (longer tiles
  // are staged in several chunks)
  A->wave_cap = int32_t(std::min<int64_t>(std::max<int64_t>(A->max_tile_nnz, 1), kWaveCap));
  if (!A->no_band) {
    if (A->rp_idx == SLA_I32) SLA_TRY(detect_band<int32_t>(A, st));
    else SLA_TRY(detect_band<int64_t>(A, st));
  }
  if (A->nnz > 0) {
    if (A->rp_idx == SLA_I32) SLA_TRY(sample_locality<int32_t>(A, st));
    else SLA_TRY(sample_locality<int64_t>(A, st));
  }
  return SLA_OK;
}

sla_status build_from_coo(sla_csr A, sla_index coo_idx, const void* row, const void* col,
                          hipStream_t st) {
  if (coo_idx == SLA_I32)
    return coo_build<int32_t>(A, (const int32_t*)row, (const int32_t*)col, st);
  return coo_build<int64_t>(A, (const int64_t*)row, (const int64_t*)col, st);
}

sla_status build_from_csr(sla_csr A, const void* rowptr, const int32_t* col, hipStream_t st) {
  const int64_t n = A->n, nnz = A->nnz;
  SLA_TRY(dev_alloc(&A->rowptr, size_t(n + 1) * A->rp_idx, "rowptr"));
  SLA_TRY(dev_alloc(&A->col, nnz == 0 ? 1 : nnz, "col"));
  SLA_TRY_HIP(hipMemcpyAsync(A->rowptr, rowptr, size_t(n + 1) * A->rp_idx,
                             hipMemcpyDeviceToDevice, st));
  if (nnz > 0)
    SLA_TRY_HIP(hipMemcpyAsync(A->col, col, sizeof(int32_t) * nnz, hipMemcpyDeviceToDevice, st));
  int* err = nullptr;
  SLA_TRY(dev_alloc(&err, 1, "validation flag"));
  hipError_t e = hipMemsetAsync(err, 0, sizeof(int), st);
  if (A->rp_idx == SLA_I32)
    k_validate_csr<int32_t><<<grid_for(n), kBlock, 0, st>>>(n, nnz, (const int32_t*)A->rowptr,
                                                            A->col, err);
  else
    k_validate_csr<int64_t><<<grid_for(n), kBlock, 0, st>>>(n, nnz, (const int64_t*)A->rowptr,
                                                            A->col, err);
  int h = 0;
  if (e == hipSuccess) e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(&h, err, sizeof(int), hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  dev_free(err);
  if (e != hipSuccess) {
    set_error("CSR validation failed: %s", hipGetErrorString(e));
    return SLA_ERR_DEVICE;
  }
  if (h) {
    set_error("sla_csr_create_from_csr: malformed CSR (%s%s%s%s%s)",
              (h & 1) ? "rowptr[0] != 0; " : "", (h & 2) ? "rowptr[n] != nnz; " : "",
              (h & 4) ? "row pointers out of order or range; " : "",
              (h & 8) ? "column out of range; " : "",
              (h & 16) ? "columns not strictly increasing in a row" : "");
    return SLA_ERR_CSR;
  }
  return SLA_OK;
}

// The transposed pattern as a handle of its own: its COO triplets are our
// slots k = 0 .. nnz-1 with row col[k] and column row(k), so the ordinary
// COO build sorts each transposed row by original row (ascending) and its
// perm maps our slots to its slots.
sla_status build_transpose(sla_csr A, hipStream_t st) {
  if (A->trans != nullptr) return SLA_OK;
  int32_t* rows = nullptr;
  SLA_TRY(dev_alloc(&rows, size_t(A->nnz > 0 ? A->nnz : 1), "row of each slot"));
  if (A->rp_idx == SLA_I32)
    k_expand_rows<int32_t><<<grid_for(A->n), kBlock, 0, st>>>(A->n, (const int32_t*)A->rowptr, rows);
  else
    k_expand_rows<int64_t><<<grid_for(A->n), kBlock, 0, st>>>(A->n, (const int64_t*)A->rowptr, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    dev_free(rows);
    set_error("transpose: kernel launch failed: %s", hipGetErrorString(e));
    return SLA_ERR_DEVICE;
  }
  sla_csr T = new sla_csr_s();
  T->device = A->device;
  T->n = A->n;
  T->nnz_coo = A->nnz;
  T->rp_idx = A->rp_idx;
  sla_status s = build_from_coo(T, SLA_I32, A->col, rows, st);
  if (s == SLA_OK) s = analyse_pattern(T, st);
  if (s == SLA_OK) {
    e = hipStreamSynchronize(st);  // `rows` is freed below
    if (e != hipSuccess) {
      set_error("transpose: %s", hipGetErrorString(e));
      s = SLA_ERR_DEVICE;
    }
  }
  dev_free(rows);
  if (s == SLA_OK && T->nnz != A->nnz) {
    // the slots of A are distinct (row, column) pairs, so none may merge
    set_error("transpose: %lld slots became %lld", (long long)A->nnz, (long long)T->nnz);
    s = SLA_ERR_CSR;
  }
  if (s != SLA_OK) {
    free_handle(T);
    return s;
  }
  A->trans = T;
  return SLA_OK;
}

sla_status launch_spmv_transpose(sla_csr A, const double* x, double* y, hipStream_t st) {
  SLA_TRY(build_transpose(A, st));
  sla_csr T = A->trans;
  // the transposed pattern was built from one COO triplet per slot of A, in
  // slot order: the triplet of each of its slots is the slot of A
  constexpr int64_t kW = kIterBlock / kWave;
  // a multiple of kXcds workgroups (the tile walk splits the tiles by XCD)
  int64_t per_xcd = (T->tiles + kW * kXcds - 1) / (kW * kXcds);
  per_xcd = per_xcd < 1 ? 1 : (per_xcd > 8191 ? 8191 : per_xcd);
  const int64_t blocks = per_xcd * kXcds;
  const int cap = T->wave_cap;  // >= 1 once the pattern is analysed
  const dim3 g(unsigned(blocks), unsigned(A->batch));
  const size_t lds = size_t(kW) * size_t(cap) * sizeof(double);
  if (T->rp_idx == SLA_I32)
    k_spmv_transpose<int32_t><<<g, kIterBlock, lds, st>>>(
        A->n, A->nnz, T->tiles, cap, (const int32_t*)T->rowptr, T->col, T->sorted_idx, A->vals,
        x, y);
  else
    k_spmv_transpose<int64_t><<<g, kIterBlock, lds, st>>>(
        A->n, A->nnz, T->tiles, cap, (const int64_t*)T->rowptr, T->col, T->sorted_idx, A->vals,
        x, y);
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status launch_values_from_coo(sla_csr A, const double* coo_val, double* vals, int64_t batch,
                                  hipStream_t st) {
  if (A->nnz == 0) return SLA_OK;
  dim3 g(grid_for(A->nnz), (unsigned)batch);
  k_values_from_coo<<<g, kBlock, 0, st>>>(A->nnz, A->nnz_coo, A->grp, A->sorted_idx, coo_val,
                                           vals);
  LAUNCH_CHECK();
  return SLA_OK;
}

sla_status launch_grad_to_coo(sla_csr A, const double* grad_vals, double* grad_coo,
                              int64_t batch, hipStream_t st) {
  if (A->nnz_coo == 0) return SLA_OK;
  dim3 g(grid_for(A->nnz_coo), (unsigned)batch);
  k_grad_to_coo<<<g, kBlock, 0, st>>>(A->nnz_coo, A->nnz, A->perm, grad_vals, grad_coo);
  LAUNCH_CHECK();
  return SLA_OK;
}

}  // namespace sla
